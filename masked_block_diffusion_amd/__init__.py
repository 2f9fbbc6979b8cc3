"""Block-diffusion denoising on MI355X (gfx950): HIP kernels behind a C ABI.

The library (libdlm.so, built from csrc/ by `build.py`) exports dlm_prefill,
dlm_denoise_step, dlm_commit and dlm_append_canvas (include/dlm.h).  This
package is the Python binding: `abi` mirrors the header with ctypes, `model`
wraps the calls over torch tensors.  There is no fallback path: when the
library is missing the binding raises.
"""
from .abi import DLMError, load_library  # noqa: F401
from .model import DLM, CanvasSteps, KVPool, Rule, Seq, ar_decode, generate  # noqa: F401
