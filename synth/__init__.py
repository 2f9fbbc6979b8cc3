"""Seeded synthetic inputs shared by the oracle's tests and the HIP path's callers.

Holds workload shapes and random draws only; no step of the method lives here.
"""
from .configs import ModelConfig, RunConfig, RUNS, get_run  # noqa: F401
from .weights import (make_weights, make_inputs, prefix_ids, prefix_lengths,  # noqa: F401
                      projection_names, to_float64_numpy, tensor_seed, quantize_e4m3_rows)
