"""Python binding over libdlm.so: the same four operations as the C ABI.

`DLM` packs a weight dictionary into the ABI's layout (Q/K/V rows concatenated
into one [(Hq + 2 Hkv) dh, d] matrix, fp8 codes plus their per-channel scales),
creates the library handle, and exposes dlm_prefill / dlm_denoise_step /
dlm_commit / dlm_append_canvas over torch tensors.  torch provides device
memory and the stream; every step of the path runs in the library's kernels.

`generate` is the host iteration loop of block diffusion: prefill the prompt,
then per canvas start all-[MASK], alternate denoise and commit for the
schedule's steps (stopping early once nothing is masked), and append the
finished canvas to the KV cache (rahulsharmavishwakarma.github.io, "Diffusion
LLMs: what changes when you stop generating one token at a time", sections 2,
4.1 and 4.2).
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import torch

from . import abi
from .abi import check

_DTYPES = {"f32": abi.DLM_F32, "bf16": abi.DLM_BF16, "fp8": abi.DLM_FP8, "mxfp4": abi.DLM_MXFP4,
           "mxfp6": abi.DLM_MXFP6}
# MX expert formats: (key suffix of the codes, element bits)
_MX = {"mxfp4": (".q4", 4), "mxfp6": (".q6", 6)}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


KV_PAGE = 64   # tokens per KV page


@dataclass
class Seq:
    """One request: its canvas int32[C], its KV cache and the ABI struct
    pointing at both (T lives in the struct).  Contiguous cache: `kv` is
    [L, 2, Hkv, capacity * dh], per layer and KV head a key block [capacity,
    dh] and a value block stored transposed, [dh, capacity].  Paged cache:
    `kv` is the pool [pages, L, 2, Hkv, 64 * dh] and `pages` the request's page
    indices (int32, device), token t in page pages[t // 64] at slot t % 64."""
    kv: torch.Tensor
    canvas: torch.Tensor
    raw: abi.dlm_seq
    head_dim: int
    pages: Optional[torch.Tensor] = None
    pool: Optional["KVPool"] = None

    @property
    def T(self) -> int:
        return self.raw.T

    @property
    def capacity(self) -> int:
        return self.raw.capacity

    def read_kv(self):
        """(keys, values), each [L, Hkv, capacity, dh] (a copy when paged)."""
        dh = self.head_dim
        if self.pages is None:
            L, _, H, _ = self.kv.shape
            k = self.kv[:, 0].view(L, H, self.capacity, dh)
            v = self.kv[:, 1].view(L, H, dh, self.capacity).transpose(-1, -2)
            return k, v
        pg = self.kv[self.pages.long()]                              # [P, L, 2, H, 64 * dh]
        P, L, _, H, _ = pg.shape
        k = pg[:, :, 0].reshape(P, L, H, KV_PAGE, dh).permute(1, 2, 0, 3, 4).reshape(L, H, P * KV_PAGE, dh)
        v = pg[:, :, 1].reshape(P, L, H, dh, KV_PAGE).permute(1, 2, 0, 4, 3).reshape(L, H, P * KV_PAGE, dh)
        return k, v

    def write_kv(self, k: torch.Tensor, v: torch.Tensor) -> None:
        """Stores keys / values [L, Hkv, n, dh] into token slots [0, n)."""
        n, dh = k.shape[2], self.head_dim
        if self.pages is None:
            ck, cv = self.read_kv()
            ck[:, :, :n].copy_(k)
            cv[:, :, :n].copy_(v)
            return
        L, H = k.shape[0], k.shape[1]
        for b in range((n + KV_PAGE - 1) // KV_PAGE):
            lo, hi = b * KV_PAGE, min(n, (b + 1) * KV_PAGE)
            page = self.kv[int(self.pages[b])]                       # [L, 2, H, 64 * dh]
            pk = page[:, 0].view(L, H, KV_PAGE, dh)
            pv = page[:, 1].view(L, H, dh, KV_PAGE)
            pk[:, :, : hi - lo].copy_(k[:, :, lo:hi])
            pv[:, :, :, : hi - lo].copy_(v[:, :, lo:hi].transpose(-1, -2))


class KVPool:
    """A device pool of 64-token KV pages shared by requests, with a free list
    on the host.  A page holds all layers and heads of its tokens:
    [L, 2, Hkv, 64 * dh] (keys [64, dh], values transposed [dh, 64])."""

    def __init__(self, model: "DLM", n_pages: int):
        c = model.cfg
        self.model = model
        self.kv = torch.empty((n_pages, c.n_layers, 2, c.n_kv_heads, KV_PAGE * c.head_dim),
                              dtype=model.kv_dtype, device=model.device)
        self.free = list(range(n_pages))

    def alloc(self, n: int, order=None) -> torch.Tensor:
        if n > len(self.free):
            raise MemoryError(f"KV pool has {len(self.free)} free pages, {n} requested")
        take = [self.free.pop(0 if order is None else order(len(self.free))) for _ in range(n)]
        return torch.tensor(take, dtype=torch.int32, device=self.model.device)

    def release(self, pages: torch.Tensor) -> None:
        self.free.extend(int(p) for p in pages.cpu())


class DLM:
    def __init__(self, cfg, weights: Dict[str, torch.Tensor], canvas: int, device="cuda"):
        self.lib = abi.load_library()
        if not torch.cuda.is_available():
            raise RuntimeError("DLM needs a HIP device")
        self.cfg = cfg
        self.C = canvas
        self.device = torch.device(device)
        self.dtype = cfg.dtype
        self._keep: List[torch.Tensor] = []
        c = abi.dlm_config(
            n_layers=cfg.n_layers, d_model=cfg.d_model, n_q_heads=cfg.n_q_heads,
            n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim, vocab=cfg.vocab,
            mask_id=cfg.mask_id, ffn=abi.DLM_FFN_MOE if cfg.ffn == "moe" else abi.DLM_FFN_DENSE,
            d_ffn=cfg.d_ffn, n_experts=cfg.n_experts, top_k=cfg.top_k, d_expert=cfg.d_expert,
            dtype=_DTYPES[cfg.dtype], canvas=canvas, rms_eps=cfg.rms_eps,
            rope_base=cfg.rope_base, expert_dtype=_DTYPES[getattr(cfg, "expert_dtype", None) or cfg.dtype])
        self.raw_cfg = c
        W = self._pack(cfg, weights)
        self._layers = (abi.dlm_layer_weights * cfg.n_layers)(*W["layers"])
        w = abi.dlm_weights(embed=W["embed"], final_norm=W["final_norm"], lm_head=W["lm_head"],
                            lm_head_s=W["lm_head_s"],
                            layers=ctypes.cast(self._layers, ctypes.POINTER(abi.dlm_layer_weights)))
        self._weights = w
        h = ctypes.c_void_p()
        check(self.lib.dlm_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(h)), "dlm_create")
        self.handle = h
        self.kv_dtype = torch.float32 if cfg.dtype == "f32" else torch.bfloat16

    def truncated(self, n_layers: int) -> "DLM":
        """A second handle over the first `n_layers` layers of this model,
        reading the same packed device weights (nothing is copied; this model
        must outlive it).  Its final norm and LM head are this model's, so its
        logits are those of the depth-`n_layers` prefix of the network.  A
        contiguous KV cache of this model serves it unchanged (layer l sits at
        the same offset); paged caches do not (their pages are sized for
        every layer)."""
        if not 1 <= n_layers <= self.cfg.n_layers:
            raise ValueError(f"n_layers {n_layers} not in [1, {self.cfg.n_layers}]")
        sub = DLM.__new__(DLM)
        sub.lib, sub.C, sub.device, sub.dtype, sub.kv_dtype = self.lib, self.C, self.device, self.dtype, self.kv_dtype
        from dataclasses import replace
        sub.cfg = replace(self.cfg, n_layers=n_layers)
        sub._keep = [self]
        c = abi.dlm_config.from_buffer_copy(self.raw_cfg)
        c.n_layers = n_layers
        sub.raw_cfg = c
        sub._layers = (abi.dlm_layer_weights * n_layers)(*self._layers[:n_layers])
        w = abi.dlm_weights(embed=self._weights.embed, final_norm=self._weights.final_norm,
                            lm_head=self._weights.lm_head, lm_head_s=self._weights.lm_head_s,
                            layers=ctypes.cast(sub._layers, ctypes.POINTER(abi.dlm_layer_weights)))
        sub._weights = w
        h = ctypes.c_void_p()
        check(self.lib.dlm_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(h)), "dlm_create")
        sub.handle = h
        return sub

    # ------------------------------------------------------------ weights --
    def _dev(self, t: torch.Tensor) -> torch.Tensor:
        t = t.to(self.device).contiguous()
        self._keep.append(t)
        return t

    def _tiled(self, t: torch.Tensor) -> torch.Tensor:
        """The library's tiled layout of a row-major [..., N, K] projection
        (dlm_pack_weight, a kernel on the current stream); the row-major
        copy is not kept."""
        t = t.to(self.device).contiguous()
        N, K = t.shape[-2], t.shape[-1]
        batch = t.numel() // (N * K)
        dt = _DTYPES[self.dtype]
        nbytes = self.lib.dlm_packed_weight_bytes(dt, batch, N, K)
        if nbytes == 0:
            raise ValueError(f"cannot pack a {tuple(t.shape)} {self.dtype} weight")
        dst = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        check(self.lib.dlm_pack_weight(dt, batch, N, K, _ptr(t), _ptr(dst), _stream()), "dlm_pack_weight")
        self._keep.append(dst)
        return dst

    def _mx(self, weights, name, fmt):
        """(packed codes pointer, packed scales pointer) of an MX expert tensor:
        codes `name.q4` (MXFP4) or `name.q6` (MXFP6) uint8 [E, N, K * bits /
        8] and E8M0 scales `name.e8` uint8 [E, N, K / 32], rearranged by
        dlm_pack_mx (a kernel on the current stream)."""
        suffix, bits = _MX[fmt]
        q = weights[name + suffix].to(self.device).contiguous()
        e = weights[name + ".e8"].to(self.device).contiguous()
        E, N, K = q.shape[0], q.shape[1], q.shape[2] * 8 // bits
        dt = _DTYPES[fmt]
        nc = self.lib.dlm_packed_mx_bytes(dt, E, N, K, 0)
        ns = self.lib.dlm_packed_mx_bytes(dt, E, N, K, 1)
        if nc == 0 or ns == 0 or tuple(e.shape) != (E, N, K // 32):
            raise ValueError(f"cannot pack {fmt} {name}: codes {tuple(q.shape)}, scales {tuple(e.shape)}")
        dc = torch.empty(nc, dtype=torch.uint8, device=self.device)
        ds = torch.empty(ns, dtype=torch.uint8, device=self.device)
        check(self.lib.dlm_pack_mx(dt, E, N, K, _ptr(q), _ptr(e), _ptr(dc), _ptr(ds), _stream()), "dlm_pack_mx")
        self._keep += [dc, ds]
        return _ptr(dc), _ptr(ds)

    def _proj(self, weights, name, cat: Sequence[str] = ()):
        """(tiled codes-or-values pointer, scale pointer) of a projection;
        `cat` concatenates several along the output dimension."""
        names = list(cat) or [name]
        if self.dtype == "fp8":
            q = torch.cat([weights[n + ".q"] for n in names], dim=-2) if len(names) > 1 else weights[name + ".q"]
            s = torch.cat([weights[n + ".s"] for n in names], dim=-1) if len(names) > 1 else weights[name + ".s"]
            return _ptr(self._tiled(q)), _ptr(self._dev(s.float()))
        w = torch.cat([weights[n] for n in names], dim=-2) if len(names) > 1 else weights[name]
        return _ptr(self._tiled(w)), None

    def _pack(self, cfg, weights):
        W = {"embed": _ptr(self._dev(weights["embed"])),
             "final_norm": _ptr(self._dev(weights["final_norm"].float()))}
        W["lm_head"], W["lm_head_s"] = self._proj(weights, "lm_head")
        layers = []
        for l in range(cfg.n_layers):
            p = f"{l}."
            L = abi.dlm_layer_weights()
            L.attn_norm = _ptr(self._dev(weights[p + "attn_norm"].float()))
            L.ffn_norm = _ptr(self._dev(weights[p + "ffn_norm"].float()))
            L.wqkv, L.wqkv_s = self._proj(weights, p + "wqkv", cat=(p + "wq", p + "wk", p + "wv"))
            L.wo, L.wo_s = self._proj(weights, p + "wo")
            L.w_gate, L.w_gate_s = self._proj(weights, p + "w_gate")
            L.w_up, L.w_up_s = self._proj(weights, p + "w_up")
            L.w_down, L.w_down_s = self._proj(weights, p + "w_down")
            if cfg.ffn == "moe":
                L.w_router = _ptr(self._dev(weights[p + "w_router"]))
                fmt = getattr(cfg, "expert_dtype", None)
                if fmt in _MX:
                    L.we_gate, L.we_gate_e8 = self._mx(weights, p + "we_gate", fmt)
                    L.we_up, L.we_up_e8 = self._mx(weights, p + "we_up", fmt)
                    L.we_down, L.we_down_e8 = self._mx(weights, p + "we_down", fmt)
                else:
                    L.we_gate, L.we_gate_s = self._proj(weights, p + "we_gate")
                    L.we_up, L.we_up_s = self._proj(weights, p + "we_up")
                    L.we_down, L.we_down_s = self._proj(weights, p + "we_down")
            layers.append(L)
        W["layers"] = layers
        return W

    # -------------------------------------------------------------- state --
    def new_seq(self, capacity: int, pool: Optional[KVPool] = None, order=None) -> Seq:
        """A request whose cache holds at least `capacity` tokens (rounded up to
        a multiple of 64, the attention kernel's key tile): its own contiguous
        cache, or pages from `pool` (`order(n_free)` picks which free page to
        take next; the default takes them in order)."""
        c = self.cfg
        capacity = -(-capacity // KV_PAGE) * KV_PAGE
        canvas = torch.full((self.C,), c.mask_id, dtype=torch.int32, device=self.device)
        if pool is None:
            kv = torch.empty((c.n_layers, 2, c.n_kv_heads, capacity * c.head_dim), dtype=self.kv_dtype,
                             device=self.device)
            raw = abi.dlm_seq(kv=kv.data_ptr(), capacity=capacity, T=0, canvas=canvas.data_ptr(),
                              page_table=None, page_size=0)
            return Seq(kv, canvas, raw, c.head_dim)
        pages = pool.alloc(capacity // KV_PAGE, order)
        raw = abi.dlm_seq(kv=pool.kv.data_ptr(), capacity=capacity, T=0, canvas=canvas.data_ptr(),
                          page_table=pages.data_ptr(), page_size=KV_PAGE)
        return Seq(pool.kv, canvas, raw, c.head_dim, pages, pool)

    def workspace_bytes(self, max_rows: int, max_kv: int) -> int:
        return int(self.lib.dlm_workspace_bytes(self.handle, max_rows, max_kv))

    def workspace(self, max_rows: int, max_kv: int) -> torch.Tensor:
        return torch.empty(self.workspace_bytes(max_rows, max_kv), dtype=torch.uint8, device=self.device)

    @staticmethod
    def _seq_array(seqs: Sequence[Seq]):
        arr = (ctypes.POINTER(abi.dlm_seq) * len(seqs))(*[ctypes.pointer(s.raw) for s in seqs])
        return arr

    # --------------------------------------------------------- operations --
    def dlm_prefill(self, seq: Seq, ids: torch.Tensor, ws: torch.Tensor) -> None:
        assert ids.dtype == torch.int32 and ids.is_contiguous() and ids.device.type == "cuda"
        check(self.lib.dlm_prefill(self.handle, ctypes.byref(seq.raw), ids.data_ptr(), ids.numel(),
                                   ws.data_ptr(), ws.numel(), _stream()), "dlm_prefill")

    def dlm_denoise_step(self, seqs: Sequence[Seq], conf: torch.Tensor, pred: torch.Tensor,
                         ws: torch.Tensor, logits: Optional[torch.Tensor] = None) -> None:
        n = len(seqs)
        assert conf.dtype == torch.float32 and conf.numel() >= n * self.C
        assert pred.dtype == torch.int32 and pred.numel() >= n * self.C
        if logits is not None:
            assert logits.dtype == torch.float32 and logits.numel() >= n * self.C * self.cfg.vocab
        arr = self._seq_array(seqs)
        check(self.lib.dlm_denoise_step(self.handle, arr, n, conf.data_ptr(), pred.data_ptr(),
                                        _ptr(logits), ws.data_ptr(), ws.numel(), _stream()),
              "dlm_denoise_step")

    def dlm_denoise_step_noalloc(self, seqs: Sequence[Seq], conf: torch.Tensor, pred: torch.Tensor,
                                 logits: Optional[torch.Tensor] = None) -> None:
        """dlm_denoise_step with the library's static per-device workspace
        (no workspace argument, nothing allocated)."""
        n = len(seqs)
        assert conf.dtype == torch.float32 and conf.numel() >= n * self.C
        assert pred.dtype == torch.int32 and pred.numel() >= n * self.C
        if logits is not None:
            assert logits.dtype == torch.float32 and logits.numel() >= n * self.C * self.cfg.vocab
        check(self.lib.dlm_denoise_step_noalloc(self.handle, self._seq_array(seqs), n, conf.data_ptr(),
                                                pred.data_ptr(), _ptr(logits), _stream()),
              "dlm_denoise_step_noalloc")

    def dlm_commit(self, seqs: Sequence[Seq], conf: torch.Tensor, pred: torch.Tensor, rule: "Rule",
                   step: int, n_committed: Optional[torch.Tensor] = None,
                   n_masked: Optional[torch.Tensor] = None) -> None:
        arr = self._seq_array(seqs)
        check(self.lib.dlm_commit(self.handle, arr, len(seqs), conf.data_ptr(), pred.data_ptr(),
                                  ctypes.byref(rule.raw), step, _ptr(n_committed), _ptr(n_masked),
                                  _stream()), "dlm_commit")

    def dlm_append_canvas(self, seqs: Sequence[Seq], ws: torch.Tensor) -> None:
        arr = self._seq_array(seqs)
        check(self.lib.dlm_append_canvas(self.handle, arr, len(seqs), ws.data_ptr(), ws.numel(),
                                         _stream()), "dlm_append_canvas")

    def dlm_check_device_status(self) -> int:
        bits = ctypes.c_int32(0)
        st = self.lib.dlm_check_device_status(self.handle, _stream(), ctypes.byref(bits))
        if st not in (abi.DLM_OK, abi.DLM_E_DEVICE):
            check(st, "dlm_check_device_status")
        return bits.value

    def dlm_debug_router(self, ids: Optional[torch.Tensor], logits: Optional[torch.Tensor] = None,
                         capacity_rows: int = 0) -> None:
        """Test hook: record each layer's router choices (int32 [L, rows, k]) and
        router logits (fp32 [L, rows, E]) of every forward."""
        check(self.lib.dlm_debug_router(self.handle, _ptr(ids), _ptr(logits), capacity_rows),
              "dlm_debug_router")

    # ------------------------------------------------------------- timing --
    def timing_enable(self, kernel_ids: Sequence[int]) -> None:
        mask = 0
        for k in kernel_ids:
            mask |= 1 << k
        check(self.lib.dlm_timing_enable(self.handle, mask), "dlm_timing_enable")

    def timing_read(self) -> Dict[str, tuple]:
        ms = (ctypes.c_float * abi.DLM_K_COUNT)()
        n = (ctypes.c_int32 * abi.DLM_K_COUNT)()
        check(self.lib.dlm_timing_read(self.handle, ms, n), "dlm_timing_read")
        return {self.lib.dlm_kernel_name(i).decode(): (ms[i], n[i])
                for i in range(abi.DLM_K_COUNT) if n[i]}

    def close(self) -> None:
        if getattr(self, "handle", None):
            self.lib.dlm_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class CanvasSteps:
    """The denoising steps of a canvas as HIP graphs, one per step: step s is
    dlm_denoise_step then dlm_commit(step=s) over `seqs` with the given
    outputs, rule and workspace, captured on torch's capture stream and
    replayed with `replay(s)`.  A graph repeats its launches exactly: the
    requests' T, cache, canvas and page-table pointers, the workspace, the
    outputs and the rule's counts are fixed at capture, so the graphs serve
    every canvas that starts with the same T in the same buffers (the canvas
    contents and the cache values may differ); `valid_for` checks all of
    them.  Capturing runs nothing."""

    def __init__(self, model: "DLM", seqs: Sequence[Seq], conf: torch.Tensor, pred: torch.Tensor, rule: "Rule",
                 ws: torch.Tensor, n_committed: Optional[torch.Tensor] = None,
                 n_masked: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None):
        self.key = self._key(seqs, conf, pred, rule, ws, n_committed, n_masked, logits)
        self.graphs = []
        self._keep = (seqs, conf, pred, rule, ws, n_committed, n_masked, logits)
        for step in range(rule.n_steps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                model.dlm_denoise_step(seqs, conf, pred, ws, logits)
                model.dlm_commit(seqs, conf, pred, rule, step, n_committed, n_masked)
            self.graphs.append(g)

    @staticmethod
    def _key(seqs, conf, pred, rule, ws, n_committed, n_masked, logits):
        per_seq = tuple((s.T, s.capacity, s.kv.data_ptr(), s.canvas.data_ptr(),
                         None if s.pages is None else s.pages.data_ptr()) for s in seqs)
        return (per_seq, conf.data_ptr(), pred.data_ptr(), ws.data_ptr(), ws.numel(), _ptr(n_committed),
                _ptr(n_masked), _ptr(logits), rule.signature())

    def valid_for(self, seqs: Sequence[Seq], conf: torch.Tensor, pred: torch.Tensor, rule: "Rule",
                  ws: torch.Tensor, n_committed: Optional[torch.Tensor] = None,
                  n_masked: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None) -> bool:
        return self.key == self._key(seqs, conf, pred, rule, ws, n_committed, n_masked, logits)

    def replay(self, step: int) -> None:
        self.graphs[step].replay()


class Rule:
    """A commit rule (top-k schedule or confidence threshold) in ABI form;
    edit_threshold > 0 adds token editing (earlier tokens whose prediction
    moved with confidence >= edit_threshold take the prediction)."""

    def __init__(self, kind: str, n_steps: int, k_per_step: Optional[Sequence[int]] = None,
                 threshold: float = 0.5, edit_threshold: float = 0.0):
        self.kind, self.n_steps = kind, n_steps
        self.edit_threshold = edit_threshold
        self._k = (ctypes.c_int32 * n_steps)(*(k_per_step or [0] * n_steps))
        self.raw = abi.dlm_commit_rule(
            kind=abi.DLM_COMMIT_TOPK if kind == "topk" else abi.DLM_COMMIT_THRESHOLD,
            n_steps=n_steps, k_per_step=ctypes.cast(self._k, ctypes.POINTER(ctypes.c_int32)),
            threshold=threshold, edit_threshold=edit_threshold)

    def signature(self) -> tuple:
        """Everything a captured commit depends on."""
        return (self.kind, self.n_steps, tuple(self._k), float(self.raw.threshold), float(self.edit_threshold))

    @staticmethod
    def topk(canvas: int, n_steps: int, edit_threshold: float = 0.0) -> "Rule":
        """Commit C // S per step, one more on the first C % S steps."""
        base, extra = divmod(canvas, n_steps)
        return Rule("topk", n_steps, [base + (1 if s < extra else 0) for s in range(n_steps)],
                    edit_threshold=edit_threshold)

    @staticmethod
    def threshold(n_steps: int, thr: float, edit_threshold: float = 0.0) -> "Rule":
        return Rule("threshold", n_steps, None, thr, edit_threshold)

    @staticmethod
    def for_run(run) -> "Rule":
        """The rule of a workload definition (its schedule, threshold and edit threshold)."""
        if run.rule == "topk":
            return Rule.topk(run.canvas, run.n_steps, run.edit_threshold)
        return Rule.threshold(run.n_steps, run.threshold, run.edit_threshold)


def generate(model: DLM, seqs: Sequence[Seq], prefixes: Sequence[torch.Tensor], rule: Rule,
             n_canvases: int, ws: torch.Tensor, on_step=None, graphs: Optional[dict] = None,
             logits: Optional[torch.Tensor] = None):
    """Prefill each request, then for each canvas: reset to [MASK], denoise and
    commit until the schedule ends (for the threshold rule, until nothing is
    masked in any request), append.  Returns the finished canvases
    [n_canvases][n_seqs, C] (device int32) and the steps run per canvas.

    `on_step(canvas_index, step, conf, pred)` sees every step after its commit
    (the canvases then hold the step's result).  `logits` (fp32, n_seqs * C *
    vocab): every step also writes its raw logits there, for inspection.
    `graphs`: a dict (kept by the caller across calls) turns the step loop into
    replays of per-step HIP graphs, captured on first use for each canvas
    index and captured again when the requests, buffers or rule differ from
    the ones they were captured with (see CanvasSteps); None runs every step
    as direct calls."""
    n = len(seqs)
    C = model.C
    for s, ids in zip(seqs, prefixes):
        model.dlm_prefill(s, ids, ws)

    def buf(name, numel, dtype):
        if graphs is None:
            return torch.empty(numel, dtype=dtype, device=model.device)
        t = graphs.get(name)
        if t is None or t.numel() != numel:
            t = graphs[name] = torch.empty(numel, dtype=dtype, device=model.device)
        return t
    conf = buf("conf", n * C, torch.float32)
    pred = buf("pred", n * C, torch.int32)
    n_masked = buf("n_masked", n, torch.int32)
    outs, steps = [], []
    for ci in range(n_canvases):
        for s in seqs:
            s.canvas.fill_(model.cfg.mask_id)
        cg = None
        if graphs is not None:
            cg = graphs.get(ci)
            if cg is None or not cg.valid_for(seqs, conf, pred, rule, ws, None, n_masked, logits):
                cg = graphs[ci] = CanvasSteps(model, seqs, conf, pred, rule, ws, None, n_masked, logits)
        st = 0
        for st in range(rule.n_steps):
            if cg is not None:
                cg.replay(st)
            else:
                model.dlm_denoise_step(seqs, conf, pred, ws, logits)
                model.dlm_commit(seqs, conf, pred, rule, st, None, n_masked)
            if on_step is not None:
                on_step(ci, st, conf, pred)
            if rule.kind == "threshold" and int(n_masked.cpu().max()) == 0:
                break
        steps.append(st + 1)
        outs.append(torch.stack([s.canvas.clone() for s in seqs]))
        model.dlm_append_canvas(seqs, ws)
    return outs, steps


def ar_decode(model: DLM, seqs: Sequence[Seq], prefixes: Sequence[torch.Tensor], n_tokens: int,
              ws: torch.Tensor, feed: Optional[Sequence[torch.Tensor]] = None,
              on_step=None, prefilled: bool = False) -> torch.Tensor:
    """Autoregressive decoding on the same weights and kernels (a block size of
    one): each pass runs a one-row canvas per request holding the newest token,
    at position T.  For one row the block attention is the causal one (the row
    sees the cache [0, T) and itself), the pass writes the row's K/V into slot
    T, and the argmax of its logits ([MASK] excluded, the LM head's fused
    reduction) is the next token; T then advances by one, which keeps that K/V
    (the append pass would compute the same values).  One forward per token.

    The prompt's last token is the first fed row, so the prompt minus that
    token is prefilled (`prefilled`: the caller did that; `prefixes` then
    only supplies the last tokens).  `feed` (teacher forcing, for parity
    tests) gives the row fed at each step instead of the previous argmax:
    [n_tokens][n_seqs].  Returns the argmax tokens [n_seqs, n_tokens] (device
    int32)."""
    assert model.C == 1, "AR decoding needs a model built with canvas=1"
    n = len(seqs)
    if not prefilled:
        for s, ids in zip(seqs, prefixes):
            assert len(ids) >= 2, "the prompt needs at least two tokens"
            model.dlm_prefill(s, ids[:-1], ws)
    conf = torch.empty(n, dtype=torch.float32, device=model.device)
    pred = torch.empty(n, dtype=torch.int32, device=model.device)
    cur = torch.stack([ids[-1:].to(model.device, torch.int32) for ids in prefixes]).view(n)
    out = torch.empty(n, n_tokens, dtype=torch.int32, device=model.device)
    for t in range(n_tokens):
        row = cur if feed is None else feed[t].to(model.device, torch.int32)
        for r, s in enumerate(seqs):
            s.canvas.copy_(row[r:r + 1])
        model.dlm_denoise_step(seqs, conf, pred, ws)
        for s in seqs:
            s.raw.T += 1
        out[:, t] = pred
        cur = pred.clone()
        if on_step is not None:
            on_step(t, conf, pred)
    return out
