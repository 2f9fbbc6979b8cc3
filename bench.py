"""Benchmark of the block-diffusion hot path on one MI355X.

One bench step is one whole request through the library: causal prefill of
the prompt, then per canvas the denoising steps (each a bidirectional forward
+ LM head + fused vocab reduction, then the confidence-ranked commit) and the
append of the finished canvas to the KV cache.  `value` is decode-only
committed tokens per second: the tokens of the K timed requests over their
wall time minus their prefills (timed with HIP events on the library's
stream); `end_to_end_tokens_per_s` counts the prefills too.  Inputs are
resident in HBM before the timed region.

Default workload: the 32-layer 26B-class MoE (d=2560, 20 Q / 4 KV heads x 128,
128 experts top-8 x 768 + shared SwiGLU 2048, vocab 262144) in bf16 at batch
1, with a 4096-token prefix and 4 canvases of 12 steps (21-22 commits each),
each appended to the KV cache -- the shape of the pages' single-GPU
measurement (4096 tokens in, 1024 out).  `--workload dense` runs the dense
16-layer d=2048 bf16 model (1024-token prefix, one canvas of 16 x 16);
`moe-fp8` the MoE with E4M3 GEMMs and the confidence-threshold rule;
`moe-batch32` 32 requests with prefixes of 512..4096 tokens denoised together.  Weights and prompts are
seeded synthetic draws (random init).  Models up to a few billion parameters
are drawn on the host and copied, so the CPU baseline reads the same bytes;
the 26B-class ones are drawn on the GPU, and the CPU baseline reads a copy of
the layers it samples.

Also reported: ms per denoising step (denoise + commit, CUDA events on the
library's stream), and the roofline of the dominant kernel of the denoising
step.  The dominant kernel is found in an untimed warmup request with every
kernel timed; in the timed region only it is bracketed by the library's HIP
events (on the stream it runs on), and its algorithmic bytes and flops per
launch (models below) over its average launch time give the achieved rate.
The CPU oracle is timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "committed tokens/s at batch 1 (256-canvas); ms per denoise step; MFMA util %"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}


def _workload_text(run) -> str:
    m = run.model
    ffn = (f"SwiGLU {m.d_ffn}" if m.ffn == "dense" else
           f"{m.n_experts} experts top-{m.top_k} x {m.d_expert} + shared {m.d_ffn}")
    rule = (f"{run.n_steps} steps top-k" if run.rule == "topk" else
            f"<= {run.n_steps} steps, confidence >= {run.threshold}")
    return (f"{m.name}: {m.n_layers}L d={m.d_model} {m.n_q_heads}q/{m.n_kv_heads}kv x {m.head_dim}, {ffn}, "
            f"vocab {m.vocab}; prefix {run.prefix_len[1]}, {run.n_canvases} x {run.canvas}-token canvas, "
            f"{rule}, append")


def experts_touched(E: int, k: int, rows: int) -> float:
    """Expected number of distinct experts a step's rows route to when each row
    picks k of E experts: E (1 - (1 - k/E)^rows)."""
    return E * (1.0 - (1.0 - k / E) ** rows)


def kernel_model(name: str, cfg, rows: int, keys_per_req, experts_used=None):
    """Algorithmic (bytes, flops) of one launch of a denoising-step kernel over
    `rows` canvas rows (R requests x C) whose requests attend to
    `keys_per_req` keys each.  Bytes: weights and activations read once,
    outputs written once (x read and written for residual adds); flops: 2 per
    multiply-add of the contraction.  Grouped expert GEMMs read the weights of
    the experts the rows route to: `experts_used` (the mean number of distinct
    experts per launch, counted from the routing), else the count expected
    from independent uniform choices (`experts_touched`)."""
    d, F, dh = cfg.d_model, cfg.d_ffn, cfg.head_dim
    qd, kvd = cfg.n_q_heads * dh, cfg.n_kv_heads * dh
    nqkv = qd + 2 * kvd
    eb = 1 if cfg.dtype == "fp8" else (4 if cfg.dtype == "f32" else 2)
    ab = 4 if cfg.dtype == "f32" else 2          # stored activation element
    M = rows
    if name == "gemm_qkv":
        return nqkv * d * eb + M * d * eb + M * nqkv * 4, 2.0 * M * nqkv * d
    if name == "gemm_o":
        return d * qd * eb + M * qd * eb + 2 * M * d * 4, 2.0 * M * d * qd
    if name == "gemm_gate_up":
        return 2 * F * d * eb + M * d * eb + M * F * ab, 2.0 * M * 2 * F * d
    if name == "gemm_down":
        return d * F * eb + M * F * eb + 2 * M * d * 4, 2.0 * M * d * F
    if name == "lm_head":
        return cfg.vocab * d * eb + M * d * eb, 2.0 * M * cfg.vocab * d
    if name == "router":
        wb = 4 if cfg.dtype == "f32" else 2
        return cfg.n_experts * d * wb + M * d * wb + M * cfg.n_experts * 4, 2.0 * M * cfg.n_experts * d
    if name in ("expert_gate_up", "expert_down") and cfg.ffn == "moe":
        De, A = cfg.d_expert, M * cfg.top_k
        used = experts_used if experts_used is not None else experts_touched(cfg.n_experts, cfg.top_k, M)
        # MX experts: 4-bit (MXFP4) or 6-bit (MXFP6) codes plus one E8M0 byte per
        # 32 weights; bf16 activations
        mx_bits = {"mxfp4": 4, "mxfp6": 6}.get(getattr(cfg, "expert_dtype", None))
        web, aeb = (mx_bits / 8 + 1.0 / 32, 2) if mx_bits else (eb, eb)
        if name == "expert_gate_up":
            return used * 2 * De * d * web + A * d * aeb + A * De * ab, 2.0 * A * 2 * De * d
        return used * d * De * web + A * De * aeb + A * d * 4, 2.0 * A * d * De
    if name == "attention":
        keys = sum(keys_per_req)
        return (2 * keys * kvd * ab + 2 * M * qd * ab,
                4.0 * (M // len(keys_per_req)) * cfg.n_q_heads * keys * dh)
    return None


def traffic_record(kernel: str, workload: str, root: str = ROOT):
    """The committed PMC traffic record (profiles/*_traffic.md under `root`)
    of `kernel` on `workload`, if the sources it was measured on are unchanged:
    the record holds the SHA-256 of those files, recomputed here (a source
    that no longer exists makes the record stale)."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(root, "profiles", "*_traffic.md"))):
        for line in open(path):
            if not line.startswith("traffic-record: "):
                continue
            rec = json.loads(line[len("traffic-record: "):])
            if rec.get("kernel") != kernel or rec.get("workload") != workload:
                continue
            h = hashlib.sha256()
            for f in rec["sources"]:
                src = os.path.join(root, "masked_block_diffusion_amd", "csrc", f)
                if not os.path.exists(src):        # a source renamed or removed since: stale
                    h = None
                    break
                h.update(f.encode())
                with open(src, "rb") as fh:
                    h.update(fh.read())
            if h is not None and h.hexdigest() == rec["sources_sha256"]:
                rec["file"] = os.path.relpath(path, root)
                return rec
    return None


def roofline(name, cfg, rows, keys_per_req, avg_ms, experts_used=None):
    m = kernel_model(name, cfg, rows, keys_per_req, experts_used)
    if m is None or avg_ms <= 0:
        return None
    nbytes, flops = m
    s = avg_ms * 1e-3
    peak_tf = MFMA_PEAK_TFLOPS[cfg.dtype]
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (peak_tf * 1e12)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    out = {"kernel": name, "bound": bound}
    if bound == "hbm":
        out.update(achieved=nbytes / s / 1e9, peak=HBM_PEAK_GBS, unit="GB/s",
                   frac=nbytes / s / 1e9 / HBM_PEAK_GBS)
    else:
        out.update(achieved=flops / s / 1e12, peak=peak_tf, unit="TFLOP/s",
                   frac=flops / s / 1e12 / peak_tf)
    out.update(traffic=None, algorithmic_bytes_per_launch=nbytes, flops_per_launch=flops,
               avg_launch_ms=avg_ms, mfma_util_pct=100.0 * flops / s / 1e12 / peak_tf,
               hbm_gbs=nbytes / s / 1e9)
    return out


def _layer_of(name: str):
    head = name.split(".", 1)[0]
    return int(head) if head.isdigit() else None


def cpu_baseline(run, weights, prefix_cpu, steps_per_canvas: float, sample_layers=None):
    """The oracle on the host, on a bounded sample of the same workload and
    weights: prefill of request 0's prompt, one denoising step with its commit,
    and one append.  With `sample_layers` the sample model keeps only the
    first layers (full width: embedding, those layers, LM head); the per-layer
    time is scaled to the model's depth, the LM head (timed alone) counted
    once per step.  The request time is extrapolated to the schedule's steps
    and canvases, and to R requests (the oracle serves them one after another)."""
    from dataclasses import replace

    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import sampler as osampler
    from oracle.model import OracleModel, OracleWeights

    cfg = run.model
    L = cfg.n_layers
    Ls = L if sample_layers is None else min(sample_layers, L)
    cfg_s = replace(cfg, n_layers=Ls)
    host = {k: v.cpu() for k, v in weights.items() if _layer_of(k) is None or _layer_of(k) < Ls}
    om = OracleModel(cfg_s, OracleWeights(cfg_s, host))
    del host
    C = run.canvas
    st = om.new_seq(len(prefix_cpu) + C)
    t0 = time.perf_counter()
    om.prefill(st, prefix_cpu.numpy())
    t1 = time.perf_counter()
    canvas = np.full(C, cfg.mask_id, dtype=np.int32)
    conf, pred, _ = om.denoise(st, canvas)
    canvas, _ = osampler.commit(canvas, conf, pred, cfg.mask_id, run, 0)
    t2 = time.perf_counter()
    canvas[canvas == cfg.mask_id] = 0
    om.append(st, canvas)
    t3 = time.perf_counter()
    lm = 0.0
    if Ls < L:
        x = np.zeros((C, cfg.d_model))
        x[:, 0] = 1.0
        tl = time.perf_counter()
        om.logits(x)
        lm = time.perf_counter() - tl
    scale = L / Ls
    prefill_s = (t1 - t0) * scale
    step_s = (t2 - t1 - lm) * scale + lm
    append_s = (t3 - t2) * scale
    per_req = prefill_s + run.n_canvases * (steps_per_canvas * step_s + append_s)
    R = run.n_requests
    info = threadpool_info()
    threads = max([p.get("num_threads", 1) for p in info] or [1])
    blas = sorted({f"{p.get('internal_api', '?')} {p.get('version', '')}".strip() for p in info
                   if p.get("user_api") == "blas"})
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    what = (f"the whole {L}-layer model" if Ls == L else
            f"{Ls} of {L} layers at full width (embedding, {'layers 0..' + str(Ls - 1) if Ls > 1 else 'layer 0'}, LM head "
            f"{lm:.2f} s timed alone), layer time scaled x{scale:g}")
    return {
        "value": R * C * run.n_canvases / (R * per_req),
        "unit": "tokens/s",
        "cores": threads,
        "host_cpus": os.cpu_count(),
        "cpu_model": cpu_model,
        "blas": ", ".join(blas),
        "kind": "oracle",
        "sample": (f"float64 numpy oracle on the host ({threads} BLAS threads), {what}: prefill of the "
                   f"{len(prefix_cpu)}-token prompt of request 0 ({t1 - t0:.2f} s), one denoising step + commit "
                   f"({t2 - t1:.2f} s) and one append ({t3 - t2:.2f} s) with the same weights; extrapolated to "
                   f"{steps_per_canvas:g} steps x {run.n_canvases} canvas(es)"
                   + (f" x {R} requests, each taken as long as request 0" if R > 1 else "")),
        "s_per_denoise_step": step_s,
    }


def ar_sweep(args):
    """Committed tokens/s of autoregressive decoding (a block size of one: one
    row per request and pass, one token per pass) and of block diffusion (the
    workload's canvas and schedule), for each request count R, on the same
    model, weights and kernels.  Prefills are excluded on both sides; each
    side is timed after an untimed warmup (8 AR tokens; one canvas)."""
    import torch

    import synth
    from masked_block_diffusion_amd import DLM, Rule, ar_decode, generate  # noqa: F401

    def log(msg):
        print(f"[ar-sweep] {msg}", file=sys.stderr, flush=True)

    run = synth.get_run(args.workload)
    cfg, C, P = run.model, run.canvas, run.max_prefix
    big = cfg.n_params()["total"] > 4e9
    weights = synth.make_weights(cfg, seed=run.seed, device="cuda" if big else "cpu")
    weights = weights if big else {k: v.cuda() for k, v in weights.items()}
    ar_model = DLM(cfg, weights, canvas=1)
    df_model = DLM(cfg, weights, canvas=C)
    rule = Rule.for_run(run)
    N = args.ar_tokens
    rows = []
    for R in [int(x) for x in args.ar_requests.split(",")]:
        prompts = [synth.prefix_ids(run, r, P).cuda() for r in range(R)]
        # AR: prefill P - 1 tokens, 8 untimed tokens, then N timed
        cap = P + 8 + N
        seqs = [ar_model.new_seq(cap) for _ in range(R)]
        ws = ar_model.workspace(max(R, P), cap)
        for s, ids in zip(seqs, prompts):
            ar_model.dlm_prefill(s, ids[:-1], ws)
        warm = ar_decode(ar_model, seqs, prompts, 8, ws, prefilled=True)
        last = [warm[r, -1:] for r in range(R)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ar_decode(ar_model, seqs, last, N, ws, prefilled=True)
        torch.cuda.synchronize()
        t_ar = time.perf_counter() - t0
        del seqs, ws
        # block diffusion: prefill P, one untimed canvas, one timed canvas (steps + commits + append)
        cap = P + 2 * C
        seqs = [df_model.new_seq(cap) for _ in range(R)]
        ws = df_model.workspace(max(R * C, P), cap)
        conf = torch.empty(R * C, dtype=torch.float32, device="cuda")
        pred = torch.empty(R * C, dtype=torch.int32, device="cuda")
        n_masked = torch.empty(R, dtype=torch.int32, device="cuda")
        for s, ids in zip(seqs, prompts):
            df_model.dlm_prefill(s, ids, ws)

        def canvas():
            for s in seqs:
                s.canvas.fill_(cfg.mask_id)
            for st in range(rule.n_steps):
                df_model.dlm_denoise_step(seqs, conf, pred, ws)
                df_model.dlm_commit(seqs, conf, pred, rule, st, None, n_masked)
                if rule.kind == "threshold" and int(n_masked.cpu().max()) == 0:
                    break
            df_model.dlm_append_canvas(seqs, ws)
        canvas()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        canvas()
        torch.cuda.synchronize()
        t_df = time.perf_counter() - t0
        del seqs, ws
        torch.cuda.empty_cache()
        row = {"requests": R, "ar_tokens_per_s": R * N / t_ar, "ar_ms_per_pass": 1e3 * t_ar / N,
               "diffusion_tokens_per_s": R * C / t_df, "diffusion_ms_per_canvas": 1e3 * t_df}
        row["diffusion_over_ar"] = row["diffusion_tokens_per_s"] / row["ar_tokens_per_s"]
        log(json.dumps({k: round(v, 3) if isinstance(v, float) else v for k, v in row.items()}))
        rows.append(row)
    cross = next((r["requests"] for r in rows if r["diffusion_over_ar"] < 1.0), None)
    print(json.dumps({"metric": "committed tokens/s, AR decoding vs block diffusion", "unit": "tokens/s",
                      "n_gpus": 1, "workload": _workload_text(run), "ar_tokens_timed": N,
                      "data": "synthetic (seeded random-init weights and uniform random prompt ids)",
                      "dtype": cfg.dtype, "sweep": rows, "first_requests_where_ar_wins": cross}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="moe",
                    help="moe (default: the 26B-class MoE, bf16, batch 1), dense, moe-fp8, moe-batch32, tiny, "
                         "or a reduced run name")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="for runs under a profiler: no per-kernel event timing (no roofline), "
                         "no expert counting, no CPU baseline")
    ap.add_argument("--no-graphs", action="store_true", help="skip the HIP-graph replay measurement")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="with --profile: one canvas of this many denoising steps per request")
    ap.add_argument("--ar-sweep", action="store_true",
                    help="autoregressive decoding (one-row canvas, one token per pass) against block "
                         "diffusion over request counts --ar-requests, on the same weights and kernels; "
                         "prints its own JSON line")
    ap.add_argument("--ar-requests", default="1,2,4,8,16,32,64")
    ap.add_argument("--ar-tokens", type=int, default=64, help="tokens per request timed in AR mode")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only a plain 256 MiB device copy, four times (the reference kernel that scales the "
                         "HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        a = torch.randn(64 * 1024 * 1024, device="cuda")           # 256 MiB of fp32
        b = torch.empty_like(a)
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize()
        print("copied 4 x 256 MiB", flush=True)
        return
    if args.ar_sweep:
        return ar_sweep(args)
    if args.profile:
        args.no_cpu_baseline = True
        args.no_graphs = True
    elif args.profile_steps:
        ap.error("--profile-steps needs --profile")
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library runs the hot path on a single MI355X "
              "(no multi-GPU path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from masked_block_diffusion_amd import DLM, CanvasSteps, Rule
    from masked_block_diffusion_amd import abi

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    run = synth.get_run(args.workload)
    if args.profile_steps:
        from dataclasses import replace
        run = replace(run, n_canvases=1, n_steps=args.profile_steps)
    cfg, C, R = run.model, run.canvas, run.n_requests
    big = cfg.n_params()["total"] > 4e9
    t = time.perf_counter()
    weights = synth.make_weights(cfg, seed=run.seed, device="cuda" if big else "cpu")
    prefixes_cpu = synth.make_inputs(run)
    log(f"{cfg.name}: weights drawn on the {'GPU' if big else 'host'} in {time.perf_counter() - t:.1f} s")
    model = DLM(cfg, weights if big else {k: v.cuda() for k, v in weights.items()}, canvas=C)
    cap = run.capacity()
    if R > 1:     # independent requests: each cache in 64-token pages of one shared pool
        from masked_block_diffusion_amd import KVPool
        pool = KVPool(model, R * (-(-cap // 64)))
        seqs = [model.new_seq(cap, pool) for _ in range(R)]
    else:
        seqs = [model.new_seq(cap) for _ in range(R)]
    ws = model.workspace(max(R * C, run.max_prefix), cap)
    prefixes = [p.cuda() for p in prefixes_cpu]
    rule = Rule.for_run(run)
    conf = torch.empty(R * C, dtype=torch.float32, device="cuda")
    pred = torch.empty(R * C, dtype=torch.int32, device="cuda")
    n_masked = torch.empty(R, dtype=torch.int32, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4 * run.n_canvases)]
    pf_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    prefill_ms = []       # per timed request
    all_ids = list(range(abi.DLM_K_COUNT))

    moe = cfg.ffn == "moe"
    L = cfg.n_layers
    dbg_ids = torch.empty(L * R * C * max(1, cfg.top_k), dtype=torch.int32, device="cuda") if moe else None
    used_per_launch = []     # distinct experts per (step, layer), MoE only

    graph_cache = {}

    def one_request(timed_ids, count_experts=False, graphs=False, time_prefill=False):
        if time_prefill:
            pf_ev[0].record()
        for s, ids in zip(seqs, prefixes):
            s.raw.T = 0
            model.dlm_prefill(s, ids, ws)
        if time_prefill:
            pf_ev[1].record()
        steps_run = 0
        for ci in range(run.n_canvases):
            for s in seqs:
                s.canvas.fill_(cfg.mask_id)
            cg = None
            if graphs:
                cg = graph_cache.get(ci)
                if cg is None or not cg.valid_for(seqs, conf, pred, rule, ws, None, n_masked):
                    cg = graph_cache[ci] = CanvasSteps(model, seqs, conf, pred, rule, ws, None, n_masked)
            model.timing_enable(timed_ids)
            ev[4 * ci].record()
            if count_experts:
                model.dlm_debug_router(dbg_ids, None, L * R * C)
            for st in range(run.n_steps):
                if cg is not None:
                    cg.replay(st)
                    steps_run += 1
                    if run.rule == "threshold" and int(n_masked.max().cpu()) == 0:
                        break
                    continue
                model.dlm_denoise_step(seqs, conf, pred, ws)
                if count_experts:
                    hit = torch.zeros(L, cfg.n_experts, device="cuda")
                    hit.scatter_(1, dbg_ids.view(L, -1).long(), 1.0)
                    used_per_launch.append(hit.sum(1))
                model.dlm_commit(seqs, conf, pred, rule, st, None, n_masked)
                steps_run += 1
                if run.rule == "threshold" and int(n_masked.max().cpu()) == 0:
                    break
            ev[4 * ci + 1].record()
            if count_experts:
                model.dlm_debug_router(None, None, 0)
            model.timing_enable([])
            ev[4 * ci + 2].record()
            model.dlm_append_canvas(seqs, ws)
            ev[4 * ci + 3].record()
        if time_prefill:
            prefill_ms.append(pf_ev[0].elapsed_time(pf_ev[1]))     # synchronises on the prefill's end only
        return steps_run

    log(f"warmup {args.warmup} (+1 with every kernel timed)")
    for _ in range(args.warmup):
        one_request([])
    torch.cuda.synchronize()
    model.timing_read()
    if args.profile:
        steps_full, per_kernel, experts_used, dominant, dom_ids = 1, {}, None, None, []
    else:
        steps_full = one_request(all_ids, count_experts=moe)
        torch.cuda.synchronize()
        per_kernel = model.timing_read()
        experts_used = float(torch.cat(used_per_launch).mean()) if used_per_launch else None
        # MoE models run the shared expert (gemm_gate_up, gemm_down) on a second
        # stream beside the routing chain: their dispatch times include the
        # time they share the chip, so they are not candidates
        overlapped = {"gemm_gate_up", "gemm_down"} if moe else set()
        dominant = max((k for k in per_kernel if k not in overlapped), key=lambda k: per_kernel[k][0])
        dom_ids = [i for i in all_ids if model.lib.dlm_kernel_name(i).decode() == dominant]
    log(f"dominant denoise kernel: {dominant}; timing {args.steps} requests")

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n_denoise = 0
    for _ in range(args.steps):
        n_denoise += one_request(dom_ids, time_prefill=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kt = model.timing_read()
    denoise_ms = sum(ev[4 * ci].elapsed_time(ev[4 * ci + 1]) for ci in range(run.n_canvases))
    append_ms = sum(ev[4 * ci + 2].elapsed_time(ev[4 * ci + 3]) for ci in range(run.n_canvases))
    status = model.dlm_check_device_status()
    if status:
        log(f"device error word {status}")
        sys.exit(1)
    elapsed = t1 - t0
    tokens = args.steps * R * C * run.n_canvases
    steps_last = n_denoise // args.steps
    ms_k, n_k = kt.get(dominant, (0.0, 0))
    rows = R * C
    keys = [len(p) + C * (run.n_canvases + 1) / 2 for p in prefixes_cpu]   # mean over the canvases
    step_ms = denoise_ms / max(1, steps_last)
    decode_s = elapsed - 1e-3 * sum(prefill_ms)
    out = {
        "metric": METRIC,
        "value": tokens / decode_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded random-init weights and uniform random prompt ids)",
        "config": {
            "workload": _workload_text(run),
            "global_batch": R,
            "seq_len": run.max_prefix + run.n_canvases * C,
            "canvas": C,
            "prefix": run.max_prefix if R == 1 else [len(p) for p in prefixes_cpu],
            "denoise_steps_per_canvas": steps_last / run.n_canvases,
            "parallelism": "single GPU",
            "kv_cache": "paged, 64-token pages of one pool" if R > 1 else "contiguous per request",
        },
        "value_note": ("decode only: committed tokens of the timed requests over their wall time minus their "
                       "prefills (HIP events); ms_per_step is the whole request, prefill included"),
        "end_to_end_tokens_per_s": tokens / elapsed,
        "prefill_ms": sum(prefill_ms) / max(1, len(prefill_ms)),
        "ms_per_denoise_step": step_ms,
        "last_request_denoise_append_tokens_per_s": (R * C * run.n_canvases / ((denoise_ms + append_ms) * 1e-3)
                                                     if denoise_ms else None),
        "roofline": roofline(dominant, cfg, rows, keys, ms_k / max(1, n_k), experts_used) if dominant else None,
        "denoise_step_kernels_ms": {k: round(v[0] / max(1, steps_full), 4) for k, v in
                                    sorted(per_kernel.items(), key=lambda kv: -kv[1][0])},
    }
    if moe:
        out["denoise_step_kernels_note"] = ("gemm_gate_up / gemm_down are the shared expert, run on a second stream "
                                            "concurrently with router .. expert_down: their times overlap others")
    if not args.no_graphs:
        # the same requests with the step loop replayed from per-step HIP graphs
        # (captured in an untimed request; see CanvasSteps)
        log(f"graph replay: capture, then {args.steps} timed requests")
        one_request([], graphs=True)
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        g_steps = 0
        for _ in range(args.steps):
            g_steps += one_request([], graphs=True)
        torch.cuda.synchronize()
        g1 = time.perf_counter()
        g_denoise = sum(ev[4 * ci].elapsed_time(ev[4 * ci + 1]) for ci in range(run.n_canvases))
        out["graph_replay"] = {
            "value": tokens / (g1 - g0), "unit": "tokens/s",
            "ms_per_step": 1e3 * (g1 - g0) / args.steps,
            "ms_per_denoise_step": g_denoise / max(1, g_steps // args.steps),
            "note": "step loop (denoise + commit) replayed from per-step HIP graphs; prefill and append direct",
        }
    rec = traffic_record(dominant, args.workload) if dominant else None
    if rec and out["roofline"]:
        out["roofline"]["traffic"] = rec["traffic_bytes_per_launch"]
        out["roofline"]["traffic_note"] = (
            f"HBM bytes per launch: FETCH_SIZE x {rec['fetch_scale']} + WRITE_SIZE x {rec['write_scale']} "
            f"(scales from a plain 256 MiB copy), {rec['file']}")
        out["roofline"]["traffic_over_algorithmic"] = rec["traffic_bytes_per_launch"] / out["roofline"][
            "algorithmic_bytes_per_launch"]
    if experts_used is not None:
        out["experts_used_per_layer_step"] = {
            "mean": experts_used, "of": cfg.n_experts,
            "first_step": float(used_per_launch[0].mean()), "last_step": float(used_per_launch[-1].mean()),
            "uniform_expectation": experts_touched(cfg.n_experts, cfg.top_k, rows)}
    for name, (ms, n) in per_kernel.items():
        r = roofline(name, cfg, rows, keys, ms / max(1, n), experts_used)
        if r:
            out.setdefault("kernel_rooflines", {})[name] = {k: r[k] for k in ("bound", "frac", "hbm_gbs",
                                                                              "mfma_util_pct", "avg_launch_ms")}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle sample)")
        if big:
            host = {k: v for k, v in weights.items() if _layer_of(k) is None or _layer_of(k) < 1}
            del model, weights
            torch.cuda.empty_cache()
            out["cpu_baseline"] = cpu_baseline(run, host, prefixes_cpu[0], steps_last / run.n_canvases,
                                               sample_layers=1)
        else:
            del model
            out["cpu_baseline"] = cpu_baseline(run, weights, prefixes_cpu[0], steps_last / run.n_canvases)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
