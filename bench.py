"""Benchmark of the block-diffusion hot path on one MI355X.

One bench step is one whole request through the library: causal prefill of
the prompt, then per canvas the denoising steps (each a bidirectional forward
+ LM head + fused vocab reduction, then the confidence-ranked commit) and the
append of the finished canvas to the KV cache.  `value` is committed tokens per
second over the K timed steps, inputs already resident in HBM.

Default workload: the dense 16-layer d=2048 bf16 model (16 Q / 4 KV heads x
128, SwiGLU 8192, vocab 32768) with a 1024-token prefix and one 256-token
canvas, 16 steps x 16 commits, then the append.  Weights and prompt are seeded
synthetic draws (random init) generated on the host, so the CPU baseline reads
the same bytes.

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


def kernel_model(name: str, cfg, C: int, keys: int):
    """Algorithmic (bytes, flops) of one launch of a denoising-step kernel over
    a C-row canvas attending to `keys` keys.  Bytes: weights and activations
    read once, outputs written once (x read and written for residual adds);
    flops: 2 per multiply-add of the contraction."""
    d, F, dh = cfg.d_model, cfg.d_ffn, cfg.head_dim
    qd, kvd = cfg.n_q_heads * dh, cfg.n_kv_heads * dh
    nqkv = qd + 2 * kvd
    eb = 1 if cfg.dtype == "fp8" else (4 if cfg.dtype == "f32" else 2)
    ab = 4 if cfg.dtype == "f32" else 2          # stored activation element
    if name == "gemm_qkv":
        return nqkv * d * eb + C * d * eb + C * nqkv * 4, 2.0 * C * nqkv * d
    if name == "gemm_o":
        return d * qd * eb + C * qd * eb + 2 * C * d * 4, 2.0 * C * d * qd
    if name == "gemm_gate_up":
        return 2 * F * d * eb + C * d * eb + C * F * ab, 2.0 * C * 2 * F * d
    if name == "gemm_down":
        return d * F * eb + C * F * eb + 2 * C * d * 4, 2.0 * C * d * F
    if name == "lm_head":
        return cfg.vocab * d * eb + C * d * eb, 2.0 * C * cfg.vocab * d
    if name == "attention":
        return (2 * keys * kvd * ab + 2 * C * qd * ab,
                4.0 * C * cfg.n_q_heads * keys * dh)
    return None


def roofline(name, cfg, C, keys, avg_ms):
    m = kernel_model(name, cfg, C, keys)
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


def cpu_baseline(run, weights_cpu, prefix_cpu):
    """The oracle on the host, on a bounded sample of the same workload: prefill
    of the full prompt, one denoising step with its commit, and one append;
    the request time is extrapolated to the schedule's step count."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import sampler as osampler
    from oracle.model import OracleModel, OracleWeights

    cfg = run.model
    om = OracleModel(cfg, OracleWeights(cfg, weights_cpu))
    st = om.new_seq(run.capacity())
    t0 = time.perf_counter()
    om.prefill(st, prefix_cpu.numpy())
    t1 = time.perf_counter()
    canvas = np.full(run.canvas, cfg.mask_id, dtype=np.int32)
    conf, pred, _ = om.denoise(st, canvas)
    canvas, _ = osampler.commit(canvas, conf, pred, cfg.mask_id, run, 0)
    t2 = time.perf_counter()
    canvas[canvas == cfg.mask_id] = 0
    om.append(st, canvas)
    t3 = time.perf_counter()
    per_req = (t1 - t0) + run.n_canvases * (run.n_steps * (t2 - t1) + (t3 - t2))
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {
        "value": run.canvas * run.n_canvases / per_req,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"float64 numpy oracle on the host ({threads} BLAS threads): prefill of the "
                   f"{len(prefix_cpu)}-token prompt ({t1 - t0:.2f} s), one denoising step + commit "
                   f"({t2 - t1:.2f} s) and one append ({t3 - t2:.2f} s) of the same workload and weights; "
                   f"the request is extrapolated to {run.n_steps} steps per canvas"),
        "s_per_denoise_step": t2 - t1,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="dense")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build runs the hot path on a single MI355X "
              "(no multi-GPU path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from masked_block_diffusion_amd import DLM, Rule
    from masked_block_diffusion_amd import abi

    run = synth.get_run(args.workload)
    cfg, C = run.model, run.canvas
    t = time.perf_counter()
    w_cpu = synth.make_weights(cfg, seed=run.seed)
    prefix_cpu = synth.make_inputs(run)[0]
    print(f"[bench] weights generated in {time.perf_counter() - t:.1f} s", file=sys.stderr, flush=True)
    model = DLM(cfg, {k: v.cuda() for k, v in w_cpu.items()}, canvas=C)
    cap = run.capacity()
    seq = model.new_seq(cap)
    ws = model.workspace(max(C, run.max_prefix), cap)
    prefix = prefix_cpu.cuda()
    rule = Rule.topk(C, run.n_steps) if run.rule == "topk" else Rule.threshold(run.n_steps, run.threshold)
    conf = torch.empty(C, dtype=torch.float32, device="cuda")
    pred = torch.empty(C, dtype=torch.int32, device="cuda")
    n_masked = torch.empty(1, dtype=torch.int32, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * run.n_canvases)]
    all_ids = list(range(abi.DLM_K_COUNT))

    def one_request(timed_ids):
        seq.raw.T = 0
        model.dlm_prefill(seq, prefix, ws)
        steps_run = 0
        for ci in range(run.n_canvases):
            seq.canvas.fill_(cfg.mask_id)
            model.timing_enable(timed_ids)
            ev[2 * ci].record()
            for s in range(run.n_steps):
                model.dlm_denoise_step([seq], conf, pred, ws)
                model.dlm_commit([seq], conf, pred, rule, s, None, n_masked)
                steps_run += 1
                if run.rule == "threshold" and int(n_masked.cpu()[0]) == 0:
                    break
            ev[2 * ci + 1].record()
            model.timing_enable([])
            model.dlm_append_canvas([seq], ws)
        return steps_run

    print(f"[bench] warmup {args.warmup} (+1 with every kernel timed)", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        one_request([])
    torch.cuda.synchronize()
    model.timing_read()
    one_request(all_ids)
    torch.cuda.synchronize()
    per_kernel = model.timing_read()
    dominant = max(per_kernel, key=lambda k: per_kernel[k][0])
    dom_id = [i for i in all_ids if model.lib.dlm_kernel_name(i).decode() == dominant][0]

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n_denoise = 0
    for _ in range(args.steps):
        n_denoise += one_request([dom_id])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kt = model.timing_read()
    denoise_ms = sum(ev[2 * ci].elapsed_time(ev[2 * ci + 1]) for ci in range(run.n_canvases))
    status = model.dlm_check_device_status()
    if status:
        print(f"[bench] device error word {status}", file=sys.stderr)
        sys.exit(1)
    elapsed = t1 - t0
    tokens = args.steps * C * run.n_canvases
    steps_last = n_denoise // args.steps
    ms_k, n_k = kt.get(dominant, (0.0, 0))
    keys = run.max_prefix + C
    step_ms = denoise_ms / max(1, steps_last)
    out = {
        "metric": METRIC,
        "value": tokens / elapsed,
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
            "global_batch": run.n_requests,
            "seq_len": run.max_prefix + run.n_canvases * C,
            "canvas": C,
            "prefix": run.max_prefix,
            "denoise_steps_per_canvas": steps_last / run.n_canvases,
            "parallelism": "single GPU",
        },
        "ms_per_denoise_step": step_ms,
        "decode_tokens_per_s": C * run.n_canvases / (denoise_ms * 1e-3) if denoise_ms else None,
        "roofline": roofline(dominant, cfg, C, keys, ms_k / max(1, n_k)),
        "denoise_step_kernels_ms": {k: round(v[0] / max(1, steps_last), 4) for k, v in
                                    sorted(per_kernel.items(), key=lambda kv: -kv[1][0])},
    }
    for name, (ms, n) in per_kernel.items():
        r = roofline(name, cfg, C, keys, ms / max(1, n))
        if r:
            out.setdefault("kernel_rooflines", {})[name] = {k: r[k] for k in ("bound", "frac", "hbm_gbs",
                                                                              "mfma_util_pct", "avg_launch_ms")}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        del model
        out["cpu_baseline"] = cpu_baseline(run, w_cpu, prefix_cpu)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
