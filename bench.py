"""Benchmark of the block-diffusion hot path on one MI355X.

One bench step is one whole request through the library: causal prefill of
the prompt, then per canvas the denoising steps (each a bidirectional forward
+ LM head + fused vocab reduction, then the confidence-ranked commit) and the
append of the finished canvas to the KV cache.  `value` is committed tokens per
second over the K timed steps, inputs already resident in HBM.

Default workload: the dense 16-layer d=2048 bf16 model (16 Q / 4 KV heads x
128, SwiGLU 8192, vocab 32768) with a 1024-token prefix and one 256-token
canvas, 16 steps x 16 commits, then the append.  Weights and prompt are seeded
synthetic draws (random init), generated on the host so the CPU baseline reads
the same bytes.

Also reported: ms per denoising step (denoise + commit, CUDA events on the
library's stream), the dominant kernel's roofline from the library's own HIP
event timing over the timed region, and the CPU oracle timed on a bounded
sample of the same workload.
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
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0


def _workload_text(run) -> str:
    m = run.model
    ffn = (f"SwiGLU {m.d_ffn}" if m.ffn == "dense" else
           f"{m.n_experts} experts top-{m.top_k} x {m.d_expert} + shared {m.d_ffn}")
    rule = (f"{run.n_steps} steps top-k" if run.rule == "topk" else
            f"<= {run.n_steps} steps, confidence >= {run.threshold}")
    return (f"{m.name}: {m.n_layers}L d={m.d_model} {m.n_q_heads}q/{m.n_kv_heads}kv x {m.head_dim}, {ffn}, "
            f"vocab {m.vocab}; prefix {run.prefix_len[1]}, {run.n_canvases} x {run.canvas}-token canvas, "
            f"{rule}, append")


def gemm_roofline(cfg, C: int, avg_ms: float, kernel: str):
    """Algorithmic bytes / flops of one launch of the dominant GEMM at M = C rows."""
    d, F = cfg.d_model, cfg.d_ffn
    eb = 1 if cfg.dtype == "fp8" else 2
    if kernel == "gemm_gate_up":        # SwiGLU: A [C, d], gate and up [F, d], out bf16 [C, F]
        wbytes = 2 * F * d * eb
        abytes = C * d * eb
        obytes = C * F * 2
        flops = 2.0 * C * (2 * F) * d
    else:
        raise ValueError(kernel)
    total = wbytes + abytes + obytes
    s = avg_ms * 1e-3
    return {
        "kernel": f"{kernel} (M={C}, N=2x{F}, K={d}, {cfg.dtype})",
        "bound": "hbm",
        "achieved": total / s / 1e9,
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": total / s / 1e9 / HBM_PEAK_GBS,
        "traffic": None,
        "bytes_per_launch": total,
        "flops_per_launch": flops,
        "avg_launch_ms": avg_ms,
        "mfma_util_pct": 100.0 * flops / s / 1e12 / (FP8_PEAK_TFLOPS if cfg.dtype == "fp8" else BF16_PEAK_TFLOPS),
    }


def cpu_baseline(run, weights_cpu, prefix_cpu):
    """The oracle on the host, on a bounded sample of the same workload: prefill
    of the full prompt, one denoising step with its commit, and the append;
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
    per_req = (t1 - t0) + run.n_steps * (t2 - t1) + (t3 - t2)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {
        "value": run.canvas * run.n_canvases / per_req if run.n_canvases == 1 else
        run.canvas * run.n_canvases / ((t1 - t0) + run.n_canvases * (run.n_steps * (t2 - t1) + (t3 - t2))),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"float64 numpy oracle on the host: prefill of the {len(prefix_cpu)}-token prompt "
                   f"({t1 - t0:.2f} s), one denoising step + commit ({t2 - t1:.2f} s) and one append "
                   f"({t3 - t2:.2f} s) of the same workload and weights; the request is extrapolated to "
                   f"{run.n_steps} steps per canvas"),
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
    timed_kernel = "gemm_gate_up"

    def one_request(timing: bool):
        seq.raw.T = 0
        model.dlm_prefill(seq, prefix, ws)
        steps_run = 0
        for ci in range(run.n_canvases):
            seq.canvas.fill_(cfg.mask_id)
            if timing:
                model.timing_enable([abi.DLM_K_GEMM_GATE_UP])
            ev[2 * ci].record()
            for s in range(run.n_steps):
                model.dlm_denoise_step([seq], conf, pred, ws)
                model.dlm_commit([seq], conf, pred, rule, s, None, n_masked)
                steps_run += 1
                if run.rule == "threshold" and int(n_masked.cpu()[0]) == 0:
                    break
            ev[2 * ci + 1].record()
            if timing:
                model.timing_enable([])
            model.dlm_append_canvas([seq], ws)
        return steps_run

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        one_request(False)
    torch.cuda.synchronize()
    model.timing_read()
    denoise_ms, n_denoise = 0.0, 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        n_denoise += one_request(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # per-canvas denoise loop times of the last timed request, then all requests' kernel timing
    kt = model.timing_read()
    for ci in range(run.n_canvases):
        denoise_ms += ev[2 * ci].elapsed_time(ev[2 * ci + 1])
    status = model.dlm_check_device_status()
    if status:
        print(f"[bench] device error word {status}", file=sys.stderr)
        sys.exit(1)
    elapsed = t1 - t0
    tokens = args.steps * C * run.n_canvases
    steps_last = n_denoise // args.steps
    ms_k, n_k = kt.get(timed_kernel, (0.0, 0))
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
        "dtype": "bf16" if cfg.dtype == "bf16" else cfg.dtype,
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
        "ms_per_denoise_step": denoise_ms / max(1, steps_last),
        "decode_tokens_per_s": C * run.n_canvases / (denoise_ms * 1e-3) if denoise_ms else None,
        "roofline": gemm_roofline(cfg, C, ms_k / max(1, n_k), timed_kernel) if n_k else None,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        del model
        out["cpu_baseline"] = cpu_baseline(run, w_cpu, prefix_cpu)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
