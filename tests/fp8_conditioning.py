"""Conditioning of the fp8 model's logits under fp32-level arithmetic noise.

A measurement script (CPU only, oracle only; not collected by pytest):

    python tests/fp8_conditioning.py [dense|moe] [n_layers] [canvas]

It prefills a full-width workload cut to `n_layers` layers (dense: d=2048,
vocab 32768, 1024-token prompt; moe: d=2560, 128 experts, vocab 262144,
4096-token prompt) in E4M3, then runs the first denoising
step of the all-[MASK] canvas once exactly and once with every fp8 GEMM input
multiplied by (1 + eps * N(0, 1)) per element -- the relative error an fp32
dot product of a few thousand terms carries -- and prints, per eps, how many
canvas rows move by more than 0.01 and the largest move, next to the logit
tolerance 6e-2 * max|logit|.  The prefill is kept exact, as in the lockstep
parity tests, where the GPU starts each step from the oracle's cache.

Measured, 256-row canvas:
  dense, 1 layer (tolerance 0.252): eps 1e-7 moves no row by more than 0.01;
    eps 1e-6 moves 11 rows, the largest by 0.117; eps 1e-5 moves 149 rows,
    the largest by 0.158.
  moe, 2 layers (tolerance 0.331): eps 1e-7 already moves 222 rows, the
    largest by 0.293; eps 1e-6 moves every row (0.311); eps 1e-5 puts 16 rows
    beyond the tolerance (0.453).
The moves come from the per-token E4M3 quantisation: a code decided on a
near-tie flips, the flip shifts the next GEMM's output a little everywhere
(the SwiGLU intermediate, then its own 8192-element quantisation), and in a
second layer the flipped canvas rows reach every other row through
attention.  fp32 arithmetic cannot hold the logits of the two-layer fp8 MoE to
6e-2 * max|logit| of a float64 reference: the reference itself moves that far
under fp32-sized noise.
"""
import copy
import sys
from dataclasses import replace

import numpy as np

if __name__ == "__main__":
    sys.path.insert(0, __file__.rsplit("/tests/", 1)[0])
    import synth
    from oracle.model import OracleModel, OracleWeights

    workload = sys.argv[1] if len(sys.argv) > 1 else "dense"
    n_layers = int(sys.argv[2]) if len(sys.argv) > 2 else 1
    canvas = int(sys.argv[3]) if len(sys.argv) > 3 else 256
    run = synth.get_run(workload)
    run = replace(run, model=replace(run.model, n_layers=n_layers, dtype="fp8"), n_canvases=1, canvas=canvas)
    cfg, C = run.model, run.canvas
    W = OracleWeights(cfg, synth.make_weights(cfg, seed=run.seed))
    om = OracleModel(cfg, W)
    st0 = om.new_seq(run.capacity())
    om.prefill(st0, synth.make_inputs(run)[0].numpy())
    exact_linear = OracleModel.linear
    rng = np.random.default_rng(1)

    def step(eps):
        def noisy(self, x, name, w=None, s_out=None):
            if eps:
                x = x * (1.0 + eps * rng.standard_normal(x.shape))
            return exact_linear(self, x, name, w, s_out)
        OracleModel.linear = noisy
        try:
            _, _, dbg = om.denoise(copy.deepcopy(st0), np.full(C, cfg.mask_id, dtype=np.int32), debug=True)
        finally:
            OracleModel.linear = exact_linear
        lg = dbg.logits
        lg[:, cfg.mask_id] = 0.0
        return lg

    ref = step(0.0)
    tol = 6e-2 * np.abs(ref).max()
    print(f"{workload}, {n_layers} layer(s), canvas {C}: max|logit| {np.abs(ref).max():.3f}, tolerance {tol:.3f}")
    for eps in (1e-7, 1e-6, 1e-5):
        row = np.abs(step(eps) - ref).max(axis=1)
        print(f"eps {eps:g}: rows moved > 0.01: {int((row > 0.01).sum())}, largest move {row.max():.4f}, "
              f"rows beyond tolerance: {int((row > tol).sum())}")
