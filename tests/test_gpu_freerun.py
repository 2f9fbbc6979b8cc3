"""Free-running generation: the product loop `generate()` (direct calls and
HIP-graph replays) on its own prefill, its own steps and its own appends,
against the oracle's `sampler.generate` on the same prompts -- the reverse
process with block appends end to end ("Diffusion LLMs: what changes when you
stop generating one token at a time", section 2 and section 4.2 "Block
decoding").

Nothing is fed from the oracle to the GPU.  While the two runs hold the same
canvases, every step is compared like a lockstep step (tests/parity.py):
logits within the dtype's tolerance, commits and tokens bit-exact outside the
oracle's decision bands.  The first step of each canvas exercises the GPU's
own prefill (first canvas) or its own append of the previous canvas.  A
commit that differs inside a band is a legitimate divergence: from then on
the runs hold different canvases, and only the properties that hold for any
run are checked (the commit kernel applies the rule to the GPU's own
confidences, only [MASK] positions change, the schedule's counts).  The step
at which each run diverges is reported."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from oracle import sampler as osampler
from oracle.model import OracleModel, OracleWeights
from tests.parity import StepReport, compare_commit, compare_logits, router_exemptions, step_bands
from tests.progress import progress

pytestmark = pytest.mark.gpu

CASES = [("tiny", False), ("tiny", True), ("dense-mini-ragged", True), ("moe-mini", False),
         ("moe-mini-batch", True), ("dense-mini-fp8", False), ("moe-mini-mxfp4", True), ("moe-mini-mxfp6", False),
         ("dense-full", True)]


def _run(name):
    if name == "dense-full":
        return replace(synth.get_run("dense"), n_canvases=2)       # 16 steps, then a second canvas after the append
    return synth.get_run(name)


@pytest.mark.parametrize("name,graphs", CASES)
def test_free_run_against_oracle_generate(name, graphs):
    from masked_block_diffusion_amd import DLM, Rule, generate
    run = _run(name)
    cfg, C, n = run.model, run.canvas, run.n_requests
    print(f"[freerun] run={name} graphs={graphs} dtype={cfg.dtype} L={cfg.n_layers} C={C} requests={n} "
          f"canvases={run.n_canvases}", flush=True)
    w = synth.make_weights(cfg, seed=run.seed)
    om = OracleModel(cfg, OracleWeights(cfg, w))
    gm = DLM(cfg, {k: v.cuda() for k, v in w.items()}, canvas=C)
    del w
    prefixes = synth.make_inputs(run)
    cap = run.capacity()

    # the oracle's runs, one per request (requests never interact); per step
    # the bands come from the exact and a perturbed denoise of the same state
    oracle = []
    for r in range(n):
        steps = []

        def on_step(ci, s, before, conf, pred, after, st, dbg):
            # the full-size dense model's bands from one perturbation (its
            # bf16 moves scatter little between noise streams), the others' from three
            steps.append((ci, s, before.copy(), conf, pred, after.copy(), dbg,
                          step_bands(om, st, before, (conf, pred, dbg), seed=1000 * ci + 10 * s,
                                     n=1 if name == "dense-full" else 3)))
            progress(f"[freerun] {name}: oracle request {r} canvas {ci} step {s}")
        osampler.generate(om, run, prefixes[r].numpy(), capacity=cap, on_step=on_step, with_state=True)
        oracle.append(steps)

    # the product loop, capturing what each step produced
    seqs = [gm.new_seq(cap) for _ in range(n)]
    ws = gm.workspace(max(n * C, max(len(p) for p in prefixes)), cap)
    logits = torch.empty(n * C * cfg.vocab, dtype=torch.float32, device="cuda")
    moe = cfg.ffn == "moe"
    rows = max(n * C, max(len(p) for p in prefixes))
    rdbg = torch.empty(cfg.n_layers * rows * max(cfg.top_k, 1), dtype=torch.int32, device="cuda") if moe else None
    rlog = torch.empty(cfg.n_layers * rows * max(cfg.n_experts, 1), dtype=torch.float32, device="cuda") if moe else None
    gm.dlm_debug_router(rdbg, rlog, cfg.n_layers * rows)
    gpu = []

    def g_step(ci, s, conf, pred):
        g = {"at": (ci, s), "conf": conf.view(n, C).cpu().numpy().astype(np.float64),
             "pred": pred.view(n, C).cpu().numpy(), "canvas": np.stack([q.canvas.cpu().numpy() for q in seqs]),
             "logits": logits.view(n, C, cfg.vocab).cpu().numpy()}
        if moe:
            g["rsets"] = rdbg[:cfg.n_layers * n * C * cfg.top_k].view(cfg.n_layers, n, C, cfg.top_k).cpu().numpy()
            g["rlog"] = rlog[:cfg.n_layers * n * C * cfg.n_experts].view(
                cfg.n_layers, n, C, cfg.n_experts).cpu().numpy().astype(np.float64)
        gpu.append(g)
    rule = Rule.for_run(run)
    generate(gm, seqs, [p.cuda() for p in prefixes], rule, run.n_canvases, ws, on_step=g_step,
             graphs={} if graphs else None, logits=logits)
    torch.cuda.synchronize()
    assert gm.dlm_check_device_status() == 0

    sched = osampler.topk_schedule(C, run.n_steps)
    tot = StepReport()
    for r in range(n):
        diverged = None
        o_steps = {(ci, s): rest for (ci, s, *rest) in oracle[r]}
        before = None
        for g in gpu:                       # the GPU's steps in order (all requests step together)
            ci, s = g["at"]
            if s == 0:
                before = np.full(C, cfg.mask_id, dtype=np.int32)
            after = g["canvas"][r]
            # properties of any run: the commit kernel is the rule applied to
            # the GPU's own confidences, and only [MASK] positions change
            want, _ = osampler.commit(before, g["conf"][r], g["pred"][r], cfg.mask_id, run, s)
            assert np.array_equal(want, after), f"run {name} request {r}: commit kernel differs at {ci}/{s}"
            if diverged is None:
                o_before, conf_o, pred_o, o_after, dbg, bands = o_steps[(ci, s)]
                assert np.array_equal(o_before, before)
                rep = StepReport()
                ex = router_exemptions(g["rsets"][:, r] if moe else None, g["rlog"][:, r] if moe else None, dbg,
                                       bands, cfg.dtype, rep)
                compare_logits(g["logits"][r], dbg.logits, cfg.mask_id, cfg.dtype, rep, ex, bands)
                compare_commit(before, after, o_after, conf_o, dbg.logits, cfg.mask_id, run.rule, sched[s],
                               run.threshold, run.rule == "threshold" and s == run.n_steps - 1, rep, bands, ex,
                               gpu_conf=g["conf"][r])
                assert not rep.problems, f"run {name} request {r} canvas {ci} step {s}: {rep.problems}"
                tot.add(rep)
                if not np.array_equal(after, o_after):
                    diverged = (ci, s)
            before = after
        if diverged is None:
            assert len(o_steps) == len(gpu), "both runs take the same number of steps"
            progress(f"[freerun] run={name} request {r}: identical to the oracle over all {len(gpu)} steps "
                  f"of {run.n_canvases} canvas(es)")
        else:
            progress(f"[freerun] run={name} request {r}: diverged legitimately at canvas {diverged[0]} step "
                  f"{diverged[1]} (a commit inside the oracle's band)")
    progress(f"[freerun] run={name} {tot.summary()}")
    gm.close()
