"""Error paths of the C ABI on a live model: every host-detected error returns
its status, enqueues nothing and changes no state (T, canvas, KV cache,
outputs); device-detected faults set the model's error word, which
dlm_check_device_status reports once and clears.

Also the promise AR decoding relies on: the K/V a denoising step writes into
slots [T, T + C) are bit-identical to what dlm_append_canvas writes for the
same canvas, so a caller may advance T by C instead of appending
(include/dlm.h, dlm_denoise_step)."""
import ctypes

import pytest
import torch

import synth
from masked_block_diffusion_amd import abi

pytestmark = pytest.mark.gpu


def _model(name="tiny"):
    from masked_block_diffusion_amd import DLM
    run = synth.get_run(name)
    cfg = run.model
    gm = DLM(cfg, {k: v.cuda() for k, v in synth.make_weights(cfg, seed=run.seed).items()}, canvas=run.canvas)
    return run, cfg, gm


def _snapshot(seq):
    return seq.raw.T, seq.canvas.clone(), seq.kv.clone()


def _unchanged(seq, snap):
    torch.cuda.synchronize()
    T, canvas, kv = snap
    assert seq.raw.T == T
    assert torch.equal(seq.canvas, canvas)
    assert torch.equal(seq.kv, kv)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def test_capacity_errors_have_no_side_effects():
    run, cfg, gm = _model()
    lib = gm.lib
    seq = gm.new_seq(128)                         # 64-token prompt + room for 64 more
    seq.kv.zero_()                                # slots [64, 96) are read below without being written
    ids = synth.make_inputs(run)[0].cuda()
    ws = gm.workspace(256, 256)
    gm.dlm_prefill(seq, ids, ws)
    torch.cuda.synchronize()
    assert seq.raw.T == 64
    snap = _snapshot(seq)
    long_ids = torch.zeros(65, dtype=torch.int32, device="cuda")
    st = lib.dlm_prefill(gm.handle, ctypes.byref(seq.raw), long_ids.data_ptr(), 65, ws.data_ptr(), ws.numel(),
                         _stream())
    assert st == abi.DLM_E_CAPACITY and b"exceeds capacity" in lib.dlm_last_error()
    _unchanged(seq, snap)
    # denoise and append of a 32-token canvas need T + 32 <= 128
    seq.raw.T = 97
    snap = _snapshot(seq)
    conf = torch.full((run.canvas,), -7.0, device="cuda")
    pred = torch.full((run.canvas,), -7, dtype=torch.int32, device="cuda")
    arr = gm._seq_array([seq])
    st = lib.dlm_denoise_step(gm.handle, arr, 1, conf.data_ptr(), pred.data_ptr(), None, ws.data_ptr(), ws.numel(),
                              _stream())
    assert st == abi.DLM_E_CAPACITY
    st = lib.dlm_append_canvas(gm.handle, arr, 1, ws.data_ptr(), ws.numel(), _stream())
    assert st == abi.DLM_E_CAPACITY
    _unchanged(seq, snap)
    assert bool((conf == -7.0).all()) and bool((pred == -7).all())
    seq.raw.T = 96                                # exactly full: allowed
    gm.dlm_denoise_step([seq], conf, pred, ws)
    torch.cuda.synchronize()
    assert gm.dlm_check_device_status() == 0
    gm.close()


def test_workspace_errors_on_every_model_call():
    run, cfg, gm = _model()
    lib = gm.lib
    seq = gm.new_seq(run.capacity())
    ids = synth.make_inputs(run)[0].cuda()
    need_prefill = gm.workspace_bytes(len(ids), run.capacity())
    need_step = gm.workspace_bytes(run.canvas, run.capacity())
    ws = torch.empty(max(need_prefill, need_step), dtype=torch.uint8, device="cuda")
    snap = _snapshot(seq)
    for wsp, nbytes in ((ws.data_ptr(), need_prefill - 1), (None, need_prefill)):
        st = lib.dlm_prefill(gm.handle, ctypes.byref(seq.raw), ids.data_ptr(), len(ids), wsp, nbytes, _stream())
        assert st == abi.DLM_E_WORKSPACE, st
    _unchanged(seq, snap)
    gm.dlm_prefill(seq, ids, ws)
    torch.cuda.synchronize()
    snap = _snapshot(seq)
    conf = torch.full((run.canvas,), -7.0, device="cuda")
    pred = torch.full((run.canvas,), -7, dtype=torch.int32, device="cuda")
    arr = gm._seq_array([seq])
    for wsp, nbytes in ((ws.data_ptr(), need_step - 1), (None, need_step)):
        st = lib.dlm_denoise_step(gm.handle, arr, 1, conf.data_ptr(), pred.data_ptr(), None, wsp, nbytes, _stream())
        assert st == abi.DLM_E_WORKSPACE
        st = lib.dlm_append_canvas(gm.handle, arr, 1, wsp, nbytes, _stream())
        assert st == abi.DLM_E_WORKSPACE
    _unchanged(seq, snap)
    assert bool((conf == -7.0).all()) and bool((pred == -7).all())
    gm.close()


def test_commit_argument_errors_have_no_side_effects():
    from masked_block_diffusion_amd import Rule
    run, cfg, gm = _model()
    lib = gm.lib
    seq = gm.new_seq(run.capacity())
    ws = gm.workspace(max(run.canvas, 64), run.capacity())
    gm.dlm_prefill(seq, synth.make_inputs(run)[0].cuda(), ws)
    conf = torch.empty(run.canvas, device="cuda")
    pred = torch.empty(run.canvas, dtype=torch.int32, device="cuda")
    gm.dlm_denoise_step([seq], conf, pred, ws)
    torch.cuda.synchronize()
    snap = _snapshot(seq)
    ncom = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    nmask = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    arr = gm._seq_array([seq])
    rule = Rule.for_run(run)

    def commit(r, step):
        return lib.dlm_commit(gm.handle, arr, 1, conf.data_ptr(), pred.data_ptr(), ctypes.byref(r.raw), step,
                              ncom.data_ptr(), nmask.data_ptr(), _stream())
    assert commit(rule, -1) == abi.DLM_E_ARG
    assert commit(rule, rule.n_steps) == abi.DLM_E_ARG and b"outside" in lib.dlm_last_error()
    bad_k = Rule("topk", rule.n_steps, [-1] * rule.n_steps)
    assert commit(bad_k, 0) == abi.DLM_E_ARG
    for tau in (-0.5, float("nan"), float("inf")):
        assert commit(Rule.topk(run.canvas, run.n_steps, edit_threshold=tau), 0) == abi.DLM_E_ARG
    assert commit(Rule.threshold(4, -1.0), 0) == abi.DLM_E_ARG
    bad_kind = Rule.topk(run.canvas, run.n_steps)
    bad_kind.raw.kind = 7
    assert commit(bad_kind, 0) == abi.DLM_E_ARG
    _unchanged(seq, snap)
    assert int(ncom[0]) == -7 and int(nmask[0]) == -7
    assert commit(rule, rule.n_steps - 1) == abi.DLM_OK
    gm.close()


@pytest.mark.parametrize("where", ["prefill", "denoise"])
def test_token_range_sets_device_error_bit(where):
    run, cfg, gm = _model()
    seq = gm.new_seq(run.capacity())
    ws = gm.workspace(max(run.canvas, 64), run.capacity())
    ids = synth.make_inputs(run)[0].cuda()
    conf = torch.empty(run.canvas, device="cuda")
    pred = torch.empty(run.canvas, dtype=torch.int32, device="cuda")
    if where == "prefill":
        ids[5] = cfg.vocab                        # one past the vocabulary
        gm.dlm_prefill(seq, ids, ws)              # accepted on the host: only the device sees ids
    else:
        gm.dlm_prefill(seq, ids, ws)
        assert gm.dlm_check_device_status() == 0
        seq.canvas[3] = -5
        gm.dlm_denoise_step([seq], conf, pred, ws)
    bits = ctypes.c_int32(0)
    st = gm.lib.dlm_check_device_status(gm.handle, _stream(), ctypes.byref(bits))
    assert st == abi.DLM_E_DEVICE and bits.value == abi.DLM_DEVERR_TOKEN_RANGE
    assert gm.dlm_check_device_status() == 0     # read once, then cleared
    gm.close()


def test_mask_in_append_sets_device_error_bit():
    run, cfg, gm = _model()
    seq = gm.new_seq(run.capacity())
    ws = gm.workspace(max(run.canvas, 64), run.capacity())
    gm.dlm_prefill(seq, synth.make_inputs(run)[0].cuda(), ws)
    seq.canvas.fill_(1)
    seq.canvas[7] = cfg.mask_id
    gm.dlm_append_canvas([seq], ws)
    assert gm.dlm_check_device_status() == abi.DLM_DEVERR_MASK_APPEND
    assert gm.dlm_check_device_status() == 0
    gm.close()


def test_router_debug_capacity_is_checked_before_enqueueing():
    run, cfg, gm = _model("moe-mini")
    lib = gm.lib
    seq = gm.new_seq(run.capacity())
    ws = gm.workspace(max(run.canvas, 128), run.capacity())
    gm.dlm_prefill(seq, synth.make_inputs(run)[0].cuda(), ws)
    torch.cuda.synchronize()
    ids = torch.full((cfg.n_layers * run.canvas * cfg.top_k,), -7, dtype=torch.int32, device="cuda")
    gm.dlm_debug_router(ids, None, cfg.n_layers * run.canvas - 1)     # one (layer, row) short
    snap = _snapshot(seq)
    conf = torch.empty(run.canvas, device="cuda")
    pred = torch.empty(run.canvas, dtype=torch.int32, device="cuda")
    st = lib.dlm_denoise_step(gm.handle, gm._seq_array([seq]), 1, conf.data_ptr(), pred.data_ptr(), None,
                              ws.data_ptr(), ws.numel(), _stream())
    assert st == abi.DLM_E_CAPACITY
    _unchanged(seq, snap)
    assert bool((ids == -7).all())
    gm.dlm_debug_router(ids, None, cfg.n_layers * run.canvas)
    gm.dlm_denoise_step([seq], conf, pred, ws)
    torch.cuda.synchronize()
    assert bool((ids >= 0).all() and (ids < cfg.n_experts).all())
    gm.close()


@pytest.mark.parametrize("name", ["tiny", "dense-mini-ragged", "moe-mini", "dense-mini-fp8"])
def test_denoise_kv_slots_equal_append(name):
    """The scratch K/V of a denoising step are the append's K/V for the same
    canvas, bit for bit (same kernels, same inputs, same block mask)."""
    run, cfg, gm = _model(name)
    C = run.canvas
    a, b = gm.new_seq(run.capacity()), gm.new_seq(run.capacity())
    ws = gm.workspace(max(C, run.max_prefix), run.capacity())
    ids = synth.make_inputs(run)[0].cuda()
    conf = torch.empty(C, device="cuda")
    pred = torch.empty(C, dtype=torch.int32, device="cuda")
    gen = torch.Generator(device="cpu").manual_seed(3)
    canvas = torch.randint(0, cfg.vocab - 1, (C,), generator=gen, dtype=torch.int32).cuda()
    for s in (a, b):
        gm.dlm_prefill(s, ids, ws)
        s.canvas.copy_(canvas)
    T = a.raw.T
    gm.dlm_denoise_step([a], conf, pred, ws)
    gm.dlm_append_canvas([b], ws)
    torch.cuda.synchronize()
    ka, va = a.read_kv()
    kb, vb = b.read_kv()
    assert torch.equal(ka[:, :, :T + C], kb[:, :, :T + C])
    assert torch.equal(va[:, :, :T + C], vb[:, :, :T + C])
    assert b.raw.T == T + C and a.raw.T == T
    gm.close()
