"""Pins for the oracle's transformer pieces and its KV-cache bookkeeping.

Each check is independent of the function it pins: library routines on the CPU,
hand-computed values, brute force on tiny inputs, or invariants the pages fix
(causal prefill, bidirectional canvas, finished canvases cached).
"""
from dataclasses import replace

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import softmax as sp_softmax

import synth
from oracle.model import (OracleModel, OracleWeights, attention, block_mask, causal_mask,
                          rms_norm, rope, silu, softmax)
from oracle.numerics import round_bf16

RNG = np.random.default_rng(1234)


# ------------------------------------------------------------- primitives --

def test_rms_norm_matches_torch():
    x = RNG.standard_normal((7, 48))
    g = RNG.standard_normal(48)
    for eps in (1e-6, 0.5):      # a large eps makes a dropped eps visible
        want = F.rms_norm(torch.from_numpy(x), (48,), torch.from_numpy(g), eps=eps).numpy()
        np.testing.assert_allclose(rms_norm(x, g, eps), want, rtol=1e-12, atol=1e-14)


def test_softmax_matches_scipy_and_masks():
    s = RNG.standard_normal((4, 9)) * 10
    np.testing.assert_allclose(softmax(s), sp_softmax(s, axis=-1), rtol=1e-12)
    s[:, 3] = -np.inf
    p = softmax(s)
    assert np.all(p[:, 3] == 0)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-13)


def test_silu_closed_form():
    z = np.array([0.0, 1.0, -2.0, 30.0])
    np.testing.assert_allclose(silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-14)
    assert silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(silu(np.array([1.0])), 1 / (1 + np.exp(-1)), rtol=1e-15)


def _attn_brute(q, k, v, allowed):
    hq, n, dh = q.shape
    group = hq // k.shape[0]
    out = np.zeros_like(q)
    for h in range(hq):
        kh = h // group
        for i in range(n):
            scores = [np.dot(q[h, i], k[kh, j]) / np.sqrt(dh) if allowed[i, j] else None
                      for j in range(k.shape[1])]
            m = max(sc for sc in scores if sc is not None)
            w = [np.exp(sc - m) if sc is not None else 0.0 for sc in scores]
            z = sum(w)
            for j in range(k.shape[1]):
                out[h, i] += w[j] / z * v[kh, j]
    return out


@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2), (6, 2), (5, 1)])
def test_attention_brute_force(hq, hkv):
    n, m, dh = 5, 9, 8
    q = RNG.standard_normal((hq, n, dh))
    k = RNG.standard_normal((hkv, m, dh))
    v = RNG.standard_normal((hkv, m, dh))
    allowed = RNG.random((n, m)) < 0.6
    allowed[:, 0] = True
    np.testing.assert_allclose(attention(q, k, v, allowed), _attn_brute(q, k, v, allowed),
                               rtol=1e-12, atol=1e-13)


def test_attention_matches_sdpa_gqa_as_repeated_mha():
    hq, hkv, n, m, dh = 8, 2, 6, 11, 16
    q = RNG.standard_normal((hq, n, dh))
    k = RNG.standard_normal((hkv, m, dh))
    v = RNG.standard_normal((hkv, m, dh))
    pos = np.arange(m - n, m)
    allowed = causal_mask(pos, m)
    # GQA == MHA with each KV head repeated for its group of consecutive Q heads
    kr = np.repeat(k, hq // hkv, axis=0)
    vr = np.repeat(v, hq // hkv, axis=0)
    want = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(kr),
                                          torch.from_numpy(vr),
                                          attn_mask=torch.from_numpy(allowed)).numpy()
    np.testing.assert_allclose(attention(q, k, v, allowed), want, rtol=1e-11, atol=1e-12)


def test_attention_single_key_returns_value():
    q = RNG.standard_normal((3, 4, 8))
    k = RNG.standard_normal((3, 1, 8))
    v = RNG.standard_normal((3, 1, 8))
    out = attention(q, k, v, np.ones((4, 1), bool))
    np.testing.assert_allclose(out, np.broadcast_to(v, out.shape), rtol=1e-14)


def test_masks():
    cm = causal_mask(np.array([3, 4]), 6)
    assert cm.tolist() == [[True] * 4 + [False] * 2, [True] * 5 + [False]]
    assert block_mask(2, 5).all()


def test_rope_hand_values_rotate_half():
    base = 10000.0
    # dh=4: pairs (0,2) at theta_0 = 1 and (1,3) at theta_1 = base^-1/2
    v = np.array([[[1.0, 0.0, 0.0, 0.0]], [[0.0, 1.0, 0.0, 0.0]]])
    out = rope(v, np.array([1, 1]), base)
    np.testing.assert_allclose(out[0, 0], [np.cos(1), 0, np.sin(1), 0], atol=1e-15)
    t1 = base ** -0.5
    np.testing.assert_allclose(out[1, 0], [0, np.cos(t1), 0, np.sin(t1)], atol=1e-15)
    # position 0 is the identity
    w = RNG.standard_normal((3, 2, 8))
    np.testing.assert_array_equal(rope(w, np.zeros(3, int), base), w)


def test_rope_dh2_is_complex_rotation():
    v = RNG.standard_normal((6, 3, 2))
    pos = np.arange(6) * 7
    z = (v[..., 0] + 1j * v[..., 1]) * np.exp(1j * pos[:, None])
    out = rope(v, pos, 10000.0)
    np.testing.assert_allclose(out[..., 0], z.real, atol=1e-12)
    np.testing.assert_allclose(out[..., 1], z.imag, atol=1e-12)


def test_rope_norm_and_relative_position():
    q = RNG.standard_normal((1, 2, 64))
    k = RNG.standard_normal((1, 2, 64))
    for p in (0, 5, 1000):
        np.testing.assert_allclose(np.linalg.norm(rope(q, np.array([p]), 1e4)),
                                   np.linalg.norm(q), rtol=1e-13)
    def score(pq, pk):
        return np.sum(rope(q, np.array([pq]), 1e4) * rope(k, np.array([pk]), 1e4), axis=-1)
    np.testing.assert_allclose(score(10, 3), score(110, 103), rtol=1e-9)
    assert not np.allclose(score(10, 3), score(10, 4))


# ------------------------------------------------------------------ model --

def _tiny_cfg(**kw):
    base = synth.configs.ModelConfig(
        name="t", n_layers=2, d_model=32, n_q_heads=4, n_kv_heads=2, head_dim=8,
        vocab=50, mask_id=49, ffn="dense", d_ffn=24, dtype="f32")
    return replace(base, **kw)


def _model(cfg, seed=0):
    return OracleModel(cfg, OracleWeights(cfg, synth.make_weights(cfg, seed=seed)))


def test_linear_orientation_hand_value():
    cfg = _tiny_cfg()
    m = _model(cfg)
    w = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])   # [out=3, in=2]
    y = m.linear(np.array([[1.0, 0.0]]), "x", w=w)
    np.testing.assert_array_equal(y, [[1.0, 3.0, 5.0]])


def test_linear_fp8_formula():
    cfg = _tiny_cfg(dtype="fp8")
    m = _model(cfg)
    w = np.array([[1.0, -2.0], [0.5, 4.0]])               # exact E4M3 values
    s_o = np.array([0.25, 2.0])
    x = np.array([[448.0, 224.0], [0.0, 0.0]])              # row 0 amax 448 -> scale 1
    y = m.linear(x, "x", w=w, s_out=s_o)
    np.testing.assert_array_equal(y[0], [(448 - 448) * 0.25, (224 + 896) * 2.0])
    np.testing.assert_array_equal(y[1], [0.0, 0.0])


def test_swiglu_hand_value():
    cfg = _tiny_cfg()
    m = _model(cfg)
    m.W.w.update({"g": np.array([[1.0, 0.0]]), "u": np.array([[0.0, 2.0]]),
                  "d": np.array([[3.0], [-1.0]])})
    h = np.array([[1.0, 5.0]])
    s1 = 1.0 / (1.0 + np.exp(-1.0))
    np.testing.assert_allclose(m.swiglu(h, "g", "u", "d"), [[3 * s1 * 10, -s1 * 10]], rtol=1e-14)


def _moe_cfg(**kw):
    base = dict(ffn="moe", d_ffn=16, n_experts=4, top_k=2, d_expert=12)
    base.update(kw)
    return _tiny_cfg(**base)


def test_moe_topk_equals_all_is_dense_weighted_sum():
    cfg = _moe_cfg(top_k=4)
    m = _model(cfg)
    h = RNG.standard_normal((6, cfg.d_model))
    r = h @ m.W["0.w_router"].T
    p = sp_softmax(r, axis=-1)
    want = m.swiglu(h, "0.w_gate", "0.w_up", "0.w_down")
    for e in range(cfg.n_experts):
        want += p[:, e:e + 1] * m.swiglu(h, "0.we_gate", "0.we_up", "0.we_down", e=e)
    np.testing.assert_allclose(m.moe(h, 0), want, rtol=1e-12, atol=1e-14)


def test_moe_top1_renormalised_weight_is_one():
    cfg = _moe_cfg(top_k=1)
    m = _model(cfg)
    h = RNG.standard_normal((5, cfg.d_model))
    best = np.argmax(h @ m.W["0.w_router"].T, axis=-1)
    want = m.swiglu(h, "0.w_gate", "0.w_up", "0.w_down")
    for i, e in enumerate(best):
        want[i] += m.swiglu(h[i:i + 1], "0.we_gate", "0.we_up", "0.we_down", e=e)[0]
    np.testing.assert_allclose(m.moe(h, 0), want, rtol=1e-12, atol=1e-14)


def test_moe_single_expert_no_shared_is_dense_swiglu():
    cfg = _moe_cfg(n_experts=1, top_k=1)
    m = _model(cfg)
    m.W.w["0.w_down"] = np.zeros_like(m.W["0.w_down"])       # no shared expert
    h = RNG.standard_normal((4, cfg.d_model))
    want = m.swiglu(h, "0.we_gate", "0.we_up", "0.we_down", e=0)
    dense = silu(h @ m.W["0.we_gate"][0].T) * (h @ m.W["0.we_up"][0].T) @ m.W["0.we_down"][0].T
    np.testing.assert_allclose(m.moe(h, 0), dense, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(want, dense, rtol=1e-12, atol=1e-14)


def test_moe_expert_permutation_invariance():
    cfg = _moe_cfg()
    m = _model(cfg)
    h = RNG.standard_normal((8, cfg.d_model))
    y0 = m.moe(h, 0)
    perm = np.array([2, 0, 3, 1])
    for name in ("0.w_router", "0.we_gate", "0.we_up", "0.we_down"):
        m.W.w[name] = m.W[name][perm]
    np.testing.assert_allclose(m.moe(h, 0), y0, rtol=1e-12, atol=1e-14)


def test_router_ties_go_to_lower_expert():
    cfg = _moe_cfg(top_k=2, n_experts=4)
    m = _model(cfg)
    m.W.w["0.w_router"] = np.array([[1.0] + [0.0] * 31, [2.0] + [0.0] * 31,
                                    [2.0] + [0.0] * 31, [2.0] + [0.0] * 31])
    h = np.zeros((1, 32)); h[0, 0] = 1.0
    sel, w, gap, logits = m.router(h, 0)
    np.testing.assert_allclose(logits, [[1.0, 2.0, 2.0, 2.0]])
    assert sel.tolist() == [[1, 2]]
    np.testing.assert_allclose(w, [[0.5, 0.5]])
    assert gap[0] == 0.0


def _seq_forward_bruteforce(m, ids, allowed):
    """Full-sequence forward, positions 0..N-1, no KV cache, explicit mask,
    built only from the pinned primitives."""
    c = m.cfg
    x = m.W["embed"][ids].copy()
    n = len(ids)
    pos = np.arange(n)
    for l in range(c.n_layers):
        p = f"{l}."
        h = rms_norm(x, m.W[p + "attn_norm"], c.rms_eps)
        q = m.p.store(rope((h @ m.W[p + "wq"].T if c.dtype == "f32" else round_bf16(h) @ m.W[p + "wq"].T)
                           .reshape(n, c.n_q_heads, c.head_dim), pos, c.rope_base))
        k = m.p.store(rope((h @ m.W[p + "wk"].T if c.dtype == "f32" else round_bf16(h) @ m.W[p + "wk"].T)
                           .reshape(n, c.n_kv_heads, c.head_dim), pos, c.rope_base))
        v = m.p.store((h @ m.W[p + "wv"].T if c.dtype == "f32" else round_bf16(h) @ m.W[p + "wv"].T)
                      .reshape(n, c.n_kv_heads, c.head_dim))
        o = attention(q.transpose(1, 0, 2), k.transpose(1, 0, 2), v.transpose(1, 0, 2), allowed)
        o = m.p.store(o.transpose(1, 0, 2).reshape(n, c.q_dim))
        x = x + m.linear(o, p + "wo")
        h2 = rms_norm(x, m.W[p + "ffn_norm"], c.rms_eps)
        x = x + (m.swiglu(h2, p + "w_gate", p + "w_up", p + "w_down") if c.ffn == "dense"
                 else m.moe(h2, l))
    return x


def _block_causal(blocks):
    """Prefix causal; each later block sees everything before it and itself."""
    n = sum(blocks)
    allowed = np.zeros((n, n), bool)
    start = 0
    for bi, b in enumerate(blocks):
        for i in range(start, start + b):
            if bi == 0:
                allowed[i, :i + 1] = True
            else:
                allowed[i, :start + b] = True
        start += b
    return allowed


@pytest.mark.parametrize("dtype,ffn", [("f32", "dense"), ("bf16", "dense"), ("bf16", "moe")])
def test_cache_equals_full_recompute(dtype, ffn):
    cfg = _tiny_cfg(dtype=dtype) if ffn == "dense" else _moe_cfg(dtype=dtype)
    m = _model(cfg, seed=3)
    prefix = RNG.integers(0, cfg.vocab - 1, 9)
    c1 = RNG.integers(0, cfg.vocab, 6)
    c2 = np.full(6, cfg.mask_id)
    st = m.new_seq(32)
    m.prefill(st, prefix)
    # denoise over c1 with the cache == rows of the full recompute
    conf, pred, dbg = m.denoise(st, c1, debug=True)
    full = _seq_forward_bruteforce(m, np.concatenate([prefix, c1]), _block_causal([9, 6]))
    lg = m.logits(full[9:])
    lg[:, cfg.mask_id] = -np.inf
    np.testing.assert_allclose(dbg.logits, lg, rtol=1e-10, atol=1e-12)
    # append c1, denoise c2 == full block-causal recompute over [prefix; c1; c2]
    m.append(st, c1)
    assert st.T == 15
    _, _, dbg2 = m.denoise(st, c2, debug=True)
    full2 = _seq_forward_bruteforce(m, np.concatenate([prefix, c1, c2]), _block_causal([9, 6, 6]))
    lg2 = m.logits(full2[15:])
    lg2[:, cfg.mask_id] = -np.inf
    np.testing.assert_allclose(dbg2.logits, lg2, rtol=1e-10, atol=1e-12)


def test_chunked_prefill_equals_one_shot():
    cfg = _tiny_cfg()
    m = _model(cfg, seed=5)
    ids = RNG.integers(0, cfg.vocab - 1, 13)
    a, b = m.new_seq(20), m.new_seq(20)
    m.prefill(a, ids)
    m.prefill(b, ids[:5]); m.prefill(b, ids[5:11]); m.prefill(b, ids[11:])
    for l in range(cfg.n_layers):
        np.testing.assert_allclose(a.k[l], b.k[l], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(a.v[l], b.v[l], rtol=1e-12, atol=1e-14)


def test_prefill_is_causal():
    cfg = _tiny_cfg()
    m = _model(cfg, seed=6)
    ids = RNG.integers(0, cfg.vocab - 1, 12)
    a, b = m.new_seq(12), m.new_seq(12)
    m.prefill(a, ids)
    ids2 = ids.copy(); ids2[7] = (ids[7] + 1) % (cfg.vocab - 1)
    m.prefill(b, ids2)
    for l in range(cfg.n_layers):
        np.testing.assert_array_equal(a.k[l][:, :7], b.k[l][:, :7])
        assert not np.allclose(a.k[l][:, 7:], b.k[l][:, 7:])


def test_canvas_is_bidirectional_and_cache_is_untouched():
    cfg = _tiny_cfg()
    m = _model(cfg, seed=7)
    st = m.new_seq(30)
    m.prefill(st, RNG.integers(0, cfg.vocab - 1, 10))
    k_before = [k[:, :10].copy() for k in st.k]
    canvas = np.full(8, cfg.mask_id)
    canvas[5] = 3
    _, _, d1 = m.denoise(st, canvas, debug=True)
    canvas2 = canvas.copy(); canvas2[5] = 4
    _, _, d2 = m.denoise(st, canvas2, debug=True)
    keep = np.arange(cfg.vocab) != cfg.mask_id
    diff = np.abs(d1.logits[:, keep] - d2.logits[:, keep])
    assert np.all(diff.max(axis=1) > 0)          # every row, also rows before position 5
    assert st.T == 10
    for l in range(cfg.n_layers):
        np.testing.assert_array_equal(st.k[l][:, :10], k_before[l])


def test_denoise_conf_pred_hand_built():
    """OracleModel.denoise itself on a hand-built head: the prediction and the
    confidence exclude [MASK] (whose logit is made the largest), ties go to the
    lower id, and conf = 1 / sum exp(l - max) over the remaining vocabulary."""
    cfg = _tiny_cfg(vocab=4, mask_id=3)
    m = _model(cfg)
    # the transformer is bypassed so the final hidden state is known: row 0 is
    # e_0, row 1 is e_1; the head makes the logits a known function of it
    x = np.zeros((2, cfg.d_model)); x[0, 0] = 1.0; x[1, 1] = 1.0
    hn = rms_norm(x, m.W["final_norm"], cfg.rms_eps)
    scale = hn[0, 0]
    m.W.w["lm_head"] = np.zeros((4, cfg.d_model))
    m.W.w["lm_head"][1, 0] = np.log(3.0) / scale    # row 0: logits [0, log3, 0, 10 (mask)]
    m.W.w["lm_head"][3, 0] = 10.0 / scale           # mask logit largest: must be ignored
    m.W.w["lm_head"][0, 1] = 1.0 / scale            # row 1: logits [1, 0, 1, 0 (mask)] -> tie 0/2
    m.W.w["lm_head"][2, 1] = 1.0 / scale
    m.forward = lambda ids, st, causal, dbg=None: x.copy()
    st = m.new_seq(8)
    conf, pred, dbg = m.denoise(st, np.full(2, cfg.mask_id), debug=True)
    assert pred.tolist() == [1, 0]
    np.testing.assert_allclose(conf, [3 / 5, np.e / (2 * np.e + 1)], rtol=1e-12)
    assert np.all(np.isneginf(dbg.logits[:, 3]))
    # a confidence taken over the whole vocabulary (mask included) would differ
    assert abs(conf[0] - 3 / (5 + np.exp(10.0))) > 0.5
