"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: hand-worked examples
(tests/golden), closed forms, brute-force enumeration of the visibility rule through one-hot
probes, the reduction to textbook dense attention (NumPy), invariants of softmax, and a
brute-force sort for top-k.  Sources: ERNIE 5.5 Flash Base release blog, section 2.1
"Latent-Gated Sparse Attention"; xenospectrum.com article on ERNIE 5.5 Flash Base, section on
the 128-token sliding window.
"""
import json
import math
import os

import numpy as np
import pytest

from hybrid_sparse_attention_amd import synth
from oracle.dense import dense_causal

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------------------ compressor
def test_bf16_widening_known_bits(orc):
    # block = 1 makes the compressor the identity, exposing the bf16 decode of the oracle
    bits = np.array([[[0x3F80, 0xC000, 0x3F81, 0x0001, 0x8000, 0x4049]]], dtype=np.uint16)
    got = orc.hca_compress(bits, block=1)[0, 0]
    want = [1.0, -2.0, 1.0078125, 2.0 ** -133, -0.0, 3.140625]
    assert got.tolist() == want


def test_compress_constant_ramp_and_tail(orc):
    T, d, c = 300, 3, 0.25
    ramp = (np.arange(T, dtype=np.float64)[:, None] * c * np.ones((1, d)))[None]
    got = orc.hca_compress(ramp.astype(np.float32), block=128)
    assert got.shape == (1, 2, d)  # the incomplete third block (tokens 256..299) is dropped
    for b in range(2):
        assert np.all(got[0, b] == (128 * b + 63.5) * c)  # mean of an arithmetic run
    const = np.full((2, 256, 4), 7.5, dtype=np.float32)
    assert np.all(orc.hca_compress(const) == 7.5)


def test_compress_small_integers_exact(orc):
    rng = np.random.default_rng(3)
    x = rng.integers(-8, 8, size=(2, 512, 5)).astype(np.float32)
    got = orc.hca_compress(x)
    want = x.astype(np.float64).reshape(2, 4, 128, 5).sum(axis=2) / 128.0
    assert np.array_equal(got, want)


# ------------------------------------------------------------------------------ HCA
def test_hca_worked_example(orc):
    g = _gold("hca_worked_example.json")
    k = np.array(g["k"])[None]
    v = np.array(g["v"])[None]
    q = np.array(g["q"])[:, None, :][None]          # [1,T,1,d]
    kc = orc.hca_compress(k, block=g["block"])
    vc = orc.hca_compress(v, block=g["block"])
    out = orc.hca_attn(q, [0], k, v, kc, vc, window=g["window"], block=g["block"],
                       scale=g["scale"])
    want = np.array([[n / dd for n, dd in row] for row in g["o_num"]])
    np.testing.assert_allclose(out[:, 0, :], want, rtol=0, atol=1e-14)
    # gated: d_lat = 1, q_lat = 1
    ql = np.ones((1, 4, 1))
    w = np.array(g["w_gate"])
    gated = orc.hca_attn(q, [0], k, v, kc, vc, window=g["window"], block=g["block"],
                         scale=g["scale"], q_lat=ql, w_gate=w)
    np.testing.assert_allclose(gated[:, 0, :], want * np.array(g["gate_factor"]), rtol=0,
                               atol=1e-14)


def _visible_rule(t, window, block, n_cap):
    comp = [e for e in range(n_cap) if e * block + block - 1 <= t]
    win = list(range(max(0, t - window + 1), t + 1))
    return comp, win


@pytest.mark.parametrize("T,block,window", [(300, 128, 128), (37, 4, 5), (64, 8, 64)])
def test_hca_visibility_onehot(orc, T, block, window):
    """Equal logits (q = 0) weight every visible key equally, and one-hot values reveal which
    keys were used and how often; compare with a direct enumeration of the visibility rule."""
    n_cap = T // block
    d = T + n_cap
    k = np.zeros((1, T, d))
    v = np.zeros((1, T, d))
    v[0, np.arange(T), np.arange(T)] = 1.0
    kc = np.zeros((1, n_cap, d))
    vc = np.zeros((1, n_cap, d))
    vc[0, np.arange(n_cap), T + np.arange(n_cap)] = 1.0
    q = np.zeros((1, T, 1, d))
    out = orc.hca_attn(q, [0], k, v, kc, vc, window=window, block=block)[:, 0, :]
    for t in range(T):
        comp, win = _visible_rule(t, window, block, n_cap)
        want = np.zeros(d)
        want[win] = 1.0
        want[[T + e for e in comp]] = 1.0
        want /= len(comp) + len(win)
        np.testing.assert_allclose(out[t], want, rtol=0, atol=1e-15)


def test_hca_ring_window_decode(orc):
    """Decode reads the window from a ring (position p in row p % win_len); compare with the
    same keys laid out flat."""
    rng = np.random.default_rng(5)
    B, H, d, block, window, ctx = 3, 2, 16, 8, 8, [45, 8, 1]
    S = max(ctx)
    kf = rng.standard_normal((B, S, d))
    vf = rng.standard_normal((B, S, d))
    kc = orc.hca_compress(kf, block)
    vc = orc.hca_compress(vf, block)
    ring_k = np.zeros((B, window, d))
    ring_v = np.zeros((B, window, d))
    for b in range(B):
        for p in range(max(0, ctx[b] - window), ctx[b]):
            ring_k[b, p % window] = kf[b, p]
            ring_v[b, p % window] = vf[b, p]
    q = rng.standard_normal((B, 1, H, d))
    pos0 = [c - 1 for c in ctx]
    got = orc.hca_attn(q, pos0, ring_k, ring_v, kc, vc, window=window, block=block)
    want = np.concatenate([orc.hca_attn(q[b:b + 1], [pos0[b]], kf[b:b + 1], vf[b:b + 1],
                                        kc[b:b + 1], vc[b:b + 1], window=window, block=block)
                           for b in range(B)])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


def test_hca_t0_is_first_value(orc):
    x = synth.hca_prefill(100, T=130, H=3, d=8, bf16=True, gated=False)
    kc = orc.hca_compress(x["k"])
    vc = orc.hca_compress(x["v"])
    out = orc.hca_attn(x["q"], x["pos0"], x["k"], x["v"], kc, vc, rows=[0])
    v0 = synth.bf16_to_f32(x["v"][0, 0]).astype(np.float64)
    for h in range(3):
        assert np.array_equal(out[0, h], v0)


def test_hca_reduces_to_dense(orc):
    """No compressed entries and a window covering the whole sequence is dense causal
    attention."""
    x = synth.hca_prefill(101, T=150, H=3, d=32, bf16=True, gated=False)
    out = orc.hca_attn(x["q"], x["pos0"], x["k"], x["v"], None, None, window=150)
    ref = dense_causal(x["q"][0], x["k"][0], x["v"][0])
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_hca_rows_sum_to_one(orc):
    """Constant values v = 1 give O = 1: the softmax weights of every row sum to one."""
    rng = np.random.default_rng(7)
    T, d = 270, 16
    q = rng.standard_normal((1, T, 2, d)) * 3
    k = rng.standard_normal((1, T, d)) * 3
    v = np.ones((1, T, d))
    kc = orc.hca_compress(k)
    vc = orc.hca_compress(v)
    out = orc.hca_attn(q, [0], k, v, kc, vc)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-12)


def test_hca_equal_keys_mean_of_visible_values(orc):
    """All keys equal: O is the mean of the visible values; at t = 127 the single complete
    block contributes its own mean once more, so O = mean(V[0..127])."""
    rng = np.random.default_rng(8)
    T, d = 256, 8
    k = np.ones((1, T, d))
    v = rng.standard_normal((1, T, d))
    kc = orc.hca_compress(k)
    vc = orc.hca_compress(v)
    q = rng.standard_normal((1, T, 1, d))
    out = orc.hca_attn(q, [0], k, v, kc, vc)[:, 0, :]
    np.testing.assert_allclose(out[127], v[0, :128].mean(axis=0), rtol=0, atol=1e-13)
    # t = 200: entry 0 (mean of 0..127) plus raw rows 73..200
    want = (v[0, :128].mean(axis=0) + v[0, 73:201].sum(axis=0)) / 129.0
    np.testing.assert_allclose(out[200], want, rtol=0, atol=1e-13)


def test_hca_compressed_entry_becomes_visible_when_complete(orc):
    """Entry b appears exactly at t = 128b + 127: a marker value placed only in entry 1."""
    T, d = 400, 1
    k = np.zeros((1, T, d))
    v = np.zeros((1, T, d))
    kc = np.zeros((1, 3, d))
    vc = np.zeros((1, 3, d))
    vc[0, 1, 0] = 1.0
    q = np.zeros((1, T, 1, d))
    out = orc.hca_attn(q, [0], k, v, kc, vc)[:, 0, 0]
    assert np.all(out[:255] == 0.0)
    assert out[255] == pytest.approx(1.0 / (2 + 128), abs=1e-15)
    assert out[399] == pytest.approx(1.0 / (3 + 128), abs=1e-15)


# ------------------------------------------------------------------------------ gate
def test_gate_zero_weight_halves(orc):
    rng = np.random.default_rng(9)
    o = rng.standard_normal((5, 12))
    ql = rng.standard_normal((5, 4))
    out = orc.latent_gate(ql, np.zeros((4, 12)), o)
    assert np.array_equal(out, 0.5 * o)
    out = orc.latent_gate(np.zeros((5, 4)), rng.standard_normal((4, 12)), o)
    assert np.array_equal(out, 0.5 * o)


def test_gate_closed_form_and_saturation(orc):
    o = np.array([[2.0, -3.0, 1.0]])
    ql = np.array([[1.0, 0.0]])
    w = np.array([[0.7, -1.3, 60.0], [5.0, 5.0, 5.0]])
    out = orc.latent_gate(ql, w, o)[0]
    sig = [1.0 / (1.0 + math.exp(-0.7)), 1.0 / (1.0 + math.exp(1.3)), 1.0]
    np.testing.assert_allclose(out, o[0] * np.array(sig), rtol=1e-15, atol=1e-15)


def test_gate_matches_gated_attention(orc):
    x = synth.hca_prefill(102, T=140, H=2, d=16, bf16=True, d_lat=24)
    kc, vc = orc.hca_compress(x["k"]), orc.hca_compress(x["v"])
    plain = orc.hca_attn(x["q"], x["pos0"], x["k"], x["v"], kc, vc)
    gated = orc.hca_attn(x["q"], x["pos0"], x["k"], x["v"], kc, vc, q_lat=x["q_lat"],
                         w_gate=x["w_gate"])
    via = orc.latent_gate(x["q_lat"][0], x["w_gate"], plain.reshape(140, -1))
    np.testing.assert_allclose(gated.reshape(140, -1), via, rtol=0, atol=1e-14)


# ------------------------------------------------------------------------------ indexer
def test_dsa_worked_example(orc):
    g = _gold("dsa_worked_example.json")
    q = np.array(g["q_idx"], dtype=np.float32)[None, None]       # [1,1,2,2]
    w = np.array(g["w_idx"], dtype=np.float32)[None, None]       # [1,1,2]
    k = np.array(g["k_idx"], dtype=np.float32)[None]             # [1,5,2]
    sc = orc.dsa_scores(q, w, k, 0, 0, 0, 5)
    assert sc.tolist() == g["scores"]
    for case in g["cases"]:
        idx, _ = orc.dsa_topk(q, w, k, [case["t"]], case["k"])
        assert idx[0].tolist() == case["idx"], case


def test_dsa_scores_single_head_is_relu_dot(orc):
    rng = np.random.default_rng(11)
    S, di = 50, 64
    q = rng.standard_normal((1, 3, 4, di)).astype(np.float32)
    k = rng.standard_normal((1, S, di)).astype(np.float32)
    for h in range(4):
        w = np.zeros((1, 3, 4), dtype=np.float32)
        w[0, 2, h] = 1.0
        sc = orc.dsa_scores(q, w, k, 0, 2, 0, S)
        want = np.maximum(k[0].astype(np.float64) @ q[0, 2, h].astype(np.float64), 0.0)
        np.testing.assert_allclose(sc, want, rtol=1e-14, atol=1e-12)


def _brute_topk(scores, t, k):
    n = t + 1
    if n <= k:
        return list(range(n)) + [-1] * (k - n)
    order = sorted(range(n), key=lambda s: (-scores[s], s))
    return sorted(order[:k])


def test_dsa_topk_brute_force(orc):
    x = synth.dsa_index(103, B=2, Tq=40, S=200, pos0=[0, 160])
    k = 16
    idx, kth = orc.dsa_topk(x["q_idx"], x["w_idx"], x["k_idx"], x["pos0"], k)
    for r in range(80):
        b, i = divmod(r, 40)
        t = int(x["pos0"][b]) + i
        sc = orc.dsa_scores(x["q_idx"], x["w_idx"], x["k_idx"], b, i, 0, t + 1)
        assert idx[r].tolist() == _brute_topk(sc, t, k)
        if t + 1 > k:
            assert kth[r] == sorted(sc, reverse=True)[k - 1]


def test_dsa_topk_ties_lower_index_and_negative_zero(orc):
    # duplicated key rows give equal scores: the lower position wins
    rng = np.random.default_rng(12)
    base = rng.standard_normal((1, 1, 2, 8)).astype(np.float32)
    k = np.tile(rng.standard_normal((1, 1, 8)).astype(np.float32), (1, 30, 1))
    w = np.ones((1, 1, 2), dtype=np.float32)
    idx, _ = orc.dsa_topk(base, w, k, [29], 5)
    assert idx[0].tolist() == [0, 1, 2, 3, 4]
    # q = -0.0 everywhere: every dot is -0.0 or +0.0, every score zero -> positions 0..k-1
    qz = np.full((1, 1, 2, 8), -0.0, dtype=np.float32)
    kk = np.abs(rng.standard_normal((1, 30, 8))).astype(np.float32)
    idx, kth = orc.dsa_topk(qz, w, kk, [29], 7)
    assert idx[0].tolist() == list(range(7)) and kth[0] == 0.0
    sc = orc.dsa_scores(qz, w, kk, 0, 0, 0, 30)
    assert all(math.copysign(1.0, s) == 1.0 for s in sc)  # no -0.0 survives


def test_dsa_topk_all_when_short(orc):
    x = synth.dsa_index(104, B=1, Tq=10, S=10)
    idx, kth = orc.dsa_topk(x["q_idx"], x["w_idx"], x["k_idx"], x["pos0"], 12)
    for t in range(10):
        assert idx[t].tolist() == list(range(t + 1)) + [-1] * (11 - t)
        assert kth[t] == -np.inf


# ------------------------------------------------------------------------------ sparse
def test_sparse_full_selection_is_dense(orc):
    """k >= context selects every causal position, which is dense causal attention."""
    T, H, d = 70, 3, 32
    x = synth.dsa_sparse(105, B=1, Tq=T, S=T, H=H, d=d, gated=False)
    idx = synth.random_topk(105, 1, T, T, k=T, pos0=[0])
    out = orc.sparse_attn(x["q"], x["kv_lat"], idx)
    ref = dense_causal(x["q"][0], x["kv_lat"][0], x["kv_lat"][0])
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_sparse_order_invariance_and_padding(orc):
    T, H, d, k = 60, 2, 16, 20
    x = synth.dsa_sparse(106, B=1, Tq=T, S=T, H=H, d=d, distinct_v=True, gated=False)
    idx = synth.random_topk(106, 1, T, T, k=k, pos0=[0])
    out = orc.sparse_attn(x["q"], x["kv_lat"], idx, v_lat=x["v_lat"])
    rng = np.random.default_rng(13)
    shuffled = np.concatenate([idx, np.full((1, T, 7), -1, np.int32)], axis=-1)
    for t in range(T):
        rng.shuffle(shuffled[0, t])
    out2 = orc.sparse_attn(x["q"], x["kv_lat"], shuffled, v_lat=x["v_lat"])
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-12)
    # subsets written out explicitly: dense attention over exactly those rows
    from oracle.dense import bf16_to_f64
    q = bf16_to_f64(x["q"][0])
    kf = bf16_to_f64(x["kv_lat"][0])
    vf = bf16_to_f64(x["v_lat"][0])
    for t in (0, 5, 33, 59):
        sel = [s for s in idx[0, t] if s >= 0]
        lg = q[t] @ kf[sel].T / math.sqrt(d)
        p = np.exp(lg - lg.max(axis=-1, keepdims=True))
        p /= p.sum(axis=-1, keepdims=True)
        np.testing.assert_allclose(out[t], p @ vf[sel], rtol=0, atol=1e-12)


def test_sparse_empty_selection_is_zero(orc):
    x = synth.dsa_sparse(107, B=1, Tq=2, S=5, H=2, d=8, gated=False)
    idx = np.full((1, 2, 3), -1, np.int32)
    idx[0, 1, 1] = 7  # beyond S: skipped too
    assert np.all(orc.sparse_attn(x["q"], x["kv_lat"], idx) == 0.0)


def test_sparse_strided_value_view(orc):
    """A latent row holding K in its first half and V in its second half."""
    rng = np.random.default_rng(14)
    S, d = 40, 8
    row = rng.standard_normal((1, S, 2 * d))
    q = rng.standard_normal((1, 4, 2, d))
    idx = synth.random_topk(108, 1, 4, S, 6, pos0=[30])
    a = orc.sparse_attn(q, row, idx, v_lat=row[:, :, d:].copy(), dqk=d, dv=d)
    kf = row[:, :, :d].copy()
    vf = row[:, :, d:].copy()
    b = orc.sparse_attn(q, kf, idx, v_lat=vf)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


# ------------------------------------------------------------------------------ shapes
def test_model_dims_follow_the_pages():
    g = _gold("model_dims.json")
    assert synth.HIDDEN == g["hidden"]["value"] and synth.HEADS == g["heads"]["value"]
    assert synth.D_HCA == g["hca_head_dim"]["value"]
    assert synth.D_MLA == g["mla_head_dim"]["value"]
    assert synth.BLOCK == g["block"]["value"] and synth.WINDOW == g["window"]["value"]
    assert synth.D_LAT == g["latent"]["value"] == g["hidden"]["value"] // 4
    assert g["hca_layers"]["value"] + g["mla_layers"]["value"] == g["layers"]["value"]
