"""Backward of the gate, of prefill HCA and of DSA sparse attention on the GPU against the NumPy
float64 backward oracle (chain rule of the forward definitions; ERNIE 5.5 Flash Base release
blog, section 2.1)."""
import numpy as np
import pytest

import hybrid_sparse_attention_amd as lgsa
from hybrid_sparse_attention_amd import synth
from oracle import backward

from helpers import bf16_ok, f32_ok, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lgsa.load()
    return torch


def _gate_inputs(seed, M, d_lat, N, bf16):
    return (synth.normal(seed, (M, d_lat), 1.0, bf16), synth.normal(seed + 1, (d_lat, N), 0.05, bf16),
            synth.normal(seed + 2, (M, N), 1.0, bf16), synth.normal(seed + 3, (M, N), 1.0, bf16))


@pytest.mark.parametrize("M,d_lat,N", [(300, 128, 320), (1, 64, 16), (129, 192, 272)])
def test_gate_backward_bf16(torch, M, d_lat, N):
    q, w, o, dout = _gate_inputs(90 + M, M, d_lat, N, True)
    d_o, dq, dw = lgsa.latent_gate_bwd(to_dev(q), to_dev(w), to_dev(o), to_dev(dout))
    torch.cuda.synchronize()
    r_o, r_q, r_w = backward.latent_gate_bwd(q, w, o, dout)
    bf16_ok(from_dev(d_o), r_o, "d_o")
    bf16_ok(from_dev(dq), r_q, "dq_lat")
    bf16_ok(from_dev(dw), r_w, "dw_gate")


@pytest.mark.parametrize("M,d_lat,N", [(70, 24, 50), (5, 3, 7)])
def test_gate_backward_f32(torch, M, d_lat, N):
    q, w, o, dout = _gate_inputs(95 + M, M, d_lat, N, False)
    d_o, dq, dw = lgsa.latent_gate_bwd(to_dev(q), to_dev(w), to_dev(o), to_dev(dout))
    torch.cuda.synchronize()
    r_o, r_q, r_w = backward.latent_gate_bwd(q, w, o, dout)
    f32_ok(from_dev(d_o), r_o, "d_o")
    f32_ok(from_dev(dq), r_q, "dq_lat")
    f32_ok(from_dev(dw), r_w, "dw_gate")


def test_gate_backward_bf16_wide(torch):
    """A long contraction for both products (d_lat 1024, 4096 rows, 8192 channels): every d_o
    row, and sampled rows of dq_lat and columns of dw_gate, each from the oracle's float64
    formulas restricted to what they need."""
    M, d_lat, N = 4096, 1024, 8192
    q, w, o, dout = _gate_inputs(140, M, d_lat, N, True)
    d_o, dq, dw = lgsa.latent_gate_bwd(to_dev(q), to_dev(w), to_dev(o), to_dev(dout))
    torch.cuda.synchronize()
    Q, W = synth.bf16_to_f32(q).astype(np.float64), synth.bf16_to_f32(w).astype(np.float64)
    rows = [0, 1, 777, 2048, 4095]
    cols = [0, 15, 4100, 8191]
    r_o, r_q, _ = backward.latent_gate_bwd(q[rows], w, o[rows], dout[rows])
    bf16_ok(from_dev(d_o)[rows], r_o, "d_o rows")
    bf16_ok(from_dev(dq)[rows], r_q, "dq_lat rows")
    O = synth.bf16_to_f32(o[:, cols]).astype(np.float64)
    D = synth.bf16_to_f32(dout[:, cols]).astype(np.float64)
    s = 1.0 / (1.0 + np.exp(-(Q @ W[:, cols])))
    ref_w = Q.T @ (D * O * s * (1.0 - s))
    bf16_ok(from_dev(dw)[:, cols], ref_w, "dw_gate columns")


def _hca_case(torch, seed, B, T, H, window, block):
    """GPU forward (with its lse) and backward of prefill HCA on seeded bf16 inputs; returns the
    inputs and the three gradients."""
    import math
    q = synth.normal(seed, (B, T, H, 512), 1.0, True)
    k = synth.normal(seed + 1, (B, T, 512), 1.0, True)
    v = synth.normal(seed + 2, (B, T, 512), 1.0, True)
    dout = synth.normal(seed + 3, (B, T, H, 512), 1.0, True)
    dq_, dk_, dv_ = to_dev(q), to_dev(k), to_dev(v)
    kc, vc = lgsa.hca_compress(dk_, dv_, block=block)
    lse = torch.empty((B, T, H), dtype=torch.float32, device="cuda")
    pos0 = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = lgsa.hca_attn_fwd(dq_, pos0, dk_, dv_, kc if T >= block else None,
                            vc if T >= block else None, max_pos=T - 1, window=window,
                            block=block, lse=lse)
    g = lgsa.hca_attn_bwd(dq_, dk_, dv_, kc if T >= block else None, vc if T >= block else None,
                          out, lse, to_dev(dout), window=window, block=block)
    torch.cuda.synchronize()
    return (q, k, v, dout), [from_dev(x) for x in g]


@pytest.mark.parametrize("B,T,H,window,block", [(2, 300, 4, 48, 32), (1, 1100, 4, 128, 128),
                                                (1, 40, 8, 64, 128), (1, 260, 4, 100, 64),
                                                (2, 1024, 4, 128, 128)])
def test_hca_backward(torch, B, T, H, window, block):
    """dq, dk, dv against the float64 oracle (which rebuilds everything from q, k, v): the
    window path, the pooled path (an entry's gradient spread over its block) and a sequence
    shorter than a block.  (2, 1024) gives the dq and dkv kernels workgroup counts that are
    multiples of 8 (64 and 32), so both take their XCD-aware orders across two sequences."""
    (q, k, v, dout), (dq, dk, dv) = _hca_case(torch, 150 + T, B, T, H, window, block)
    r_q, r_k, r_v = backward.hca_attn_bwd(q, np.zeros(B, np.int32), k, v, dout, window=window,
                                          block=block)
    bf16_ok(dq, r_q, "dq")
    bf16_ok(dk, r_k, "dk")
    bf16_ok(dv, r_v, "dv")


def test_hca_backward_deterministic(torch):
    _, g1 = _hca_case(torch, 170, 1, 700, 4, 128, 128)
    _, g2 = _hca_case(torch, 170, 1, 700, 4, 128, 128)
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b)


def _sparse_case(torch, seed, B, Tq, S, k, distinct_v, idx=None, ws_frac=None, H=64):
    """GPU forward (ungated, with its lse) and backward of sparse attention on seeded bf16
    inputs; ws_frac < 1 hands the backward that fraction of its default workspace, so that it
    takes the rows in several chunks."""
    x = synth.dsa_sparse(seed, B=B, Tq=Tq, S=S, H=H, distinct_v=distinct_v, gated=False)
    if idx is None:
        idx = synth.random_topk(seed, B, Tq, S, k, [S - Tq] * B)
    dout = synth.normal(seed + 7, (B, Tq, H, 256), 1.0, True)
    q, kl = to_dev(x["q"]), to_dev(x["kv_lat"])
    vl = to_dev(x["v_lat"]) if distinct_v else None
    ix = to_dev(idx)
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device="cuda")
    out = lgsa.sparse_attn_fwd(q, kl, ix, v_lat=vl, lse=lse)
    do = to_dev(dout)
    ws = None
    if ws_frac is not None:
        n = lgsa.sparse_attn_bwd_workspace_bytes(q, kl, ix, out, lse, do, v_lat=vl)
        ws = torch.empty(int(n * ws_frac) // 16 * 16, dtype=torch.uint8, device="cuda")
    g = lgsa.sparse_attn_bwd(q, kl, ix, out, lse, do, v_lat=vl, workspace=ws)
    torch.cuda.synchronize()
    return x, idx, dout, from_dev(lse), [None if t is None else from_dev(t) for t in g]


@pytest.mark.parametrize("B,Tq,S,k,distinct_v,ws_frac", [
    (1, 40, 300, 64, False, None),     # two tiles per row, every row a full list
    (2, 33, 200, 100, True, None),     # ragged last tile, distinct values, two sequences
    (1, 70, 90, 128, False, None),     # early rows list fewer keys than k (-1 padding)
    (1, 57, 400, 96, False, 0.45),     # rows taken in three chunks (accumulator carried)
    (2, 20, 150, 40, True, 0.6),       # chunks and distinct values
    (1, 12, 70000, 64, False, None),   # more keys than the LDS counters hold: global counters
])
def test_sparse_backward(torch, B, Tq, S, k, distinct_v, ws_frac):
    """dq and the latent-row gradients (dk, and dv when the values are distinct) against the
    float64 oracle, which rebuilds the softmax from q and the rows; the forward's lse against
    the oracle's log-sum-exp."""
    x, idx, dout, lse, (dq, dk, dv) = _sparse_case(torch, 300 + Tq, B, Tq, S, k, distinct_v,
                                                   ws_frac=ws_frac)
    r_q, r_k, r_v = backward.sparse_attn_bwd(x["q"], x["kv_lat"], idx, dout,
                                             v_lat=x.get("v_lat"))
    bf16_ok(dq, r_q, "dq")
    bf16_ok(dk, r_k, "dk")
    if distinct_v:
        bf16_ok(dv, r_v, "dv")
    r_lse = backward.sparse_attn_lse(x["q"], x["kv_lat"], idx)
    assert np.allclose(lse, r_lse, rtol=0, atol=1e-3), float(np.max(np.abs(lse - r_lse)))


def test_sparse_backward_repeats_skips_and_empty_rows(torch):
    """Entries listed twice count twice, out-of-range and negative entries are skipped, a row
    with no valid entry gets dq = 0 and lse = -inf, and rows no entry lists get zero gradient."""
    B, Tq, S, k = 1, 6, 80, 48
    rng = np.random.default_rng(11)
    idx = rng.integers(0, 60, size=(B, Tq, k)).astype(np.int32)
    idx[0, 0, 5] = idx[0, 0, 6]
    idx[0, 1, :10] = -1
    idx[0, 2, 3] = S + 3
    idx[0, 3, :] = -1
    x, idx, dout, lse, (dq, dk, _) = _sparse_case(torch, 320, B, Tq, S, k, False, idx=idx)
    r_q, r_k, _ = backward.sparse_attn_bwd(x["q"], x["kv_lat"], idx, dout)
    bf16_ok(dq, r_q, "dq")
    bf16_ok(dk, r_k, "dk")
    assert np.all(dq[0, 3] == 0) and np.all(lse[0, 3] == -np.inf)
    assert np.all(dk[0, 60:] == 0)


@pytest.mark.parametrize("distinct_v", [False, True])
def test_sparse_backward_two_head_groups(torch, distinct_v):
    """128 heads: two workgroups per row, each writing its own contribution of every entry
    (summed by the reduction); with a small workspace so that chunks are carried too."""
    B, Tq, S, k = 1, 24, 180, 72
    x, idx, dout, lse, (dq, dk, dv) = _sparse_case(torch, 340, B, Tq, S, k, distinct_v,
                                                   ws_frac=0.7, H=128)
    r_q, r_k, r_v = backward.sparse_attn_bwd(x["q"], x["kv_lat"], idx, dout,
                                             v_lat=x.get("v_lat"))
    bf16_ok(dq, r_q, "dq")
    bf16_ok(dk, r_k, "dk")
    if distinct_v:
        bf16_ok(dv, r_v, "dv")


def test_sparse_lse_and_backward_split_rows(torch):
    """Few rows with long lists: the forward splits each list over workgroups and writes the
    log-sum-exp from its combine kernel; the backward then uses it (two sequences at different
    positions, one row with a short list)."""
    B, S, k = 2, 5000, 2048
    x = synth.dsa_sparse(350, B=B, Tq=2, S=S, H=64, gated=False)
    idx = synth.random_topk(350, B, 2, S, k, [4990, 1500])
    dout = synth.normal(357, (B, 2, 64, 256), 1.0, True)
    q, kl, ix = to_dev(x["q"]), to_dev(x["kv_lat"]), to_dev(idx)
    lse = torch.empty((B, 2, 64), dtype=torch.float32, device="cuda")
    out = lgsa.sparse_attn_fwd(q, kl, ix, lse=lse)
    dq, dk, _ = lgsa.sparse_attn_bwd(q, kl, ix, out, lse, to_dev(dout))
    torch.cuda.synchronize()
    r_lse = backward.sparse_attn_lse(x["q"], x["kv_lat"], idx)
    got = from_dev(lse)
    assert np.allclose(got, r_lse, rtol=0, atol=1e-3), float(np.max(np.abs(got - r_lse)))
    r_q, r_k, _ = backward.sparse_attn_bwd(x["q"], x["kv_lat"], idx, dout)
    bf16_ok(from_dev(dq), r_q, "dq")
    bf16_ok(from_dev(dk), r_k, "dk")


def test_sparse_backward_deterministic(torch):
    g1 = _sparse_case(torch, 330, 1, 64, 500, 128, False)[-1]
    g2 = _sparse_case(torch, 330, 1, 64, 500, 128, False)[-1]
    for a, b in zip(g1[:2], g2[:2]):
        assert np.array_equal(a, b)

