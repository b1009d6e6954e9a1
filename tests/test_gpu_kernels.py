"""GPU parity of every entry point against the fp64 oracle on small seeded inputs that span
several tiles and a ragged tail, plus the method's edge cases.  Every call goes through the
C ABI (liblgsa.so) via the ctypes binding.  Tolerances are stated in tests/helpers.py.
"""
import numpy as np
import pytest

import hybrid_sparse_attention_amd as lgsa
from hybrid_sparse_attention_amd import synth

from helpers import bf16_ok, check_topk_row, f32_ok, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lgsa.load()
    return torch


# ------------------------------------------------------------------------------ compressor
@pytest.mark.parametrize("bf16,B,T", [(True, 2, 300), (False, 1, 1024), (True, 1, 127)])
def test_compress(torch, orc, bf16, B, T):
    k = synth.normal(200, (B, T, 512), 1.0, bf16)
    v = synth.normal(201, (B, T, 512), 1.0, bf16)
    kc, vc = lgsa.hca_compress(to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    for got, x in ((kc, k), (vc, v)):
        ref = orc.hca_compress(x)
        assert got.shape == ref.shape
        g = from_dev(got)
        if bf16:
            bf16_ok(g, ref, "compress")
            # rounding of an fp32 sum: within one bf16 ulp of the exact mean
            assert np.all(np.abs(g - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6)
        else:
            f32_ok(g, ref, "compress")


# ------------------------------------------------------------------------------ gate
# (4352, 1024, 4096) and (4400, 256, 4112) run the 256 x 256-tile kernel over hundreds of
# tiles, the second with ragged tiles on both edges; they are checked on sampled rows
@pytest.mark.parametrize("M,d_lat,N,inplace", [(200, 128, 96, False), (130, 1024, 2048, True),
                                               (8, 1024, 512, False), (600, 1024, 800, True),
                                               (512, 192, 1024, False), (37, 1024, 1008, True),
                                               (64, 1024, 4096, False), (4352, 1024, 4096, True),
                                               (4400, 256, 4112, False)])
def test_gate_bf16(torch, orc, M, d_lat, N, inplace):
    ql = synth.normal(210, (M, d_lat), 1.0, True)
    w = synth.normal(211, (d_lat, N), 0.02, True)
    o = synth.normal(212, (M, N), 1.0, True)
    od = to_dev(o)
    out = lgsa.latent_gate(to_dev(ql), to_dev(w), od, out=od if inplace else None)
    torch.cuda.synchronize()
    # large shapes: every 37th row and the last (all row tiles, all columns)
    rows = np.unique(np.r_[np.arange(0, M, 37), M - 1]) if M > 1024 else np.arange(M)
    bf16_ok(from_dev(out)[rows], orc.latent_gate(ql, w, o, rows=rows), "gate")


def test_gate_f32(torch, orc):
    ql = synth.normal(213, (70, 37))
    w = synth.normal(214, (37, 50), 0.3)
    o = synth.normal(215, (70, 50))
    out = lgsa.latent_gate(to_dev(ql), to_dev(w), to_dev(o))
    torch.cuda.synchronize()
    f32_ok(from_dev(out), orc.latent_gate(ql, w, o), "gate f32")


# ------------------------------------------------------------------------------ HCA
def _hca_gpu(x, kc, vc, max_pos, gated, window=128, dev_out=None):
    return lgsa.hca_attn_fwd(to_dev(x["q"]), to_dev(x["pos0"]), to_dev(x["k"]), to_dev(x["v"]),
                             kc, vc, max_pos=max_pos, window=window,
                             q_lat=to_dev(x["q_lat"]) if gated else None,
                             w_gate=to_dev(x["w_gate"]) if gated else None, out=dev_out)


# (1100, 30) leaves half of the last 4-head group idle; (1500, 64) is the full head count with
# 752 (token tile, head group) workgroups; (1100, 8) gated takes the fused kernel's XCD order
# (head count a multiple of 8) over 9 token tiles, each XCD starting one tile further on
@pytest.mark.parametrize("T,H,gated", [(1100, 3, True), (1100, 2, False), (100, 2, True),
                                       (257, 1, True), (1100, 30, True), (1500, 64, False),
                                       (1100, 8, True)])
def test_hca_prefill_bf16(torch, orc, T, H, gated):
    x = synth.hca_prefill(220 + T % 7, T=T, H=H, bf16=True, gated=gated)
    kd, vd = to_dev(x["k"]), to_dev(x["v"])
    kc, vc = lgsa.hca_compress(kd, vd) if T >= 128 else (None, None)
    out = _hca_gpu(x, kc, vc, T - 1, gated)
    torch.cuda.synchronize()
    okc = orc.hca_compress(x["k"]) if T >= 128 else None
    ovc = orc.hca_compress(x["v"]) if T >= 128 else None
    ref = orc.hca_attn(x["q"], x["pos0"], x["k"], x["v"], okc, ovc,
                       q_lat=x.get("q_lat"), w_gate=x.get("w_gate"))
    bf16_ok(from_dev(out)[0], ref, "hca prefill")


def test_hca_prefill_chunked_positions(torch, orc):
    """Two sequences whose query rows start at different positions: the window reaches back
    before the first query row, the compressed entries come from the whole prefix."""
    B, Ttot, Tq, H = 2, 700, 400, 2
    q = synth.normal(230, (B, Tq, H, 512), 1.0, True)
    k = synth.normal(231, (B, Ttot, 512), 1.0, True)
    v = synth.normal(232, (B, Ttot, 512), 1.0, True)
    pos0 = np.array([0, 300], np.int32)
    kc, vc = lgsa.hca_compress(to_dev(k), to_dev(v))
    out = lgsa.hca_attn_fwd(to_dev(q), to_dev(pos0), to_dev(k), to_dev(v), kc, vc, max_pos=699)
    torch.cuda.synchronize()
    ref = orc.hca_attn(q, pos0, k, v, orc.hca_compress(k), orc.hca_compress(v))
    bf16_ok(from_dev(out).reshape(-1, H, 512), ref, "hca chunked")


@pytest.mark.parametrize("d_lat", [384, 128, 192, 64])
def test_hca_prefill_gated_ring_positions(torch, orc, d_lat):
    """The gated prefill over a ring of raw rows: two sequences whose 200 query rows start at
    positions 0 and 1000, raw rows in a 512-row ring (position p in row p % 512; 512 >= window
    + 199), entries from each whole prefix.  The gate runs in the attention epilogue through a
    ring of four stages, steps of 32: contractions of 384 (three rounds of the four stages),
    128 (one round), 192 (a round and a half) and 64 (two steps, fewer than the three the ring
    keeps in flight).  The log-sum-exp written matches the ungated kernel's."""
    B, Tq, H, W, ctx = 2, 200, 3, 512, 1200
    pos0 = np.array([0, 1000], np.int32)
    q = synth.normal(233, (B, Tq, H, 512), 1.0, True)
    k = synth.normal(234, (B, ctx, 512), 1.0, True)
    v = synth.normal(235, (B, ctx, 512), 1.0, True)
    ql = synth.normal(236, (B, Tq, d_lat), 1.0, True)
    wg = synth.normal(237, (d_lat, H * 512), 0.02, True)
    ring_k = np.zeros((B, W, 512), np.uint16)
    ring_v = np.zeros((B, W, 512), np.uint16)
    for b in range(B):
        last = pos0[b] + Tq - 1
        for p_ in range(max(0, last - W + 1), last + 1):
            ring_k[b, p_ % W] = k[b, p_]
            ring_v[b, p_ % W] = v[b, p_]
    kc, vc = lgsa.hca_compress(to_dev(k), to_dev(v))
    args = (to_dev(q), to_dev(pos0), to_dev(ring_k), to_dev(ring_v), kc, vc)
    lse_g = torch.empty((B, Tq, H), dtype=torch.float32, device="cuda")
    lse_u = torch.empty_like(lse_g)
    out = lgsa.hca_attn_fwd(*args, max_pos=ctx - 1, q_lat=to_dev(ql), w_gate=to_dev(wg),
                            lse=lse_g)
    lgsa.hca_attn_fwd(*args, max_pos=ctx - 1, lse=lse_u)
    torch.cuda.synchronize()
    ref = orc.hca_attn(q, pos0, ring_k, ring_v, orc.hca_compress(k), orc.hca_compress(v),
                       q_lat=ql, w_gate=wg)
    bf16_ok(from_dev(out).reshape(-1, H, 512), ref, "hca gated ring")
    a, u = lse_g.cpu().numpy(), lse_u.cpu().numpy()
    assert np.all(np.isfinite(a))
    np.testing.assert_allclose(a, u, rtol=1e-5, atol=1e-5)


def test_hca_prefill_f32_config0(torch, orc):
    """The tiny fp32 workload: T=1024, 4 heads, 8 compressed entries, gated."""
    x = synth.hca_prefill(0, T=1024, H=4, bf16=False, qkv_scale=1.0)
    kc, vc = lgsa.hca_compress(to_dev(x["k"]), to_dev(x["v"]))
    out = _hca_gpu(x, kc, vc, 1023, True)
    torch.cuda.synchronize()
    ref = orc.hca_attn(x["q"], x["pos0"], x["k"], x["v"], orc.hca_compress(x["k"]),
                       orc.hca_compress(x["v"]), q_lat=x["q_lat"], w_gate=x["w_gate"])
    f32_ok(from_dev(out)[0], ref, "hca f32")


@pytest.mark.parametrize("contexts,gated", [([1000, 130, 5], True), ([131072], False),
                                            ([128, 127, 129, 256], True), ([20, 3], True),
                                            ([300] * 65, True), ([50] * 64, True),
                                            ([100] * 63 + [20], True)])
def test_hca_decode_bf16(torch, orc, contexts, gated):
    """Decode against the oracle.  Gated with at most 64 sequences and at most four key
    splits, the gate kernel merges the splits in its epilogue: one split ([20, 3]), two
    ([50] x 64) and four (63 sequences at 100 and one at 20, whose last splits are empty);
    more splits ([1000, 130, 5], [128, 127, 129, 256]) and 65 sequences take the combine
    kernel, then the gate GEMM."""
    B = len(contexts)
    x = synth.hca_decode(240 + B, B=B, context=max(contexts), H=64, contexts=contexts,
                         gated=gated)
    kc, vc = to_dev(x["kc"]), to_dev(x["vc"])
    out = lgsa.hca_attn_fwd(to_dev(x["q"]), to_dev(x["pos0"]), to_dev(x["k_win"]),
                            to_dev(x["v_win"]), kc if x["kc"].shape[1] else None,
                            vc if x["kc"].shape[1] else None, max_pos=max(contexts) - 1,
                            q_lat=to_dev(x["q_lat"]) if gated else None,
                            w_gate=to_dev(x["w_gate"]) if gated else None)
    torch.cuda.synchronize()
    ref = orc.hca_attn(x["q"], x["pos0"], x["k_win"], x["v_win"],
                       x["kc"] if x["kc"].shape[1] else None,
                       x["vc"] if x["kc"].shape[1] else None,
                       q_lat=x.get("q_lat"), w_gate=x.get("w_gate"))
    bf16_ok(from_dev(out).reshape(B, 64, 512), ref, "hca decode")


def test_hca_deterministic_and_fully_written(torch):
    x = synth.hca_prefill(250, T=600, H=2, bf16=True)
    kc, vc = lgsa.hca_compress(to_dev(x["k"]), to_dev(x["v"]))
    outs = []
    for _ in range(2):
        o = torch.full((1, 600, 2, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        outs.append(_hca_gpu(x, kc, vc, 599, True, dev_out=o))
    torch.cuda.synchronize()
    assert not torch.isnan(outs[0]).any()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


# ------------------------------------------------------------------------------ indexer
def _check_index(orc, x, gpu_idx, k, rows):
    B, Tq = x["q_idx"].shape[:2]
    orc_idx, kth = orc.dsa_topk(x["q_idx"], x["w_idx"], x["k_idx"], x["pos0"], k, rows=rows)
    same = 0
    for j, r in enumerate(rows):
        b, i = divmod(int(r), Tq)
        t = int(x["pos0"][b]) + i
        sc = orc.dsa_scores(x["q_idx"], x["w_idx"], x["k_idx"], b, i, 0, t + 1)
        same += check_topk_row(gpu_idx[b, i], orc_idx[j], t, k, sc, kth[j])
    return same


@pytest.mark.parametrize("T,k", [(3000, 256), (4500, 2048), (700, 1024)])
def test_index_prefill(torch, orc, T, k):
    x = synth.dsa_index(260 + k % 5, B=1, Tq=T, S=T)
    idx = lgsa.dsa_index_topk(to_dev(x["q_idx"]), to_dev(x["w_idx"]), to_dev(x["k_idx"]),
                              to_dev(x["pos0"]), k, max_pos=T - 1)
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    rows = sorted(set([0, 1, k - 2, k - 1, k, k + 1, k + 5, T - 1] +
                      list(np.random.default_rng(1).integers(0, T, 40))))
    rows = [r for r in rows if 0 <= r < T]
    same = _check_index(orc, x, g, k, rows)
    assert same >= len(rows) - 2  # ties straddling the k-th score are rare


def test_index_prefill_small_workspace_chunks(torch, orc):
    """A workspace holding 100 rows of scores forces many query chunks."""
    T, k = 1500, 300
    x = synth.dsa_index(265, B=1, Tq=T, S=T)
    ws = torch.empty(100 * T * 4, dtype=torch.uint8, device="cuda")
    idx = lgsa.dsa_index_topk(to_dev(x["q_idx"]), to_dev(x["w_idx"]), to_dev(x["k_idx"]),
                              to_dev(x["pos0"]), k, max_pos=T - 1, workspace=ws)
    torch.cuda.synchronize()
    _check_index(orc, x, idx.cpu().numpy(), k, [0, 299, 300, 777, 1499])


def test_index_ties_and_zero_scores(torch, orc):
    """Duplicated key rows tie exactly; a query of -0.0 makes every score zero: the lower
    positions must win, bit for bit."""
    T, k = 2500, 2048
    x = synth.dsa_index(266, B=1, Tq=T, S=T)
    x["k_idx"][0, 1::2] = x["k_idx"][0, 0::2][: x["k_idx"][0, 1::2].shape[0]]
    x["q_idx"][0, -5:] = -0.0
    idx = lgsa.dsa_index_topk(to_dev(x["q_idx"]), to_dev(x["w_idx"]), to_dev(x["k_idx"]),
                              to_dev(x["pos0"]), k, max_pos=T - 1)
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    rows = [2048, 2049, 2100, 2200, 2499, 2495]
    orc_idx, kth = orc.dsa_topk(x["q_idx"], x["w_idx"], x["k_idx"], x["pos0"], k, rows=rows)
    for j, r in enumerate(rows):
        if kth[j] == 0.0:  # the boundary lies among exact zeros: the index rule decides alone
            assert g[0, r].tolist() == orc_idx[j].tolist(), r
        else:
            sc = orc.dsa_scores(x["q_idx"], x["w_idx"], x["k_idx"], 0, r, 0, r + 1)
            check_topk_row(g[0, r], orc_idx[j], r, k, sc, kth[j])
    assert g[0, 2499].tolist() == list(range(2048))
    assert kth[rows.index(2499)] == 0.0


def test_index_prefill_long_rows(torch, orc):
    """Rows of more than 65536 positions on the many-query path: their selection runs over the
    scores in global memory rather than from on-chip 16-bit images."""
    S, k, Tq = 70000, 2048, 8
    x = synth.dsa_index(269, B=1, Tq=Tq, S=S, pos0=[S - Tq])
    idx = lgsa.dsa_index_topk(to_dev(x["q_idx"]), to_dev(x["w_idx"]), to_dev(x["k_idx"]),
                              to_dev(x["pos0"]), k, max_pos=S - 1)
    torch.cuda.synchronize()
    same = _check_index(orc, x, idx.cpu().numpy(), k, [0, 3, 7])
    assert same >= 2


def test_index_prefill_tie_group_in_threshold_bin(torch, orc):
    """1500 identical key rows score identically for every query; where the k-th score falls
    among them, the kept members must be the lowest-positioned ones (a prefix of the group)."""
    T, k = 6000, 2048
    x = synth.dsa_index(270, B=1, Tq=T, S=T)
    g0, g1 = 1000, 2500
    x["k_idx"][0, g0:g1] = x["k_idx"][0, g0]
    idx = lgsa.dsa_index_topk(to_dev(x["q_idx"]), to_dev(x["w_idx"]), to_dev(x["k_idx"]),
                              to_dev(x["pos0"]), k, max_pos=T - 1)
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    rows = [2600, 3000, 4000, 5000, 5999] + list(range(2048, 6000, 97))
    same = _check_index(orc, x, g, k, rows)
    assert same >= len(rows) - 2
    straddled = 0
    for r in rows:
        sel = g[0, r][g[0, r] >= 0]
        grp = sel[(sel >= g0) & (sel < g1)]
        assert grp.tolist() == list(range(g0, g0 + len(grp))), r
        straddled += 0 < len(grp) < g1 - g0
    assert straddled > 0  # some row's k-th score lies in the group


@pytest.mark.parametrize("pos0,k", [([39999, 20000, 1500], 2048), ([16383, 16384, 2047], 2048),
                                   ([39999, 33000, 999], 1000)])
def test_index_decode(torch, orc, pos0, k):
    S = 40000
    x = synth.dsa_index(267, B=3, Tq=1, S=S, pos0=pos0)
    idx = lgsa.dsa_index_topk(to_dev(x["q_idx"]), to_dev(x["w_idx"]), to_dev(x["k_idx"]),
                              to_dev(x["pos0"]), k, max_pos=max(pos0))
    torch.cuda.synchronize()
    same = _check_index(orc, x, idx.cpu().numpy(), k, [0, 1, 2])
    assert same >= 2


def test_index_decode_heavy_ties(torch, orc):
    """Row 0 scores every one of 131072 positions exactly 0 (its indexer query is zero), so
    every segment's candidates tie at its k-th key and more candidates survive the merge's
    lower bound than it holds on chip; the lower-index rule alone decides: 0 .. k-1.  Row 1 is
    an ordinary row over the same keys, checked against the oracle."""
    S, k = 131072, 2048
    x = synth.dsa_index(268, B=2, Tq=1, S=S, pos0=[S - 1, S - 1])
    x["q_idx"][0] = 0.0
    idx = lgsa.dsa_index_topk(to_dev(x["q_idx"]), to_dev(x["w_idx"]), to_dev(x["k_idx"]),
                              to_dev(x["pos0"]), k, max_pos=S - 1)
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    assert g[0, 0].tolist() == list(range(k))
    assert _check_index(orc, x, g, k, [1]) >= 0


def test_index_decode_ties_beyond_lds(torch, orc):
    """Row 0 scores all 262144 positions exactly 0: every segment's bound equals every key, so
    all 16 x 2048 segment candidates pass the filter, more than the final selection holds on
    chip, and it selects over global memory: the lower-index rule gives 0 .. k-1.  Row 1 is an
    ordinary row over the same keys, checked against the oracle."""
    S, k = 262144, 2048
    x = synth.dsa_index(269, B=2, Tq=1, S=S, pos0=[S - 1, S - 1])
    x["q_idx"][0] = 0.0
    idx = lgsa.dsa_index_topk(to_dev(x["q_idx"]), to_dev(x["w_idx"]), to_dev(x["k_idx"]),
                              to_dev(x["pos0"]), k, max_pos=S - 1)
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    assert g[0, 0].tolist() == list(range(k))
    assert _check_index(orc, x, g, k, [1]) >= 0


# ------------------------------------------------------------------------------ sparse
@pytest.mark.parametrize("Tq,S,k,distinct_v,gated", [(300, 300, 128, False, True),
                                                     (200, 1000, 96, True, False),
                                                     (70, 70, 100, False, True)])
def test_sparse_prefill(torch, orc, Tq, S, k, distinct_v, gated):
    x = synth.dsa_sparse(270 + k % 3, B=1, Tq=Tq, S=S, H=64, distinct_v=distinct_v,
                         gated=gated)
    pos0 = [S - Tq]
    idx = synth.random_topk(270, 1, Tq, S, k, pos0)
    out = lgsa.sparse_attn_fwd(to_dev(x["q"]), to_dev(x["kv_lat"]), to_dev(idx),
                               v_lat=to_dev(x["v_lat"]) if distinct_v else None,
                               q_lat=to_dev(x["q_lat"]) if gated else None,
                               w_gate=to_dev(x["w_gate"]) if gated else None)
    torch.cuda.synchronize()
    ref = orc.sparse_attn(x["q"], x["kv_lat"], idx, v_lat=x.get("v_lat"),
                          q_lat=x.get("q_lat"), w_gate=x.get("w_gate"))
    bf16_ok(from_dev(out)[0], ref, "sparse")


def test_sparse_decode_split_and_order(torch, orc):
    """Few query rows with long lists are split over workgroups; permuting the list and
    padding it with -1 (and out-of-range entries) changes nothing beyond rounding."""
    B, S, k = 3, 5000, 2048
    x = synth.dsa_sparse(280, B=B, Tq=1, S=S, H=64, gated=True)
    pos0 = [4999, 3000, 100]
    idx = synth.random_topk(280, B, 1, S, k, pos0)
    out = lgsa.sparse_attn_fwd(to_dev(x["q"]), to_dev(x["kv_lat"]), to_dev(idx),
                               q_lat=to_dev(x["q_lat"]), w_gate=to_dev(x["w_gate"]))
    rng = np.random.default_rng(3)
    idx2 = np.concatenate([idx, np.full((B, 1, 64), -1, np.int32)], axis=-1)
    idx2[:, :, -3] = S + 5
    for b in range(B):
        rng.shuffle(idx2[b, 0])
    out2 = lgsa.sparse_attn_fwd(to_dev(x["q"]), to_dev(x["kv_lat"]), to_dev(idx2),
                                q_lat=to_dev(x["q_lat"]), w_gate=to_dev(x["w_gate"]))
    torch.cuda.synchronize()
    ref = orc.sparse_attn(x["q"], x["kv_lat"], idx, q_lat=x["q_lat"], w_gate=x["w_gate"])
    bf16_ok(from_dev(out).reshape(B, 64, 256), ref, "sparse decode")
    bf16_ok(from_dev(out2).reshape(B, 64, 256), ref, "sparse decode permuted")


def test_sparse_empty_rows_are_zero(torch):
    x = synth.dsa_sparse(281, B=1, Tq=3, S=50, H=64, gated=False)
    idx = np.full((1, 3, 40), -1, np.int32)
    idx[0, 1, 5] = 7
    out = lgsa.sparse_attn_fwd(to_dev(x["q"]), to_dev(x["kv_lat"]), to_dev(idx))
    torch.cuda.synchronize()
    o = from_dev(out)
    assert np.all(o[0, 0] == 0) and np.all(o[0, 2] == 0) and np.any(o[0, 1] != 0)


def test_gather_probe_checksums(torch):
    """The measurement helper gathers what the lists name: its checksums (first 64 words of
    the row in slot 32t + 16w of every tile) match a host recomputation, for lists with
    skipped and out-of-range entries and a ragged last tile."""
    S, n_lists, k = 3000, 37, 100
    rng = np.random.default_rng(71)
    rows = rng.integers(0, 2 ** 16, size=(S, 264), dtype=np.uint16)  # stride 264 elements
    idx = rng.integers(-5, S + 5, size=(n_lists, k)).astype(np.int32)
    got = lgsa.sparse_gather_probe(to_dev(rows), to_dev(idx))
    torch.cuda.synchronize()
    got = got.cpu().numpy().view(np.uint32)
    words = rows[:, :128].copy().view(np.uint32)  # [S, 64]
    want = np.zeros((n_lists, 2), np.uint64)
    for l in range(n_lists):
        for t in range((k + 31) // 32):
            for w in range(2):
                j = 32 * t + 16 * w
                s = int(idx[l, j]) if j < k else -1
                s = s if 0 <= s < S else 0
                want[l, w] += int(words[s].astype(np.uint64).sum())
    assert np.array_equal(got.astype(np.uint64), want % (1 << 32))
