"""GPU parity at the five workload sizes, in the launch configuration bench.py times, against
the fp64 oracle.  Tolerances are stated in tests/helpers.py; every maximum is taken over the
whole compared set.

What is compared:
  - tiny HCA prefill (fp32): every row, every head;
  - model-shape HCA prefill: the compressor's entries in full; the attention output in full
    (every one of the 32768 rows, all 64 heads, every channel; the same shape with unit
    variance inputs on the declared row sample of helpers.declared_rows);
  - HCA decode: all 64 sequences, all heads;
  - DSA prefill: the top-k of every row t = 2040 .. 2180 (the k-th score is exactly 0 there,
    so the lower-index rule decides) plus first/last rows and seeded random rows (about 300);
    sparse attention on the declared row sample of its 65536 rows (about 3500); every row of
    both in test_gpu_full_rows.py, which runs with LGSA_FULL_PARITY=1 (five minutes of oracle);
  - mixed long-context decode: all 8 sequences of every part.
Inputs are the seeded synthetic tensors of each configuration.
"""
import math

import numpy as np
import pytest

import hybrid_sparse_attention_amd as lgsa
from hybrid_sparse_attention_amd import synth

from helpers import (bf16_ok, check_topk_row, declared_rows, f32_ok, from_dev, rows_of,
                     to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lgsa.load()
    return torch


def _rows(T, extra, seed, n_random):
    rng = np.random.default_rng(seed)
    rows = set(r for r in extra if 0 <= r < T)
    rows.update(int(x) for x in rng.integers(0, T, n_random))
    return sorted(rows)


def _report(what, err, tol, n):
    print("%s: %d rows, max|err| %.3g (tol %.3g)" % (what, n, err, tol))


def test_config0_hca_prefill_tiny_fp32(torch, orc):
    """seq 1024, 4 heads, head dim 512, fp32, 8 compressed entries, gated: every row."""
    x = synth.hca_prefill(0, T=1024, H=4, bf16=False)
    kc, vc = lgsa.hca_compress(to_dev(x["k"]), to_dev(x["v"]))
    out = lgsa.hca_attn_fwd(to_dev(x["q"]), to_dev(x["pos0"]), to_dev(x["k"]), to_dev(x["v"]),
                            kc, vc, max_pos=1023, q_lat=to_dev(x["q_lat"]),
                            w_gate=to_dev(x["w_gate"]))
    torch.cuda.synchronize()
    okc, ovc = orc.hca_compress(x["k"]), orc.hca_compress(x["v"])
    f32_ok(from_dev(kc), okc, "compress")
    ref = orc.hca_attn(x["q"], x["pos0"], x["k"], x["v"], okc, ovc, q_lat=x["q_lat"],
                       w_gate=x["w_gate"])
    f32_ok(from_dev(out)[0], ref, "config0")


def test_config1_hca_prefill_model_shape(torch, orc):
    """seq 32768, 64 heads, head dim 512, bf16, inputs N(0,1)/sqrt(512), gated: the entries in
    full and every row of the output (all heads), compared in chunks of 4096 rows as the
    oracle produces them; the tolerance is taken over the whole output tensor."""
    T, H = 32768, 64
    x = synth.hca_prefill(1, T=T, H=H, qkv_scale=1.0 / math.sqrt(512))
    kd, vd = to_dev(x["k"]), to_dev(x["v"])
    kc, vc = lgsa.hca_compress(kd, vd)
    out = lgsa.hca_attn_fwd(to_dev(x["q"]), to_dev(x["pos0"]), kd, vd, kc, vc, max_pos=T - 1,
                            q_lat=to_dev(x["q_lat"]), w_gate=to_dev(x["w_gate"]))
    torch.cuda.synchronize()
    okc, ovc = orc.hca_compress(x["k"]), orc.hca_compress(x["v"])
    bf16_ok(from_dev(kc), okc, "config1 compress k")
    bf16_ok(from_dev(vc), ovc, "config1 compress v")
    err = ref_max = 0.0
    for r0 in range(0, T, 4096):
        rows = np.arange(r0, min(T, r0 + 4096))
        ref = orc.hca_attn(x["q"], x["pos0"], x["k"], x["v"], okc, ovc, q_lat=x["q_lat"],
                           w_gate=x["w_gate"], rows=rows)
        got = from_dev(out[0, r0:r0 + len(rows)])
        assert np.all(np.isfinite(got)), "config1: non-finite output"
        err = max(err, float(np.max(np.abs(got - ref))))
        ref_max = max(ref_max, float(np.max(np.abs(ref))))
    tol = 1e-2 * ref_max + 1e-3
    _report("config1", err, tol, T)
    assert err <= tol, "config1: max|err| %.3g > tol %.3g" % (err, tol)


def test_config1_shape_unit_variance(torch, orc):
    """The model shape with N(0,1) inputs: logits of order 1 make the softmax far from
    uniform, a sharper check than the literal 1/sqrt(512) inputs (an extra, not a config)."""
    T, H = 32768, 64
    x = synth.hca_prefill(101, T=T, H=H, qkv_scale=1.0)
    kd, vd = to_dev(x["k"]), to_dev(x["v"])
    kc, vc = lgsa.hca_compress(kd, vd)
    out = lgsa.hca_attn_fwd(to_dev(x["q"]), to_dev(x["pos0"]), kd, vd, kc, vc, max_pos=T - 1,
                            q_lat=to_dev(x["q_lat"]), w_gate=to_dev(x["w_gate"]))
    torch.cuda.synchronize()
    rows = declared_rows(T, 12, n_random=512, edge=64)
    ref = orc.hca_attn(x["q"], x["pos0"], x["k"], x["v"], orc.hca_compress(x["k"]),
                       orc.hca_compress(x["v"]), q_lat=x["q_lat"], w_gate=x["w_gate"],
                       rows=rows)
    err, tol = bf16_ok(rows_of(out, rows), ref, "config1 unit variance")
    _report("config1 unit variance", err, tol, len(rows))


def test_config2_hca_decode(torch, orc):
    """64 sequences, context 131072: 1024 compressed entries + 128-row ring, 64 heads, gated;
    every sequence compared."""
    B, ctx, H = 64, 131072, 64
    x = synth.hca_decode(2, B=B, context=ctx, H=H)
    out = lgsa.hca_attn_fwd(to_dev(x["q"]), to_dev(x["pos0"]), to_dev(x["k_win"]),
                            to_dev(x["v_win"]), to_dev(x["kc"]), to_dev(x["vc"]),
                            max_pos=ctx - 1, q_lat=to_dev(x["q_lat"]),
                            w_gate=to_dev(x["w_gate"]))
    torch.cuda.synchronize()
    ref = orc.hca_attn(x["q"], x["pos0"], x["k_win"], x["v_win"], x["kc"], x["vc"],
                       q_lat=x["q_lat"], w_gate=x["w_gate"])
    err, tol = bf16_ok(from_dev(out).reshape(B, H, 512), ref, "config2")
    _report("config2", err, tol, B)


@pytest.fixture(scope="module")
def config3(torch):
    T = 65536
    xi = synth.dsa_index(3, B=1, Tq=T, S=T)
    xs = synth.dsa_sparse(3, B=1, Tq=T, S=T, H=64)
    return T, xi, xs


def test_config3_indexer_topk(torch, orc, config3):
    """seq 65536, indexer 4 heads x 64 fp32, top-2048: every row t = 2040 .. 2180 (where the
    k-th score is exactly 0 and the lower-index rule decides bit for bit), the first and last
    rows and seeded random rows, against the oracle's selection (identical sets, or
    differences only inside the tie band)."""
    T, xi, _ = config3
    k = 2048
    idx = lgsa.dsa_index_topk(to_dev(xi["q_idx"]), to_dev(xi["w_idx"]), to_dev(xi["k_idx"]),
                              to_dev(xi["pos0"]), k, max_pos=T - 1)
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    extra = list(range(0, 16)) + list(range(2040, 2181)) + list(range(T - 16, T))
    rows = _rows(T, extra + [4095, 4096, 32767, 32768], 13, 120)
    orc_idx, kth = orc.dsa_topk(xi["q_idx"], xi["w_idx"], xi["k_idx"], xi["pos0"], k, rows=rows)
    same = diff = outside_abs = zero_kth = 0
    for j, r in enumerate(rows):
        sc = orc.dsa_scores(xi["q_idx"], xi["w_idx"], xi["k_idx"], 0, r, 0, r + 1)
        res = check_topk_row(g[0, r], orc_idx[j], r, k, sc, kth[j])
        same += res.same
        diff += res.n_diff
        outside_abs += res.outside_abs
        if kth[j] == 0.0:
            zero_kth += 1
            assert res.same, "row %d: the exact-zero threshold must select bit for bit" % r
    print("config3 top-k: %d rows (%d with an exactly zero k-th score), %d identical, %d "
          "differing positions (all inside the relative band; %d outside the absolute 1e-5 "
          "band)" % (len(rows), zero_kth, same, diff, outside_abs))
    assert zero_kth >= 50
    assert same >= len(rows) - 8


def test_config3_sparse_attention(torch, orc, config3):
    """seq 65536, 64 heads, d 256, V = K, top-2048 lists (seeded stratified selection), gated:
    the declared row sample (about 3500 rows), all heads."""
    T, _, xs = config3
    k = 2048
    idx = synth.stratified_topk(3, 1, T, T, k, [0])
    out = lgsa.sparse_attn_fwd(to_dev(xs["q"]), to_dev(xs["kv_lat"]), to_dev(idx),
                               q_lat=to_dev(xs["q_lat"]), w_gate=to_dev(xs["w_gate"]))
    torch.cuda.synchronize()
    rows = declared_rows(T, 14)
    ref = orc.sparse_attn(xs["q"], xs["kv_lat"], idx, q_lat=xs["q_lat"], w_gate=xs["w_gate"],
                          rows=rows)
    err, tol = bf16_ok(rows_of(out, rows), ref, "config3 sparse")
    _report("config3 sparse", err, tol, len(rows))


def test_config3_chain(torch, orc, config3):
    """Indexer then sparse attention on the GPU, against the oracle's own chain, on sampled
    rows whose selected sets agree (the rest differ only inside the tie band)."""
    T, xi, xs = config3
    k = 2048
    idx = lgsa.dsa_index_topk(to_dev(xi["q_idx"]), to_dev(xi["w_idx"]), to_dev(xi["k_idx"]),
                              to_dev(xi["pos0"]), k, max_pos=T - 1)
    out = lgsa.sparse_attn_fwd(to_dev(xs["q"]), to_dev(xs["kv_lat"]), idx,
                               q_lat=to_dev(xs["q_lat"]), w_gate=to_dev(xs["w_gate"]))
    torch.cuda.synchronize()
    rows = _rows(T, [5, 2048, 40000, 65535], 15, 4)
    orc_idx, _ = orc.dsa_topk(xi["q_idx"], xi["w_idx"], xi["k_idx"], xi["pos0"], k, rows=rows)
    g = idx.cpu().numpy()[0]
    agree = [r for j, r in enumerate(rows) if set(g[r]) == set(orc_idx[j])]
    assert len(agree) >= len(rows) - 1
    full_idx = np.full((1, T, k), -1, np.int32)
    for j, r in enumerate(rows):
        full_idx[0, r] = orc_idx[j]
    ref = orc.sparse_attn(xs["q"], xs["kv_lat"], full_idx, q_lat=xs["q_lat"],
                          w_gate=xs["w_gate"], rows=agree)
    bf16_ok(from_dev(out)[0][agree], ref, "config3 chain")


def test_config4_mixed_long_context_decode(torch, orc):
    """8 sequences at context 1,048,576: HCA decode over 8192 entries + 128 ring (d 512), the
    indexer over 1,048,576 fp32 keys with top-2048, then sparse attention (d 256) over the
    selected bf16 latent rows; 64 heads; both layers gated."""
    B, ctx, H, k = 8, 1 << 20, 64, 2048
    xh = synth.hca_decode(4, B=B, context=ctx, H=H)
    out_h = lgsa.hca_attn_fwd(to_dev(xh["q"]), to_dev(xh["pos0"]), to_dev(xh["k_win"]),
                              to_dev(xh["v_win"]), to_dev(xh["kc"]), to_dev(xh["vc"]),
                              max_pos=ctx - 1, q_lat=to_dev(xh["q_lat"]),
                              w_gate=to_dev(xh["w_gate"]))
    torch.cuda.synchronize()
    ref_h = orc.hca_attn(xh["q"], xh["pos0"], xh["k_win"], xh["v_win"], xh["kc"], xh["vc"],
                         q_lat=xh["q_lat"], w_gate=xh["w_gate"])
    err, tol = bf16_ok(from_dev(out_h).reshape(B, H, 512), ref_h, "config4 hca")
    _report("config4 hca", err, tol, B)
    del xh

    xi = synth.dsa_index(4, B=B, Tq=1, S=ctx, pos0=[ctx - 1] * B)
    idx = lgsa.dsa_index_topk(to_dev(xi["q_idx"]), to_dev(xi["w_idx"]), to_dev(xi["k_idx"]),
                              to_dev(xi["pos0"]), k, max_pos=ctx - 1)
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    orc_idx, kth = orc.dsa_topk(xi["q_idx"], xi["w_idx"], xi["k_idx"], xi["pos0"], k)
    same = outside_abs = 0
    for b in range(B):
        sc = orc.dsa_scores(xi["q_idx"], xi["w_idx"], xi["k_idx"], b, 0, 0, ctx)
        res = check_topk_row(g[b, 0], orc_idx[b], ctx - 1, k, sc, kth[b])
        same += res.same
        outside_abs += res.outside_abs
    print("config4 top-k: %d of %d sequences identical; %d differing positions outside the "
          "absolute 1e-5 band" % (same, B, outside_abs))
    assert same >= B - 1
    del xi

    xs = synth.dsa_sparse(4, B=B, Tq=1, S=ctx, H=H, qname="q_dsa", latname="q_lat_dsa",
                          wname="w_gate_dsa")
    sel = orc_idx.reshape(B, 1, k)  # the oracle's selection feeds both sides
    out_s = lgsa.sparse_attn_fwd(to_dev(xs["q"]), to_dev(xs["kv_lat"]), to_dev(sel),
                                 q_lat=to_dev(xs["q_lat"]), w_gate=to_dev(xs["w_gate"]))
    torch.cuda.synchronize()
    ref_s = orc.sparse_attn(xs["q"], xs["kv_lat"], sel, q_lat=xs["q_lat"], w_gate=xs["w_gate"])
    err, tol = bf16_ok(from_dev(out_s).reshape(B, H, 256), ref_s, "config4 sparse")
    _report("config4 sparse", err, tol, B)
