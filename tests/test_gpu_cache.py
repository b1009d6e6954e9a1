"""GPU parity of the decode-time cache appends (hca_cache_append, dsa_cache_append) against
the NumPy oracle in oracle/cache.py, and the property that makes them useful: a sequence
appended token by token ends with exactly the caches a prefill builds (the compressor's
entries bit for bit, the ring holding the last window of raw rows), and decode attention over
them matches the oracle's attention over the whole history.  ERNIE 5.5 Flash Base release
blog, section 2.1; 128-token window from the xenospectrum.com article."""
import math

import numpy as np
import pytest

import hybrid_sparse_attention_amd as lgsa
import oracle
from hybrid_sparse_attention_amd import synth
from oracle import cache as oc

from helpers import bf16_ok, f32_ok, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lgsa.load()
    return torch


@pytest.mark.parametrize("bf16", [True, False])
def test_hca_append_parity(torch, bf16):
    B, d, W, n_cap, block = 6, 512, 128, 8, 128
    # mid-block, first block's last token, a later block's last token, mid-block, a completed
    # block beyond the capacity, no new token
    pos = np.array([57, 127, 383, 1000, 128 * n_cap + 127, -1], dtype=np.int32)
    kw = synth.normal(300, (B, W, d), 1.0, bf16)
    vw = synth.normal(301, (B, W, d), 1.0, bf16)
    kc = synth.normal(302, (B, n_cap, d), 1.0, bf16)
    vc = synth.normal(303, (B, n_cap, d), 1.0, bf16)
    kn = synth.normal(304, (B, d), 1.0, bf16)
    vn = synth.normal(305, (B, d), 1.0, bf16)
    dkw, dvw, dkc, dvc = to_dev(kw), to_dev(vw), to_dev(kc), to_dev(vc)
    lgsa.hca_cache_append(to_dev(pos), to_dev(kn), to_dev(vn), dkw, dvw, dkc, dvc, block=block)
    torch.cuda.synchronize()
    rkw, rvw, rkc, rvc = oc.hca_cache_append(pos, kn, vn, kw, vw, kc, vc, block=block)
    assert np.array_equal(from_dev(dkw), rkw) and np.array_equal(from_dev(dvw), rvw)
    written = [(1, 0), (2, 2)]
    ok = bf16_ok if bf16 else f32_ok
    for dev, ref, init in ((dkc, rkc, kc), (dvc, rvc, vc)):
        got = from_dev(dev)
        keep = np.ones((B, n_cap), bool)
        for b, e in written:
            keep[b, e] = False
            ok(got[b, e], ref[b, e], "entry (%d, %d)" % (b, e))
        assert np.array_equal(got[keep], oc._f64(init)[keep]), "entries not completed changed"


def test_hca_append_sequence_rebuilds_prefill_caches_and_decodes(torch, orc):
    B, T, d, W, n_cap, H, block = 2, 700, 512, 128, 8, 64, 128
    lag = 37  # sequence 1 starts `lag` calls later (its negative positions are skipped)
    K = synth.normal(310, (B, T, d), 1.0 / math.sqrt(512), True)
    V = synth.normal(311, (B, T, d), 1.0 / math.sqrt(512), True)
    dK, dV = to_dev(K), to_dev(V)
    kw = torch.zeros((B, W, d), dtype=torch.bfloat16, device="cuda")
    vw, kc, vc = torch.zeros_like(kw), torch.zeros((B, n_cap, d), dtype=torch.bfloat16,
                                                    device="cuda"), None
    vc = torch.zeros_like(kc)
    for t in range(T):
        p = [t, t - lag]
        rows = [p[0], max(p[1], 0)]
        kn = torch.stack([dK[0, rows[0]], dK[1, rows[1]]])
        vn = torch.stack([dV[0, rows[0]], dV[1, rows[1]]])
        pos = torch.tensor(p, dtype=torch.int32, device="cuda")
        lgsa.hca_cache_append(pos, kn, vn, kw, vw, kc, vc, block=block)
    torch.cuda.synchronize()
    gkw, gvw, gkc, gvc = from_dev(kw), from_dev(vw), from_dev(kc), from_dev(vc)
    for b, n in enumerate([T, T - lag]):
        ref_kc, ref_vc = lgsa.hca_compress(dK[b:b + 1, :n], dV[b:b + 1, :n], block=block)
        ne = n // block
        assert np.array_equal(gkc[b, :ne], from_dev(ref_kc)[0]), "entries differ from prefill"
        assert np.array_equal(gvc[b, :ne], from_dev(ref_vc)[0])
        assert not gkc[b, ne:].any() and not gvc[b, ne:].any()
        Kb, Vb = synth.bf16_to_f32(K[b]), synth.bf16_to_f32(V[b])
        for p in range(n - W, n):
            assert np.array_equal(gkw[b, p % W], Kb[p]) and np.array_equal(gvw[b, p % W], Vb[p])
    # decode attention of each sequence's last token over the maintained caches
    q = synth.normal(312, (B, 1, H, d), 1.0, True)
    pos0 = np.array([T - 1, T - 1 - lag], dtype=np.int32)
    out = lgsa.hca_attn_fwd(to_dev(q), to_dev(pos0), kw, vw, kc, vc, max_pos=T - 1)
    torch.cuda.synchronize()
    ref = orc.hca_attn(q, pos0, K, V, orc.hca_compress(K), orc.hca_compress(V))
    bf16_ok(from_dev(out).reshape(ref.shape), ref, "decode over appended caches")


def test_dsa_append_parity_and_sequence(torch):
    B, S, di, row, stride = 3, 300, 64, 256, 320
    ki = synth.normal(320, (B, S, di))
    kv = synth.normal(321, (B, S, stride), 1.0, True)
    kin = synth.normal(322, (B, di))
    kvn = synth.normal(323, (B, row), 1.0, True)
    pos = np.array([17, -1, S - 1], dtype=np.int32)
    dki, dkv = to_dev(ki), to_dev(kv)
    lgsa.dsa_cache_append(to_dev(pos), to_dev(kin), dki, to_dev(kvn), dkv)
    torch.cuda.synchronize()
    rki, rkv = oc.dsa_cache_append(pos, kin, ki, kvn, kv)
    assert np.array_equal(from_dev(dki), rki) and np.array_equal(from_dev(dkv), rkv)
    # a whole sequence appended call by call equals the tensors it came from
    KI = to_dev(synth.normal(324, (B, S, di)))
    KV = to_dev(synth.normal(325, (B, S, row), 1.0, True))
    dki = torch.zeros_like(KI)
    dkv = torch.zeros((B, S, stride), dtype=torch.bfloat16, device="cuda")
    for t in range(S):
        p = torch.full((B,), t, dtype=torch.int32, device="cuda")
        lgsa.dsa_cache_append(p, KI[:, t].contiguous(), dki, KV[:, t].contiguous(), dkv)
    torch.cuda.synchronize()
    assert torch.equal(dki, KI) and torch.equal(dkv[:, :, :row], KV)
    assert not dkv[:, :, row:].any()
