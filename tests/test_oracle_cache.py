"""Pins of the decode-time cache oracle (oracle/cache.py) against things it does not compute
itself: appending a sequence token by token must rebuild the prefill compressor's entries
(computed by the separate C++ oracle) and leave the ring holding the last win_len tokens;
ERNIE 5.5 Flash Base release blog, section 2.1 (one entry per completed block of 128 tokens,
a window of recent raw tokens)."""
import numpy as np

import oracle
from oracle import cache as oc


def _rand(rng, shape):
    return rng.standard_normal(shape)


def _append_all(K, V, W, n_cap, block, offsets):
    B, T, d = K.shape
    kw = np.zeros((B, W, d))
    vw = np.zeros((B, W, d))
    kc = np.zeros((B, n_cap, d))
    vc = np.zeros((B, n_cap, d))
    for t in range(T):
        pos = np.array([t - o for o in offsets])
        kn = np.stack([K[b, max(p, 0)] for b, p in enumerate(pos)])
        vn = np.stack([V[b, max(p, 0)] for b, p in enumerate(pos)])
        kw, vw, kc, vc = oc.hca_cache_append(pos, kn, vn, kw, vw, kc, vc, block=block)
    return kw, vw, kc, vc


def test_sequential_appends_rebuild_the_compressor():
    rng = np.random.default_rng(5)
    B, T, d, W, block = 2, 700, 24, 128, 128
    K, V = _rand(rng, (B, T, d)), _rand(rng, (B, T, d))
    offsets = [0, 37]  # sequence 1 starts 37 calls later (negative positions are skipped)
    kw, vw, kc, vc = _append_all(K, V, W, n_cap=8, block=block, offsets=offsets)
    for b, off in enumerate(offsets):
        n = T - off  # tokens appended to sequence b
        ref_k = oracle.hca_compress(K[b:b + 1, :n], block)[0]
        ref_v = oracle.hca_compress(V[b:b + 1, :n], block)[0]
        ne = n // block
        assert np.allclose(kc[b, :ne], ref_k, rtol=0, atol=1e-12)
        assert np.allclose(vc[b, :ne], ref_v, rtol=0, atol=1e-12)
        assert not kc[b, ne:].any() and not vc[b, ne:].any()  # incomplete blocks: no entry
        for p in range(n - W, n):  # the ring holds the last W positions
            assert np.array_equal(kw[b, p % W], K[b, p]) and np.array_equal(vw[b, p % W], V[b, p])


def test_block_completion_without_room_and_negative_positions():
    rng = np.random.default_rng(6)
    B, d, W, block = 3, 8, 16, 16
    kw, vw = _rand(rng, (B, W, d)), _rand(rng, (B, W, d))
    kc, vc = _rand(rng, (B, 2, d)), _rand(rng, (B, 2, d))
    kn, vn = _rand(rng, (B, d)), _rand(rng, (B, d))
    pos = np.array([47, -3, 31])  # 47: entry 2 is not held; -3: skipped; 31: entry 1 written
    kw2, vw2, kc2, vc2 = oc.hca_cache_append(pos, kn, vn, kw, vw, kc, vc, block=block)
    assert np.array_equal(kc2[0], kc[0]) and np.array_equal(kw2[0, 47 % W], kn[0])
    assert np.array_equal(kw2[1], kw[1]) and np.array_equal(kc2[1], kc[1])
    rows = [kw[2, p % W] for p in range(16, 31)] + [kn[2]]
    assert np.allclose(kc2[2, 1], np.mean(rows, axis=0), rtol=0, atol=1e-14)
    assert np.array_equal(kc2[2, 0], kc[2, 0])


def test_bf16_inputs_widen_exactly():
    x = np.array([[0x3F80, 0xC040, 0x0000, 0x8000]], dtype=np.uint16)  # 1, -3, +0, -0
    kw, _, _, _ = oc.hca_cache_append(np.array([2]), x, x, np.zeros((1, 4, 4), np.uint16),
                                      np.zeros((1, 4, 4), np.uint16), block=4)
    assert kw[0, 2].tolist() == [1.0, -3.0, 0.0, -0.0]


def test_dsa_sequential_appends_rebuild_the_caches():
    rng = np.random.default_rng(7)
    B, S, di, row, stride = 2, 50, 8, 16, 24
    KI, KV = _rand(rng, (B, S, di)), _rand(rng, (B, S, row))
    ki, kv = np.zeros((B, S, di)), np.zeros((B, S, stride))
    for t in range(S + 5):  # sequence 1 trails by 5; positions >= S are skipped
        pos = np.array([t, t - 5])
        kin = np.stack([KI[b, min(max(p, 0), S - 1)] for b, p in enumerate(pos)])
        kvn = np.stack([KV[b, min(max(p, 0), S - 1)] for b, p in enumerate(pos)])
        ki, kv = oc.dsa_cache_append(pos, kin, ki, kvn, kv)
    assert np.array_equal(ki, KI)
    assert np.array_equal(kv[:, :, :row], KV) and not kv[:, :, row:].any()
