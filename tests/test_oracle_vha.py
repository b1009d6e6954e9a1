"""Pins of the VHA oracle (oracle/vha.py) against things it does not compute itself: a dense
per-element evaluation of out = (I + U V^T) o over the heads, the identity skip when a factor is
zero, a rank-1 case in closed form, and equivariance under a permutation of the heads.
ERNIE 5.5 Flash Base release blog, section 2.1 (a low-rank cross-head mix with an identity
skip connection, after attention)."""
import numpy as np

from oracle import vha


def test_matches_dense_mixing_matrix():
    rng = np.random.default_rng(11)
    M, H, d, r = 3, 6, 5, 2
    o, u, v = rng.standard_normal((M, H, d)), rng.standard_normal((H, r)), rng.standard_normal((H, r))
    A = np.eye(H)
    for h in range(H):
        for h2 in range(H):
            A[h, h2] += sum(u[h, k] * v[h2, k] for k in range(r))
    ref = np.zeros((M, H, d))
    for m in range(M):
        for h in range(H):
            for j in range(d):
                ref[m, h, j] = sum(A[h, h2] * o[m, h2, j] for h2 in range(H))
    assert np.allclose(vha.vha_mix(o, u, v), ref, rtol=0, atol=1e-12)


def test_zero_factor_is_the_identity_skip():
    rng = np.random.default_rng(12)
    o, v = rng.standard_normal((4, 8, 16)), rng.standard_normal((8, 3))
    assert np.array_equal(vha.vha_mix(o, np.zeros((8, 3)), v), o)


def test_rank_one_unit_factors_add_one_head_to_another():
    rng = np.random.default_rng(13)
    H, a, b = 8, 2, 5
    o = rng.standard_normal((3, H, 7))
    u, v = np.zeros((H, 1)), np.zeros((H, 1))
    u[a, 0], v[b, 0] = 1.0, 1.0
    out = vha.vha_mix(o, u, v)
    expect = o.copy()
    expect[:, a] += o[:, b]
    assert np.array_equal(out, expect)


def test_head_permutation_equivariance():
    rng = np.random.default_rng(14)
    M, H, d, r = 2, 9, 4, 3
    o, u, v = rng.standard_normal((M, H, d)), rng.standard_normal((H, r)), rng.standard_normal((H, r))
    perm = rng.permutation(H)
    assert np.allclose(vha.vha_mix(o[:, perm], u[perm], v[perm]), vha.vha_mix(o, u, v)[:, perm],
                       rtol=0, atol=1e-12)


def test_bf16_bits_widen_exactly():
    o = np.array([[[0x3F80], [0x4000]]], dtype=np.uint16)  # heads 1.0 and 2.0
    u = np.array([[0x3F80], [0x0000]], dtype=np.uint16)     # u = [1, 0]
    v = np.array([[0x0000], [0x3F00]], dtype=np.uint16)     # v = [0, 0.5]
    assert vha.vha_mix(o, u, v)[0, :, 0].tolist() == [2.0, 2.0]
