"""Pins of the backward oracle (oracle/backward.py) against finite differences of the forward
oracle (oracle.cpp), which it does not share code with: for L = sum(dout * forward(...)), the
central difference of L in each input entry must match the gradient the backward returns.
The forward definitions follow ERNIE 5.5 Flash Base release blog, section 2.1."""
import numpy as np

from oracle import backward


def _fd(f, x, eps=1e-6):
    """Central differences of the scalar f at every entry of x (float64, modified in place)."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        fp = f()
        x[i] = old - eps
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


def test_gate_backward_matches_finite_differences(orc):
    rng = np.random.default_rng(81)
    M, d_lat, N = 3, 4, 5
    q = rng.standard_normal((M, d_lat))
    w = rng.standard_normal((d_lat, N)) * 0.5
    o = rng.standard_normal((M, N))
    dout = rng.standard_normal((M, N))
    loss = lambda: float(np.sum(dout * orc.latent_gate(q, w, o)))
    d_o, dq, dw = backward.latent_gate_bwd(q, w, o, dout)
    assert np.allclose(d_o, _fd(loss, o), rtol=1e-6, atol=1e-8)
    assert np.allclose(dq, _fd(loss, q), rtol=1e-6, atol=1e-8)
    assert np.allclose(dw, _fd(loss, w), rtol=1e-6, atol=1e-8)


def test_gate_backward_zero_latent_is_half_gate():
    """q_lat = 0 gives s = 1/2 everywhere: do = dout / 2 and dG = dout * o / 4, so
    dW = 0 and dq_lat = (dout * o / 4) W^T in closed form."""
    rng = np.random.default_rng(82)
    M, d_lat, N = 4, 3, 6
    w = rng.standard_normal((d_lat, N))
    o, dout = rng.standard_normal((M, N)), rng.standard_normal((M, N))
    d_o, dq, dw = backward.latent_gate_bwd(np.zeros((M, d_lat)), w, o, dout)
    assert np.array_equal(d_o, dout / 2)
    assert np.allclose(dq, (dout * o / 4) @ w.T, rtol=0, atol=1e-14)
    assert np.array_equal(dw, np.zeros((d_lat, N)))


def test_hca_backward_matches_finite_differences(orc):
    """Prefill HCA with the window rows the sequence's own rows and the entries their block
    means (both recomputed from K and V inside the loss), 2 sequences at different positions."""
    rng = np.random.default_rng(83)
    B, T, Tq, H, d, block, window = 2, 11, 5, 2, 4, 4, 3
    pos0 = np.array([T - Tq, T - Tq - 2], np.int32)
    q = rng.standard_normal((B, Tq, H, d))
    k = rng.standard_normal((B, T, d))
    v = rng.standard_normal((B, T, d))
    dout = rng.standard_normal((B, Tq, H, d))

    def loss():
        out = orc.hca_attn(q, pos0, k, v, orc.hca_compress(k, block), orc.hca_compress(v, block),
                           window=window, block=block)
        return float(np.sum(dout.reshape(B * Tq, H, d) * out))

    dq, dk, dv = backward.hca_attn_bwd(q, pos0, k, v, dout, window=window, block=block)
    assert np.allclose(dq, _fd(loss, q), rtol=1e-5, atol=1e-7)
    assert np.allclose(dk, _fd(loss, k), rtol=1e-5, atol=1e-7)
    assert np.allclose(dv, _fd(loss, v), rtol=1e-5, atol=1e-7)


def test_hca_backward_without_a_complete_block(orc):
    """A sequence shorter than a block: only the window path, no entry at all."""
    rng = np.random.default_rng(85)
    B, T, H, d, block, window = 1, 3, 2, 4, 4, 2
    q = rng.standard_normal((B, T, H, d))
    k = rng.standard_normal((B, T, d))
    v = rng.standard_normal((B, T, d))
    dout = rng.standard_normal((B, T, H, d))
    pos0 = np.zeros(B, np.int32)
    loss = lambda: float(np.sum(dout.reshape(B * T, H, d) *
                                orc.hca_attn(q, pos0, k, v, window=window, block=block)))
    dq, dk, dv = backward.hca_attn_bwd(q, pos0, k, v, dout, window=window, block=block)
    assert np.allclose(dq, _fd(loss, q), rtol=1e-5, atol=1e-7)
    assert np.allclose(dk, _fd(loss, k), rtol=1e-5, atol=1e-7)
    assert np.allclose(dv, _fd(loss, v), rtol=1e-5, atol=1e-7)


def test_sparse_backward_matches_finite_differences(orc):
    """Latent rows serving as both keys and values (V = K), with a repeated and a skipped entry
    in the lists; then distinct value rows."""
    rng = np.random.default_rng(84)
    B, Tq, S, H, d, k = 1, 3, 7, 2, 4, 4
    q = rng.standard_normal((B, Tq, H, d))
    lat = rng.standard_normal((B, S, d))
    vl = rng.standard_normal((B, S, d))
    idx = np.array([[[0, 3, 3, -1], [6, 2, 5, 1], [4, 9, 0, 2]]], np.int32)
    dout = rng.standard_normal((B, Tq, H, d))
    loss = lambda: float(np.sum(dout.reshape(B * Tq, H, d) * orc.sparse_attn(q, lat, idx)))
    dq, dlat, none = backward.sparse_attn_bwd(q, lat, idx, dout)
    assert none is None
    assert np.allclose(dq, _fd(loss, q), rtol=1e-5, atol=1e-7)
    assert np.allclose(dlat, _fd(loss, lat), rtol=1e-5, atol=1e-7)
    loss2 = lambda: float(np.sum(dout.reshape(B * Tq, H, d) * orc.sparse_attn(q, lat, idx, vl)))
    dq2, dk2, dv2 = backward.sparse_attn_bwd(q, lat, idx, dout, v_lat=vl)
    assert np.allclose(dq2, _fd(loss2, q), rtol=1e-5, atol=1e-7)
    assert np.allclose(dk2, _fd(loss2, lat), rtol=1e-5, atol=1e-7)
    assert np.allclose(dv2, _fd(loss2, vl), rtol=1e-5, atol=1e-7)


def test_sparse_lse_closed_forms():
    """Equal keys: lse = scale <q, k> + log n (n counts repeats); one key: scale <q, k>; no
    valid entry: -inf; a huge logit does not overflow."""
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 3, 2, 8))
    row = rng.standard_normal(8)
    lat = np.tile(row, (1, 6, 1))
    idx = np.array([[[0, 1, 2, 2, -1], [4, -1, -1, 9, -1], [-1, -1, 6, 7, -3]]], np.int32)
    lse = backward.sparse_attn_lse(q, lat, idx, scale=0.5)
    dot = 0.5 * (q[0] @ row)
    assert np.allclose(lse[0, 0], dot[0] + np.log(4.0), rtol=0, atol=1e-12)
    assert np.allclose(lse[0, 1], dot[1], rtol=0, atol=1e-12)
    assert np.all(lse[0, 2] == -np.inf)
    big = backward.sparse_attn_lse(np.full((1, 1, 1, 2), 300.0), np.ones((1, 2, 2)),
                                   np.array([[[0, 1]]], np.int32), scale=1.0)
    assert np.isclose(big[0, 0, 0], 600.0 + np.log(2.0), rtol=0, atol=1e-9)


def test_sparse_lse_normalises_the_forward(orc):
    """exp(scale <q, K_j> - lse) are the softmax weights of the forward oracle: with V set to
    the identity rows, the forward returns exactly those weights."""
    rng = np.random.default_rng(8)
    S, d = 12, 16
    q = rng.standard_normal((1, 2, 3, d))
    lat = rng.standard_normal((1, S, d))
    idx = np.array([[[0, 3, 5, 11], [2, 2, 7, -1]]], np.int32)
    lse = backward.sparse_attn_lse(q, lat, idx)
    eye = np.zeros((1, S, d))
    eye[0, np.arange(S), np.arange(S)] = 1.0
    out = orc.sparse_attn(q, lat, idx, v_lat=eye)
    for i in range(2):
        w = np.zeros((3, d))
        for s in idx[0, i]:
            if s >= 0:
                w[:, s] += np.exp(q[0, i] @ lat[0, s] / np.sqrt(d) - lse[0, i])
        assert np.allclose(out[i] if out.ndim == 3 else out[0, i], w, rtol=0, atol=1e-12)

