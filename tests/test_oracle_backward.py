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
