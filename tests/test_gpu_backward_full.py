"""The backward calls at the model shapes bench.py times, in the same launch configuration,
against the float64 backward oracle on sampled outputs that it can compute one by one (chain
rule of the forward definitions; ERNIE 5.5 Flash Base release blog, section 2.1).

- a gradient row of a query (dq, d_o, dq_lat) depends on that row's inputs only, so the
  oracle runs on that row alone;
- a column of dW_gate depends on that column of the gate only;
- the raw-key gradients of HCA positions in the last block come from the last 128 query rows
  only (their window, and the last block's entry, which only the last row sees);
- the latent-row gradient of a sparse-attention key comes from the rows whose lists hold it,
  which are few for late keys.

Inputs are seeded normal draws made on the device by torch (rounded to bfloat16), with the
bench's scales; the sparse lists are stratified draws (one position per stratum of [0, t])."""
import math

import numpy as np
import pytest

import hybrid_sparse_attention_amd as lgsa
from oracle import backward

from helpers import bf16_ok, from_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lgsa.load()
    return torch


def _randn(torch, g, shape, scale=1.0):
    return (torch.randn(*shape, device="cuda", generator=g) * scale).to(torch.bfloat16)


def _bits(torch, t):
    """bfloat16 device tensor -> its bits on the host (the oracle reads bfloat16 bits)."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def test_gate_backward_model_shape(torch):
    """32768 rows x 32768 channels, d_lat 1024 (the HCA prefill gate): sampled rows of d_o and
    dq_lat, sampled columns of dW_gate."""
    M, N, d_lat = 32768, 32768, 1024
    g = torch.Generator(device="cuda").manual_seed(21)
    q = _randn(torch, g, (M, d_lat))
    w = _randn(torch, g, (d_lat, N), 0.02)
    o = _randn(torch, g, (M, N))
    dout = _randn(torch, g, (M, N))
    d_o, dq, dw = lgsa.latent_gate_bwd(q, w, o, dout)
    torch.cuda.synchronize()
    wb = _bits(torch, w)
    rows = [0, 1, 12345, M - 1]
    r_o, r_q, _ = backward.latent_gate_bwd(_bits(torch, q[rows]), wb, _bits(torch, o[rows]),
                                           _bits(torch, dout[rows]))
    bf16_ok(from_dev(d_o[rows]), r_o, "d_o rows")
    bf16_ok(from_dev(dq[rows]), r_q, "dq_lat rows")
    cols = [0, 777, N - 1]
    _, _, r_w = backward.latent_gate_bwd(_bits(torch, q), wb[:, cols], _bits(torch, o[:, cols]),
                                         _bits(torch, dout[:, cols]))
    bf16_ok(from_dev(dw[:, cols]), r_w, "dW_gate columns")
    del q, w, o, dout, d_o, dq, dw
    torch.cuda.empty_cache()


def test_hca_backward_model_shape(torch):
    """seq 32768, 64 heads, head dim 512, 128-token blocks and window, q, k, v ~ N(0,1)/sqrt(512)
    and dO ~ N(0,1): dq of sampled rows; dk, dv of the last block's positions."""
    T, H, d, blk = 32768, 64, 512, 128
    g = torch.Generator(device="cuda").manual_seed(22)
    sc = 1.0 / math.sqrt(d)
    q = _randn(torch, g, (1, T, H, d), sc)
    k = _randn(torch, g, (1, T, d), sc)
    v = _randn(torch, g, (1, T, d), sc)
    dout = _randn(torch, g, (1, T, H, d))
    kc, vc = lgsa.hca_compress(k, v, block=blk)
    lse = torch.empty(1, T, H, dtype=torch.float32, device="cuda")
    pos0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = lgsa.hca_attn_fwd(q, pos0, k, v, kc, vc, max_pos=T - 1, window=blk, block=blk, lse=lse)
    dq, dk, dv = lgsa.hca_attn_bwd(q, k, v, kc, vc, out, lse, dout, window=blk, block=blk)
    torch.cuda.synchronize()
    kb, vb = _bits(torch, k), _bits(torch, v)
    for t in (0, 127, 128, 5000, T - 1):
        r_q, _, _ = backward.hca_attn_bwd(_bits(torch, q[:, t:t + 1]), np.array([t]), kb, vb,
                                          _bits(torch, dout[:, t:t + 1]), window=blk, block=blk)
        bf16_ok(from_dev(dq[:, t:t + 1]), r_q, "dq row %d" % t)
    t0 = T - blk
    _, r_k, r_v = backward.hca_attn_bwd(_bits(torch, q[:, t0:]), np.array([t0]), kb, vb,
                                        _bits(torch, dout[:, t0:]), window=blk, block=blk)
    bf16_ok(from_dev(dk[:, t0:]), r_k[:, t0:], "dk of the last block")
    bf16_ok(from_dev(dv[:, t0:]), r_v[:, t0:], "dv of the last block")
    del q, k, v, dout, out, dq, dk, dv, lse, kc, vc
    torch.cuda.empty_cache()


def test_sparse_backward_model_shape(torch):
    """seq 65536, top-2048 stratified lists, 64 heads, d 256, latent rows as keys and values,
    all N(0,1): dq of sampled rows; the latent-row gradients of late keys (every row that lists
    them, found on the host).  The default workspace takes the rows in several chunks."""
    T, H, d, k = 65536, 64, 256, 2048
    g = torch.Generator(device="cuda").manual_seed(23)
    q = _randn(torch, g, (1, T, H, d))
    lat = _randn(torch, g, (1, T, d))
    dout = _randn(torch, g, (1, T, H, d))
    t = torch.arange(T, device="cuda", dtype=torch.float64).view(T, 1) + 1.0
    j = torch.arange(k, device="cuda", dtype=torch.float64).view(1, k)
    u = torch.rand(T, k, device="cuda", generator=g, dtype=torch.float64)
    strat = torch.floor((j + u) * t / k)
    idx = torch.where(t > k, strat, torch.where(j < t, j, torch.full_like(j, -1.0)))
    idx = idx.to(torch.int32).view(1, T, k).contiguous()
    del t, j, u, strat
    lse = torch.empty(1, T, H, dtype=torch.float32, device="cuda")
    out = lgsa.sparse_attn_fwd(q, lat, idx, lse=lse)
    dq, dk, _ = lgsa.sparse_attn_bwd(q, lat, idx, out, lse, dout)
    torch.cuda.synchronize()
    latb = _bits(torch, lat)
    ix = idx.cpu().numpy()
    rows = [0, 2047, 2048, 40000, T - 1]
    r_q, _, _ = backward.sparse_attn_bwd(_bits(torch, q[:, rows]), latb, ix[:, rows],
                                         _bits(torch, dout[:, rows]))
    bf16_ok(from_dev(dq[:, rows]), r_q, "dq rows")
    for s in (T - 1, 65000, 63000):
        lst = np.nonzero((ix[0] == s).any(axis=1))[0]
        if len(lst) == 0:  # no row lists it: zero gradient
            assert np.all(from_dev(dk[:, s:s + 1]) == 0)
            continue
        _, r_k, _ = backward.sparse_attn_bwd(_bits(torch, q[:, lst]), latb, ix[:, lst],
                                             _bits(torch, dout[:, lst]))
        bf16_ok(from_dev(dk[:, s:s + 1]), r_k[:, s:s + 1], "dk of key %d (%d rows)" % (s, len(lst)))
    del q, lat, dout, out, dq, dk, lse, idx
    torch.cuda.empty_cache()
