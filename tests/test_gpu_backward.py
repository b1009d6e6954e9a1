"""Backward of the gate on the GPU against the NumPy float64 backward oracle (chain rule of the
forward definitions; ERNIE 5.5 Flash Base release blog, section 2.1 for the gate)."""
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
