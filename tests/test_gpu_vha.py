"""GPU parity of vha_mix (the Virtual Head Attention mixing step, ERNIE 5.5 Flash Base release
blog, section 2.1) against the NumPy oracle in oracle/vha.py.  The factors are scaled so that
the cross-head term is as large as the skip term: with the small weights of a trained layer
the check would barely see the mix.  Tolerances are stated in tests/helpers.py."""
import numpy as np
import pytest

import hybrid_sparse_attention_amd as lgsa
from hybrid_sparse_attention_amd import synth
from oracle import vha

from helpers import bf16_ok, f32_ok, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lgsa.load()
    return torch


@pytest.mark.parametrize("M,d,r,inplace", [(37, 512, 16, True), (50, 256, 5, False),
                                           (1, 1024, 1, False), (300, 512, 16, False)])
def test_vha_bf16(torch, M, d, r, inplace):
    H = 64
    o = synth.normal(400 + r, (M, H, d), 1.0, True)
    u = synth.normal(401 + r, (H, r), 0.25, True)
    v = synth.normal(402 + r, (H, r), 0.25, True)
    od = to_dev(o)
    out = lgsa.vha_mix(od, to_dev(u), to_dev(v), out=od if inplace else None)
    torch.cuda.synchronize()
    ref = vha.vha_mix(o, u, v)
    assert np.abs(ref - vha._f64(o)).max() > 0.5 * np.abs(ref).max() * 0.1  # the mix matters
    bf16_ok(from_dev(out), ref, "vha bf16")


@pytest.mark.parametrize("M,H,d,r", [(20, 4, 64, 3), (3, 64, 40, 16), (5, 7, 9, 1)])
def test_vha_f32(torch, M, H, d, r):
    o = synth.normal(410 + H, (M, H, d))
    u = synth.normal(411 + H, (H, r), 0.25)
    v = synth.normal(412 + H, (H, r), 0.25)
    out = lgsa.vha_mix(to_dev(o), to_dev(u), to_dev(v))
    torch.cuda.synchronize()
    f32_ok(from_dev(out), vha.vha_mix(o, u, v), "vha f32")


def test_vha_zero_factor_is_exact_identity_and_deterministic(torch):
    M, H, d, r = 9, 64, 512, 16
    o = to_dev(synth.normal(420, (M, H, d), 1.0, True))
    v = to_dev(synth.normal(421, (H, r), 0.25, True))
    out = lgsa.vha_mix(o, torch.zeros((H, r), dtype=torch.bfloat16, device="cuda"), v)
    assert torch.equal(out, o)  # z U^T adds exactly 0, so o passes through bit for bit
    u = to_dev(synth.normal(422, (H, r), 0.25, True))
    a = lgsa.vha_mix(o, u, v)
    b = lgsa.vha_mix(o, u, v)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
