"""The allocation-free entry point hca_attn_fwd_static, through the C ABI, against
hca_attn_fwd with a caller workspace: same kernels and plan, so the outputs must be
bit-identical (inside the bfloat16 tolerance of the other parity tests a fortiori).  Two
decode calls in a row share the static scratch, the second with a smaller input (fewer
sequences and a shorter context, so fewer and shorter splits), then a prefill call that needs
no scratch.
"""
import numpy as np
import pytest

import hybrid_sparse_attention_amd as lgsa
from hybrid_sparse_attention_amd import synth

from helpers import bf16_ok, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lgsa.load()
    return torch


def _decode(torch, seed, B, contexts):
    x = synth.hca_decode(seed, B=B, context=max(contexts), H=64, contexts=contexts)
    d = {k: to_dev(v) for k, v in x.items()}
    kw = dict(max_pos=max(contexts) - 1, q_lat=d["q_lat"], w_gate=d["w_gate"])
    args = (d["q"], d["pos0"], d["k_win"], d["v_win"], d["kc"], d["vc"])
    ref = lgsa.hca_attn_fwd(*args, **kw)
    got = lgsa.hca_attn_fwd_static(*args, **kw)
    return ref, got


def test_static_scratch_two_decode_calls_then_prefill(torch):
    # 1: the HCA decode workload, 64 sequences at context 131072 (4 splits each, 33.7 MB of
    #    partials in the static scratch)
    ref1, got1 = _decode(torch, 2, 64, [131072] * 64)
    torch.cuda.synchronize()
    # 2: smaller, 8 sequences at mixed contexts up to 20000 (9 splits of 32 keys each)
    ref2, got2 = _decode(torch, 41, 8, [20000, 19999, 12345, 128, 127, 1, 5000, 17000])
    torch.cuda.synchronize()
    for ref, got, what in ((ref1, got1, "first call"), (ref2, got2, "second call")):
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), what
        bf16_ok(from_dev(got), from_dev(ref), what)
    # 3: a gated prefill (no scratch needed) through the same entry point
    x = synth.hca_prefill(42, T=300, H=4, bf16=True)
    d = {k: to_dev(v) for k, v in x.items()}
    kc, vc = lgsa.hca_compress(d["k"], d["v"])
    kw = dict(max_pos=299, q_lat=d["q_lat"], w_gate=d["w_gate"])
    ref = lgsa.hca_attn_fwd(d["q"], d["pos0"], d["k"], d["v"], kc, vc, **kw)
    got = lgsa.hca_attn_fwd_static(d["q"], d["pos0"], d["k"], d["v"], kc, vc, **kw)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), "prefill"


def test_static_scratch_refuses_oversized_call(torch):
    # 160 sequences of 64 heads need 42,106,880 bytes of partials: refused, nothing enqueued
    x = torch.zeros((160, 1, 64, 512), dtype=torch.bfloat16, device="cuda")
    ring = torch.zeros((160, 128, 512), dtype=torch.bfloat16, device="cuda")
    ent = torch.zeros((160, 1024, 512), dtype=torch.bfloat16, device="cuda")
    pos0 = torch.full((160,), 131071, dtype=torch.int32, device="cuda")
    with pytest.raises(lgsa.LgsaError) as e:
        lgsa.hca_attn_fwd_static(x, pos0, ring, ring, ent, ent, max_pos=131071)
    assert e.value.code == lgsa.LGSA_EWORKSPACE
