"""GPU parity of the attention calls with the head mix (VHA, ERNIE 5.5 Flash Base release
blog, section 2.1: after attention, a light low-rank mix across heads with an identity skip)
against the fp64 oracle composed with the NumPy VHA oracle: out = vha_mix(gated attention).

  - sparse_attn_fwd with many query rows: the gate factors come first from the gate GEMM, and
    the gate and the mix are applied in the attention kernel's epilogue (a workgroup holds the
    64 heads of its row); values shared with the keys and distinct; gated and ungated;
  - sparse_attn_fwd with few rows and long lists (split, merged by the combine kernel, then the
    mix as a pass of its own);
  - hca_attn_fwd prefill (gate in the attention epilogue, then the mix pass) and decode.
The factors are scaled so that the cross-head term is comparable to the skip term.
Tolerances are stated in tests/helpers.py."""
import numpy as np
import pytest

import hybrid_sparse_attention_amd as lgsa
from hybrid_sparse_attention_amd import synth
from oracle import vha

from helpers import bf16_ok, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lgsa.load()
    return torch


def _factors(seed, H, r):
    return (synth.normal(seed, (H, r), 0.25, True), synth.normal(seed + 1, (H, r), 0.25, True))


@pytest.mark.parametrize("Tq,S,k,r,distinct,gated", [
    (300, 600, 128, 16, False, True),   # 300 rows, lists too short to split
    (1100, 1500, 64, 7, False, True),   # one workgroup per row (no split), V = K
    (1100, 1500, 64, 16, True, True),   # distinct values
    (1100, 1500, 64, 3, False, False),  # ungated, mix only
    (2, 5000, 2048, 16, False, True),   # decode-like: lists split and merged, then the mix pass
])
def test_sparse_gate_and_vha(torch, orc, Tq, S, k, r, distinct, gated):
    H = 64
    x = synth.dsa_sparse(430 + Tq % 97 + r, B=1, Tq=Tq, S=S, H=H, distinct_v=distinct,
                         gated=gated)
    idx = synth.random_topk(431 + r, 1, Tq, S, k, [S - Tq])
    u, v = _factors(432 + r, H, r)
    vl = to_dev(x["v_lat"]) if distinct else None
    out = lgsa.sparse_attn_fwd(to_dev(x["q"]), to_dev(x["kv_lat"]), to_dev(idx), v_lat=vl,
                               q_lat=to_dev(x["q_lat"]) if gated else None,
                               w_gate=to_dev(x["w_gate"]) if gated else None,
                               vha_u=to_dev(u), vha_v=to_dev(v))
    torch.cuda.synchronize()
    att = orc.sparse_attn(x["q"], x["kv_lat"], idx, v_lat=x.get("v_lat") if distinct else None,
                          q_lat=x.get("q_lat"), w_gate=x.get("w_gate"))
    ref = vha.vha_mix(att, u, v)
    assert np.abs(ref - att).max() > 0.05 * np.abs(ref).max()  # the mix matters
    bf16_ok(from_dev(out).reshape(-1, H, 256), ref, "sparse gate + vha")


def test_sparse_gate_without_vha(torch, orc):
    """The gated path alone (the gate GEMM rescales the attention output afterwards), with a
    ragged row count, against the oracle."""
    Tq, S, k, H = 1030, 1400, 96, 64
    x = synth.dsa_sparse(440, B=1, Tq=Tq, S=S, H=H)
    idx = synth.random_topk(441, 1, Tq, S, k, [S - Tq])
    out = lgsa.sparse_attn_fwd(to_dev(x["q"]), to_dev(x["kv_lat"]), to_dev(idx),
                               q_lat=to_dev(x["q_lat"]), w_gate=to_dev(x["w_gate"]))
    torch.cuda.synchronize()
    ref = orc.sparse_attn(x["q"], x["kv_lat"], idx, q_lat=x["q_lat"], w_gate=x["w_gate"])
    bf16_ok(from_dev(out).reshape(-1, H, 256), ref, "sparse gate")


def test_hca_prefill_gate_and_vha(torch, orc):
    T, H, r = 600, 64, 16
    x = synth.hca_prefill(445, T=T, H=H, bf16=True)
    u, v = _factors(446, H, r)
    kd, vd = to_dev(x["k"]), to_dev(x["v"])
    kc, vc = lgsa.hca_compress(kd, vd)
    out = lgsa.hca_attn_fwd(to_dev(x["q"]), to_dev(x["pos0"]), kd, vd, kc, vc, max_pos=T - 1,
                            q_lat=to_dev(x["q_lat"]), w_gate=to_dev(x["w_gate"]),
                            vha_u=to_dev(u), vha_v=to_dev(v))
    torch.cuda.synchronize()
    att = orc.hca_attn(x["q"], x["pos0"], x["k"], x["v"], orc.hca_compress(x["k"]),
                       orc.hca_compress(x["v"]), q_lat=x["q_lat"], w_gate=x["w_gate"])
    bf16_ok(from_dev(out)[0], vha.vha_mix(att, u, v), "hca prefill gate + vha")


def test_hca_decode_gate_and_vha(torch, orc):
    B, H, r = 5, 64, 9
    contexts = [3000, 129, 128, 1, 2500]
    x = synth.hca_decode(447, B=B, context=max(contexts), H=H, contexts=contexts)
    u, v = _factors(448, H, r)
    out = lgsa.hca_attn_fwd(to_dev(x["q"]), to_dev(x["pos0"]), to_dev(x["k_win"]),
                            to_dev(x["v_win"]), to_dev(x["kc"]), to_dev(x["vc"]),
                            max_pos=max(contexts) - 1, q_lat=to_dev(x["q_lat"]),
                            w_gate=to_dev(x["w_gate"]), vha_u=to_dev(u), vha_v=to_dev(v))
    torch.cuda.synchronize()
    att = orc.hca_attn(x["q"], x["pos0"], x["k_win"], x["v_win"], x["kc"], x["vc"],
                       q_lat=x["q_lat"], w_gate=x["w_gate"])
    bf16_ok(from_dev(out).reshape(B, H, 512), vha.vha_mix(att, u, v), "hca decode gate + vha")
