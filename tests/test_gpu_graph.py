"""The calls under HIP graph capture (torch.cuda.graph): the library enqueues kernels only (no
allocation, no memset, no host synchronisation), so a captured step replays.  Captured here:
a gated HCA decode through hca_attn_fwd_static (its split partials in the library's static
scratch) followed by the decode top-k and gated sparse attention of a DSA layer (their
workspaces allocated by the binding from the graph's memory pool).  Each graph is replayed
several times, with eager work and synchronisations between the replays, and every replay is
compared with the eager result bit for bit (the same kernels on the same inputs)."""
import numpy as np
import pytest

import hybrid_sparse_attention_amd as lgsa
from hybrid_sparse_attention_amd import synth

from helpers import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lgsa.load()
    return torch


def _capture(torch, fn):
    """fn() once on a side stream (warm-up, as graph capture asks), then captured."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    return g, outs


def test_decode_step_replays(torch):
    B, ctx, H = 64, 4096, 64
    xh = synth.hca_decode(70, B=B, context=ctx, H=H)
    dh = {k: to_dev(v) for k, v in xh.items()}
    Bd, S, k = 4, 20000, 2048
    xi = synth.dsa_index(71, B=Bd, Tq=1, S=S, pos0=[S - 1, 15000, 9000, 1000])
    xs = synth.dsa_sparse(72, B=Bd, Tq=1, S=S, H=H)
    di = {k_: to_dev(v) for k_, v in xi.items()}
    ds = {k_: to_dev(v) for k_, v in xs.items()}

    def step():
        o_h = lgsa.hca_attn_fwd_static(dh["q"], dh["pos0"], dh["k_win"], dh["v_win"], dh["kc"],
                                       dh["vc"], max_pos=ctx - 1, q_lat=dh["q_lat"],
                                       w_gate=dh["w_gate"])
        idx = lgsa.dsa_index_topk(di["q_idx"], di["w_idx"], di["k_idx"], di["pos0"], k,
                                  max_pos=S - 1)
        o_s = lgsa.sparse_attn_fwd(ds["q"], ds["kv_lat"], idx, q_lat=ds["q_lat"],
                                   w_gate=ds["w_gate"])
        return o_h, idx, o_s

    eager = [t.clone() for t in step()]
    torch.cuda.synchronize()
    g, outs = _capture(torch, step)
    junk = torch.empty(1 << 24, dtype=torch.float32, device="cuda")
    for rep in range(4):
        for t in outs:
            t.zero_()
        junk.normal_()  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("hca decode", "top-k", "sparse"), outs, eager):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.int32 else a,
                               b.view(torch.uint8) if b.dtype != torch.int32 else b), \
                "replay %d: %s differs from the eager call" % (rep, name)
    assert np.any(eager[0].float().cpu().numpy() != 0)
