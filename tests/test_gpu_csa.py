"""Compressed sparse attention on the GPU (hca_compress with block 4, dsa_index_topk with block
4, sparse_attn_fwd with distinct values), against the oracle's composite (ERNIE 5.5 Flash Base
release blog, section 2.1: history compressed 4x, then a sparse part of it attended)."""
import numpy as np
import pytest

import hybrid_sparse_attention_amd as lgsa
from hybrid_sparse_attention_amd import synth

from helpers import bf16_ok, check_topk_row, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lgsa.load()
    return torch


def _run(torch, x, k_top, block, gated, pos0=None):
    B, T = x["k_idx"].shape[:2]
    pos0 = np.zeros(B, np.int32) if pos0 is None else np.asarray(pos0, np.int32)
    kw = dict(q_lat=to_dev(x["q_lat"]), w_gate=to_dev(x["w_gate"])) if gated else {}
    out, idx = lgsa.csa_attn_fwd(to_dev(x["q"]), to_dev(pos0), to_dev(x["kv_lat"]),
                                 to_dev(x["v_lat"]), to_dev(x["q_idx"]), to_dev(x["w_idx"]),
                                 to_dev(x["k_idx"]), k_top, max_pos=int(pos0.max()) + x["q"].shape[1] - 1,
                                 block=block, **kw)
    torch.cuda.synchronize()
    return from_dev(out), idx.cpu().numpy(), pos0


@pytest.mark.parametrize("T,k_top,gated", [(3000, 256, True), (2100, 64, False)])
def test_csa_chain_against_oracle(torch, orc, T, k_top, gated):
    """Selections agree with the oracle's up to the tie band; on rows whose selections agree,
    the outputs agree to the bf16 bound."""
    block = 4
    x = synth.csa(41, B=1, T=T, H=64, gated=gated)
    out, g, pos0 = _run(torch, x, k_top, block, gated)
    rng = np.random.default_rng(5)
    rows = sorted(set([0, 2, 3, 4, 7, 4 * k_top - 1, 4 * k_top + 3, T - 1] +
                      list(rng.integers(0, T, 24))))
    kw = dict(q_lat=x["q_lat"], w_gate=x["w_gate"]) if gated else {}
    ref, oidx, kth, _, _, kic = orc.csa_attn(x["q"], pos0, x["kv_lat"], x["v_lat"], x["q_idx"],
                                             x["w_idx"], x["k_idx"], k_top, block=block,
                                             rows=rows, **kw)
    agree = []
    for j, r in enumerate(rows):
        n = (r + 1) // block
        sc = orc.dsa_scores(x["q_idx"], x["w_idx"], kic, 0, r, 0, n)
        if n == 0:
            assert np.all(g[0, r] == -1)
            agree.append(j)
            continue
        if check_topk_row(g[0, r], oidx[j], n - 1, k_top, sc, kth[j]):
            agree.append(j)
    assert len(agree) >= len(rows) - 2
    bf16_ok(out[0][[rows[j] for j in agree]], ref[agree], "csa chain")


def test_csa_rows_before_the_first_block_are_zero_and_all_entries_kept_is_dense(torch, orc):
    """Positions 0..2 see no complete block (zeros); with k_top above the entry count every
    row keeps all its visible entries (in order) and matches the oracle exactly as a dense
    attention over the complete blocks would."""
    T, block, k_top = 600, 4, 256
    x = synth.csa(42, B=1, T=T, H=64, gated=False)
    out, g, pos0 = _run(torch, x, k_top, block, False)
    assert np.all(out[0, :3] == 0.0)
    for t in [0, 2, 3, 7, 100, 599]:
        n = min((t + 1) // block, k_top)
        assert g[0, t].tolist() == list(range(n)) + [-1] * (k_top - n), t
    rows = [3, 4, 50, 511, 512, 599]
    ref = orc.csa_attn(x["q"], pos0, x["kv_lat"], x["v_lat"], x["q_idx"], x["w_idx"],
                       x["k_idx"], k_top, block=block, rows=rows)[0]
    bf16_ok(out[0][rows], ref, "csa all kept")


def test_csa_decode_rows_at_later_positions(torch, orc):
    """Two sequences whose query rows sit at different positions (pos0 > 0): the compressed
    entries each row sees follow its own position."""
    T, block, k_top, Tq = 2048, 4, 128, 4
    x = synth.csa(43, B=2, T=T, H=64, gated=True)
    # the last Tq positions of each sequence are the queries
    q = x["q"][:, T - Tq:].copy()
    xq = dict(x)
    xq["q"], xq["q_idx"], xq["w_idx"] = q, x["q_idx"][:, T - Tq:].copy(), x["w_idx"][:, T - Tq:].copy()
    xq["q_lat"] = x["q_lat"][:, T - Tq:].copy()
    pos0 = np.array([T - Tq, T - Tq - 9], np.int32)
    out, g, _ = _run(torch, xq, k_top, block, True, pos0=pos0)
    rows = list(range(2 * Tq))
    ref, oidx, kth, _, _, kic = orc.csa_attn(xq["q"], pos0, x["kv_lat"], x["v_lat"], xq["q_idx"],
                                             xq["w_idx"], x["k_idx"], k_top, block=block,
                                             rows=rows, q_lat=xq["q_lat"], w_gate=x["w_gate"])
    agree = []
    for j, r in enumerate(rows):
        b, i = divmod(r, Tq)
        n = (int(pos0[b]) + i + 1) // block
        sc = orc.dsa_scores(xq["q_idx"], xq["w_idx"], kic, b, i, 0, n)
        if check_topk_row(g[b, i], oidx[j], n - 1, k_top, sc, kth[j]):
            agree.append(j)
    assert len(agree) >= len(rows) - 1
    got = np.concatenate([out[0], out[1]])[[rows[j] for j in agree]]
    bf16_ok(got, ref[agree], "csa decode rows")
