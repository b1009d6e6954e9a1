"""Pins of the compressed sparse attention composite (oracle.csa_attn) and of the block rule
of the oracle's top-k, against things they do not compute themselves.  ERNIE 5.5 Flash Base
release blog, section 2.1: a compressed sparse layer compresses the history 4x and attends to
a sparse part of it; here a compressed entry becomes visible once its block is complete, as
HCA's entries do, and the indexer's top-k picks among the visible entries."""
import numpy as np
import pytest

from oracle import dense


def _inputs(rng, T=37, H=3, d=16, Hi=4):
    q = rng.standard_normal((1, T, H, d)).astype(np.float32)
    k = rng.standard_normal((1, T, d)).astype(np.float32)
    v = rng.standard_normal((1, T, d)).astype(np.float32)
    q_idx = rng.standard_normal((1, T, Hi, 64)).astype(np.float32)
    w_idx = rng.uniform(0, 1, (1, T, Hi)).astype(np.float32)
    k_idx = rng.standard_normal((1, T, 64)).astype(np.float32)
    return q, k, v, q_idx, w_idx, k_idx


def _pool(x, block):
    """Mean of every complete block of rows, written out with a loop (not the oracle's)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[1] // block
    out = np.zeros((x.shape[0], n) + x.shape[2:])
    for e in range(n):
        out[:, e] = sum(x[:, block * e + i] for i in range(block)) / block
    return out


def test_all_entries_kept_is_dense_attention_over_completed_blocks(orc):
    """With k at least the number of entries, every visible entry is kept: the result is
    textbook softmax attention over the complete blocks' means."""
    rng = np.random.default_rng(71)
    q, k, v, q_idx, w_idx, k_idx = _inputs(rng)
    T, block = q.shape[1], 4
    out, idx, _, _, _, _ = orc.csa_attn(q, [0], k, v, q_idx, w_idx, k_idx, 64, block=block)
    kc, vc = _pool(k, block)[0], _pool(v, block)[0]
    d = q.shape[-1]
    for t in range(T):
        n = (t + 1) // block
        assert list(idx[t][:n]) == list(range(n)) and all(x == -1 for x in idx[t][n:])
        if n == 0:
            assert np.all(out[t] == 0.0)
            continue
        logits = np.einsum("hd,sd->hs", q[0, t].astype(np.float64), kc[:n]) / np.sqrt(d)
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        assert np.allclose(out[t], p @ vc[:n], rtol=0, atol=1e-12), t


def test_block_one_keeping_everything_is_dense_causal_attention(orc):
    rng = np.random.default_rng(72)
    q, k, v, q_idx, w_idx, k_idx = _inputs(rng, T=20)
    out, _, _, _, _, _ = orc.csa_attn(q, [0], k, v, q_idx, w_idx, k_idx, 32, block=1)
    ref = dense.dense_causal(q[0], k[0], v[0])
    assert np.allclose(out, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("block,k_top", [(4, 3), (4, 5), (2, 4), (8, 2)])
def test_topk_over_compressed_entries_is_brute_force(orc, block, k_top):
    """Scores of the pooled indexer keys from a NumPy loop, ordered by (score desc, index asc),
    agree with the oracle's selection for every row, and the rule hides incomplete blocks."""
    rng = np.random.default_rng(73 + block)
    T = 41
    _, _, _, q_idx, w_idx, k_idx = _inputs(rng, T=T)
    kic = _pool(k_idx, block).astype(np.float32)
    idx, kth = orc.dsa_topk(q_idx, w_idx, kic, [0], k_top, block=block)
    for t in range(T):
        n = (t + 1) // block
        sc = [sum(float(w_idx[0, t, h]) * max(0.0, float(np.dot(q_idx[0, t, h].astype(np.float64),
                                                                 kic[0, s].astype(np.float64))))
                  for h in range(4)) for s in range(n)]
        order = sorted(range(n), key=lambda s: (-sc[s], s))
        keep = sorted(order[:k_top])
        assert list(idx[t][:len(keep)]) == keep and all(x == -1 for x in idx[t][len(keep):]), t
        if n <= k_top:
            assert kth[t] == -np.inf
        else:  # the same sum in another order: equal to rounding
            assert abs(kth[t] - sc[order[k_top - 1]]) <= 1e-12 * max(1.0, abs(kth[t]))


def test_entry_visible_only_once_its_block_is_complete(orc):
    rng = np.random.default_rng(74)
    _, _, _, q_idx, w_idx, k_idx = _inputs(rng, T=16)
    kic = _pool(k_idx, 4).astype(np.float32)
    idx, _ = orc.dsa_topk(q_idx, w_idx, kic, [0], 8, block=4)
    for t, n in [(0, 0), (2, 0), (3, 1), (6, 1), (7, 2), (15, 4)]:
        assert list(idx[t][:n]) == list(range(n)) and all(x == -1 for x in idx[t][n:]), t


def test_rows_past_the_held_entries_are_rejected(orc):
    """A query whose visible entries are not all held (S too small) is an argument error."""
    rng = np.random.default_rng(75)
    _, _, _, q_idx, w_idx, k_idx = _inputs(rng, T=16)
    kic = _pool(k_idx, 4).astype(np.float32)[:, :2]
    with pytest.raises(ValueError):
        orc.dsa_topk(q_idx, w_idx, kic, [0], 8, block=4)
