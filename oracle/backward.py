"""Backward of the forward path's steps, written out in NumPy float64.

TEST INFRASTRUCTURE ONLY: like the rest of this package, only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may use it, and it shares
no code with the HIP library.

Each function is the chain rule applied to the forward definition it names, for a loss L whose
gradient with respect to the forward output is given (dout).  The pages give no backward
formulas; training through these layers is what they describe (ERNIE 5.5 Flash Base release
blog, section 3), so the gradients are those of the forward steps as this package defines them.

Gate (release blog, section 2.1: the attention output is multiplied per channel by a sigmoid
gate of the low-rank query latent): out = o * s with s = sigmoid(G), G = q_lat W.  Then
    do = dout * s,   dG = dout * o * s * (1 - s),   dq_lat = dG W^T,   dW = q_lat^T dG.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    """Stored values as float64 (uint16 arrays hold bfloat16 bits); widening is exact."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def latent_gate_bwd(q_lat, w_gate, o, dout):
    """q_lat [M, d_lat], w_gate [d_lat, N], o and dout [M, N] -> (do [M, N], dq_lat [M, d_lat],
    dw_gate [d_lat, N]), float64."""
    Q, W, O, D = _f64(q_lat), _f64(w_gate), _f64(o), _f64(dout)
    s = 1.0 / (1.0 + np.exp(-(Q @ W)))
    dG = D * O * s * (1.0 - s)
    return D * s, dG @ W.T, Q.T @ dG


def _attn_rows_bwd(q, keys, vals, dO, scale):
    """Softmax attention backward for the rows of one query position: q [H, d] against keys
    [n, d] and values [n, dv] with output gradient dO [H, dv].  Returns (dq [H, d],
    dkeys [n, d], dvals [n, dv]).  With p = softmax(scale q k^T) and o = p v:
    dv = p^T dO, dp = dO v^T, ds = p (dp - rowsum(p dp)), dq = scale ds k, dk = scale ds^T q."""
    logits = scale * (q @ keys.T)
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    dp = dO @ vals.T
    ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    return scale * ds @ keys, scale * ds.T @ q, p.T @ dO


def hca_attn_bwd(q, pos0, k, v, dout, *, window=128, block=128, scale=None):
    """Backward of Heavily Compressed Attention in prefill, where the window rows are the
    sequence's own keys and values and the entries are their block means (release blog,
    section 2.1; xenospectrum.com article for the 128-token window): query (b, i) at position
    t = pos0[b] + i attends to entries e with block e + block - 1 <= t (entry = mean of K, V
    over positions block e .. block e + block - 1) and to positions max(0, t - window + 1) .. t.
    An entry's key gradient flows back to each of its block's positions divided by block.

    q [B, Tq, H, d]; k, v [B, T, d]; dout [B, Tq, H, d] -> (dq [B, Tq, H, d], dk [B, T, d],
    dv [B, T, d]), float64."""
    Q, K, V, D = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Tq, H, d = Q.shape
    T = K.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    ne_all = T // block
    dq = np.zeros_like(Q)
    dk = np.zeros_like(K)
    dv = np.zeros_like(V)
    for b in range(B):
        kc = K[b, :ne_all * block].reshape(ne_all, block, d).mean(axis=1)
        vc = V[b, :ne_all * block].reshape(ne_all, block, V.shape[-1]).mean(axis=1)
        dkc = np.zeros_like(kc)
        dvc = np.zeros_like(vc)
        for i in range(Tq):
            t = int(pos0[b]) + i
            if t < 0:
                continue
            ne = min((t + 1) // block, ne_all)
            lo = max(0, t - window + 1)
            keys = np.concatenate([kc[:ne], K[b, lo:t + 1]])
            vals = np.concatenate([vc[:ne], V[b, lo:t + 1]])
            g_q, g_k, g_v = _attn_rows_bwd(Q[b, i], keys, vals, D[b, i], scale)
            dq[b, i] = g_q
            dkc[:ne] += g_k[:ne]
            dvc[:ne] += g_v[:ne]
            dk[b, lo:t + 1] += g_k[ne:]
            dv[b, lo:t + 1] += g_v[ne:]
        dk[b, :ne_all * block] += np.repeat(dkc / block, block, axis=0)
        dv[b, :ne_all * block] += np.repeat(dvc / block, block, axis=0)
    return dq, dk, dv


def sparse_attn_bwd(q, k_lat, idx, dout, v_lat=None, *, dqk=None, dv=None, scale=None):
    """Backward of DSA sparse core attention (release blog, section 2.1: attention over the
    selected positions only): query (b, i) attends to the rows idx[b, i, :] (negative entries
    and entries >= S skipped; a row listed twice counts twice); key = first dqk entries of a
    k_lat row, value = first dv entries of a v_lat row (v_lat None: the k_lat rows, so both
    gradients land on the same latent row).

    q [B, Tq, H, dqk]; k_lat [B, S, wk]; idx [B, Tq, k]; dout [B, Tq, H, dv] -> (dq, dk_lat
    [B, S, wk], dv_lat [B, S, wv] or None when v_lat is None), float64."""
    Q, KL, D = _f64(q), _f64(k_lat), _f64(dout)
    VL = KL if v_lat is None else _f64(v_lat)
    B, Tq, H, dq_ = Q.shape
    S = KL.shape[1]
    dqk = dq_ if dqk is None else dqk
    dv = D.shape[-1] if dv is None else dv
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    idx = np.asarray(idx)
    gq = np.zeros_like(Q)
    gk = np.zeros_like(KL)
    gv = gk if v_lat is None else np.zeros_like(VL)
    for b in range(B):
        for i in range(Tq):
            sel = [int(s) for s in idx[b, i] if 0 <= int(s) < S]
            if not sel:
                continue
            g_q, g_k, g_v = _attn_rows_bwd(Q[b, i, :, :dqk], KL[b, sel, :dqk], VL[b, sel, :dv],
                                           D[b, i, :, :dv], scale)
            gq[b, i, :, :dqk] = g_q
            for j, s in enumerate(sel):
                gk[b, s, :dqk] += g_k[j]
                gv[b, s, :dv] += g_v[j]
    return gq, gk, (None if v_lat is None else gv)


def sparse_attn_lse(q, k_lat, idx, *, dqk=None, scale=None):
    """Log-sum-exp of each DSA sparse attention row (release blog, section 2.1): for query
    (b, i) and head h, log sum_j exp(scale <q[b,i,h], K_j>) over the keys idx[b, i, :] lists
    (entries < 0 or >= S skipped, a repeated entry counted each time it appears), or -inf for
    a row with no valid entry.  This is the normaliser the softmax divides by, in natural log.

    q [B, Tq, H, d]; k_lat [B, S, wk]; idx [B, Tq, k] -> [B, Tq, H] float64."""
    Q, KL = _f64(q), _f64(k_lat)
    B, Tq, H, d = Q.shape
    S = KL.shape[1]
    dqk = d if dqk is None else dqk
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    idx = np.asarray(idx)
    out = np.full((B, Tq, H), -np.inf)
    for b in range(B):
        for i in range(Tq):
            sel = [int(s) for s in idx[b, i] if 0 <= int(s) < S]
            if not sel:
                continue
            z = scale * (Q[b, i, :, :dqk] @ KL[b, sel, :dqk].T)
            m = z.max(axis=1)
            out[b, i] = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    return out

