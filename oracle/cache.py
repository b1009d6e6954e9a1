"""Decode-time cache maintenance written out in NumPy float64.

TEST INFRASTRUCTURE ONLY: like the rest of this package, only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may use it, and it shares
no code with the HIP library.

ERNIE 5.5 Flash Base release blog, section 2.1: an HCA layer keeps one cache entry per
completed block of 128 tokens (read, as for the prefill compressor, as the mean of the block's
keys and, separately, values) plus a window of the most recent raw tokens (128 of them, per
the xenospectrum.com article on ERNIE 5.5 Flash Base, long-context section), held here in a
ring whose row p % win_len holds position p.  A DSA layer keeps one indexer key and one latent
row per position.  A decode step appends its new token's rows before its attention runs.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    """Stored values as float64 (uint16 arrays hold bfloat16 bits); widening is exact."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def hca_cache_append(pos, k_new, v_new, k_win, v_win, kc=None, vc=None, block=128):
    """One decode step's HCA cache update; returns updated float64 copies (k_win, v_win, kc, vc).

    For each sequence b with t = pos[b] >= 0: ring row t % win_len takes the new key / value;
    when t is the last token of its block (t % block == block - 1) and the entry index
    e = t // block is held (e < n_cap), entry e becomes the mean of the block's rows: positions
    t - block + 1 .. t - 1 from the ring and position t from the new row.  Sequences with a
    negative position are left as they are.
    """
    kn, vn = _f64(k_new), _f64(v_new)
    kw, vw = _f64(k_win), _f64(v_win)
    kw_out, vw_out = kw.copy(), vw.copy()
    kc_out = None if kc is None else _f64(kc).copy()
    vc_out = None if vc is None else _f64(vc).copy()
    W = kw.shape[1]
    for b, t in enumerate(np.asarray(pos).tolist()):
        if t < 0:
            continue
        for new, ring_in, ring_out, cache in ((kn, kw, kw_out, kc_out), (vn, vw, vw_out, vc_out)):
            ring_out[b, t % W] = new[b]
            if cache is None or t % block != block - 1 or t // block >= cache.shape[1]:
                continue
            rows = [new[b] if p == t else ring_in[b, p % W] for p in range(t - block + 1, t + 1)]
            cache[b, t // block] = np.sum(np.stack(rows), axis=0) / block
    return kw_out, vw_out, kc_out, vc_out


def dsa_cache_append(pos, k_idx_new, k_idx, kv_new, kv_lat):
    """One decode step's DSA cache append; returns updated float64 copies (k_idx, kv_lat).

    For each sequence b with 0 <= t = pos[b] < S: k_idx[b, t] = k_idx_new[b] and the first
    row = kv_new.shape[1] elements of kv_lat[b, t] take kv_new[b].  Other sequences are left as
    they are.
    """
    ki, kv = _f64(k_idx).copy(), _f64(kv_lat).copy()
    kin, kvn = _f64(k_idx_new), _f64(kv_new)
    S, row = ki.shape[1], kvn.shape[1]
    for b, t in enumerate(np.asarray(pos).tolist()):
        if 0 <= t < S:
            ki[b, t] = kin[b]
            kv[b, t, :row] = kvn[b]
    return ki, kv
