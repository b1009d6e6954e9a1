"""NumPy float64 brute-force dense causal attention, used only to pin the oracle.

TEST INFRASTRUCTURE ONLY.  This is textbook softmax attention written with NumPy matrix
products, independent of ``oracle.cpp``: when HCA has no compressed entries and a window at
least as long as the sequence, and when DSA keeps every causal position (k >= context),
both must reduce to exactly this (ERNIE 5.5 Flash Base release blog, section 2.1: HCA and
DSA are restrictions of full-context attention to a visible or selected subset).
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(a):
    """Widen an array of bfloat16 bit patterns (uint16) to float64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def dense_causal(q, k, v, scale=None):
    """q [T,H,d], k [T,dk], v [T,dv] -> O [T,H,dv] with O[t] = softmax(scale q_t K[:t+1]^T) V[:t+1]."""
    q = bf16_to_f64(q)
    k = bf16_to_f64(k)
    v = bf16_to_f64(v)
    T, H, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    logits = np.einsum("thd,sd->ths", q, k) * scale        # [T,H,T]
    causal = np.tril(np.ones((T, T), dtype=bool))          # s <= t
    logits = np.where(causal[:, None, :], logits, -np.inf)
    logits -= logits.max(axis=-1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=-1, keepdims=True)
    return np.einsum("ths,sd->thd", p, v)
