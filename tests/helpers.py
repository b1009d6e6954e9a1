"""Shared helpers of the GPU parity tests: host <-> device conversion and the tolerance checks.

Tolerances (written here once): bfloat16 outputs pass when
    max|gpu - ref| <= 1e-2 * max|ref| + 1e-3
and float32 outputs when
    max|gpu - ref| <= 1e-5 * max|ref|,
both maxima taken over the compared tensor.  Top-k sets pass when they are identical except
for positions whose oracle score lies within 1e-5 * max(1, |s_k|) of the k-th score s_k.
"""
import numpy as np

from hybrid_sparse_attention_amd import synth


def to_dev(a, device="cuda"):
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def from_dev(t):
    """Device tensor -> float64 numpy (bf16 widened exactly)."""
    import torch

    t = t.detach()
    if t.dtype == torch.bfloat16:
        return synth.bf16_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(
            np.float64)
    return t.cpu().numpy().astype(np.float64)


def bf16_ok(got, ref, what=""):
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    tol = 1e-2 * float(np.max(np.abs(ref))) + 1e-3 if ref.size else 1e-3
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    assert err <= tol, "%s: max|err| %.3g > tol %.3g" % (what, err, tol)
    return err, tol


def f32_ok(got, ref, what=""):
    err = float(np.max(np.abs(got - ref)))
    tol = 1e-5 * float(np.max(np.abs(ref)))
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    assert err <= tol, "%s: max|err| %.3g > tol %.3g" % (what, err, tol)
    return err, tol


def check_topk_row(gpu_row, orc_row, t, k, scores, kth):
    """One query row: structure of the GPU list (ascending, distinct, causal, -1 padded) and
    equality with the oracle's set up to the tie band.  `scores` are the oracle's float64
    scores of positions 0..t.  Returns True when the sets are identical."""
    n = min(k, t + 1)
    g = [int(x) for x in gpu_row]
    assert all(x == -1 for x in g[n:]), "padding"
    sel = g[:n]
    assert all(0 <= x <= t for x in sel), "causal range"
    assert all(sel[i] < sel[i + 1] for i in range(n - 1)), "ascending and distinct"
    o = set(int(x) for x in orc_row[:n])
    if set(sel) == o:
        return True
    band = 1e-5 * max(1.0, abs(kth))
    for s in set(sel) ^ o:
        assert abs(scores[s] - kth) <= band, \
            "position %d (score %.9g) outside the tie band of s_k=%.9g" % (s, scores[s], kth)
    return False
