"""Independent fp64 CPU oracle for the Latent-Gated Sparse Attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package.  It shares no code with the HIP library
(``hybrid_sparse_attention_amd``) and imports nothing from it.

The arithmetic lives in ``oracle.cpp`` (plain C++17 in float64, built by g++ with OpenMP);
this module only builds it, loads it and marshals numpy arrays through ctypes.
``dense.py`` holds a NumPy brute-force dense causal attention used to pin the oracle.

Sources: ERNIE 5.5 Flash Base release blog, section 2.1 "Latent-Gated Sparse Attention";
xenospectrum.com article on ERNIE 5.5 Flash Base, section on the 128-token sliding window.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.environ.get("LGSA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

DT_F32, DT_BF16, DT_F64 = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.cpp with g++ into liboracle.so next to it and return the path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared", "-Wall",
               "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P, L, I, D = ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_double
        lib.orc_hca_compress.argtypes = [P, I, L, L, L, L, P]
        lib.orc_hca_attn.argtypes = [P, I, L, L, L, L, P, P, P, I, L, L, P, P, I, L, L, D,
                                     P, P, I, L, P, L, P]
        lib.orc_latent_gate.argtypes = [P, I, P, I, P, I, L, L, L, P, L, P]
        lib.orc_dsa_scores.argtypes = [P, P, P, L, L, L, L, L, L, L, L, L, P]
        lib.orc_dsa_topk.argtypes = [P, P, P, L, L, L, L, L, L, L, P, P, L, P, P]
        lib.orc_sparse_attn.argtypes = [P, I, L, L, L, L, L, P, L, P, L, I, L, P, L, D, P, P,
                                        I, L, P, L, P]
        for f in (lib.orc_hca_compress, lib.orc_hca_attn, lib.orc_latent_gate,
                  lib.orc_dsa_scores, lib.orc_dsa_topk, lib.orc_sparse_attn):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def set_threads(n: int) -> None:
    """Set the OpenMP thread count the oracle uses (for the CPU-baseline timing)."""
    os.environ["OMP_NUM_THREADS"] = str(int(n))
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(ctypes.c_int(int(n)))
    except OSError:
        pass


def max_threads() -> int:
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_get_max_threads.restype = ctypes.c_int
        return int(gomp.omp_get_max_threads())
    except OSError:
        return 1


# ----------------------------------------------------------------------------- helpers
def _tensor(a):
    """Return (contiguous array, dtype code).  uint16 arrays hold bfloat16 bits."""
    if a is None:
        return None, DT_F32
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, DT_F32
    if a.dtype == np.uint16:
        return a, DT_BF16
    if a.dtype == np.float64:
        return a, DT_F64
    raise TypeError("oracle tensors must be float32, float64 or uint16 (bf16 bits), got %s"
                    % a.dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _rows(rows, total):
    if rows is None:
        rows = np.arange(total, dtype=np.int64)
    return np.ascontiguousarray(np.asarray(rows, dtype=np.int64))


def _check(rc, name):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments (code %d)" % (name, rc))


# ----------------------------------------------------------------------------- API
def hca_compress(x, block: int = 128):
    """Mean of every complete block of `block` rows: x [B,T,d] -> [B,T//block,d] float64."""
    x, dt = _tensor(x)
    B, T, d = x.shape
    out = np.zeros((B, T // block, d), dtype=np.float64)
    _check(_load().orc_hca_compress(_ptr(x), dt, B, T, d, block, _ptr(out)), "hca_compress")
    return out


def hca_attn(q, pos0, k_win, v_win, kc=None, vc=None, *, window=128, block=128, scale=None,
             q_lat=None, w_gate=None, rows=None):
    """Heavily Compressed Attention (optionally gated) for the listed flat query rows.

    q [B,Tq,H,d]; pos0 [B] int; k_win, v_win [B,win_len,d] (row of position p is
    p % win_len); kc, vc [B,n_cap,d] or None; q_lat [B,Tq,d_lat]; w_gate [d_lat,H*d].
    Returns float64 [n_rows,H,d].
    """
    q, dtq = _tensor(q)
    B, Tq, H, d = q.shape
    k_win, dtw = _tensor(k_win)
    v_win, dtw2 = _tensor(v_win)
    assert dtw == dtw2 and k_win.shape == v_win.shape and k_win.shape[0] == B
    win_len = k_win.shape[1]
    if kc is None:
        n_cap, dtc = 0, DT_F32
    else:
        kc, dtc = _tensor(kc)
        vc, dtc2 = _tensor(vc)
        assert dtc == dtc2 and kc.shape == vc.shape
        n_cap = kc.shape[1]
    ql, dtg = _tensor(q_lat)
    wg, dtg2 = _tensor(w_gate)
    d_lat = 0
    if ql is not None:
        assert dtg == dtg2
        d_lat = ql.shape[-1]
    pos0 = np.ascontiguousarray(np.asarray(pos0, dtype=np.int32))
    rows = _rows(rows, B * Tq)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((len(rows), H, d), dtype=np.float64)
    rc = _load().orc_hca_attn(_ptr(q), dtq, B, Tq, H, d, _ptr(pos0), _ptr(k_win), _ptr(v_win),
                              dtw, win_len, window, _ptr(kc), _ptr(vc), dtc, n_cap, block,
                              float(scale), _ptr(ql), _ptr(wg), dtg, d_lat, _ptr(rows),
                              len(rows), _ptr(out))
    _check(rc, "hca_attn")
    return out


def latent_gate(q_lat, w_gate, o, rows=None):
    """out[m,n] = o[m,n] * sigmoid(q_lat[m] . w_gate[:,n]) for the listed rows m."""
    ql, dtl = _tensor(q_lat)
    w, dtw = _tensor(w_gate)
    o, dto = _tensor(o)
    M, d_lat = ql.shape
    N = w.shape[1]
    assert o.shape == (M, N) and w.shape[0] == d_lat
    rows = _rows(rows, M)
    out = np.zeros((len(rows), N), dtype=np.float64)
    _check(_load().orc_latent_gate(_ptr(ql), dtl, _ptr(w), dtw, _ptr(o), dto, M, d_lat, N,
                                   _ptr(rows), len(rows), _ptr(out)), "latent_gate")
    return out


def dsa_scores(q_idx, w_idx, k_idx, b, i, s0, s1):
    """float64 indexer scores of query row (b, i) for positions [s0, s1)."""
    q_idx = np.ascontiguousarray(q_idx, dtype=np.float32)
    w_idx = np.ascontiguousarray(w_idx, dtype=np.float32)
    k_idx = np.ascontiguousarray(k_idx, dtype=np.float32)
    B, Tq, Hi, di = q_idx.shape
    S = k_idx.shape[1]
    out = np.zeros(s1 - s0, dtype=np.float64)
    _check(_load().orc_dsa_scores(_ptr(q_idx), _ptr(w_idx), _ptr(k_idx), B, Tq, S, Hi, di, b,
                                  i, s0, s1, _ptr(out)), "dsa_scores")
    return out


def dsa_topk(q_idx, w_idx, k_idx, pos0, k, rows=None, block=1):
    """Top-k keys per query row (ascending, -1 padded) and the k-th highest score.  block > 1:
    key s is the compressed entry of positions block*s .. block*s + block - 1, visible to the
    query at t once complete (s < (t + 1) // block)."""
    q_idx = np.ascontiguousarray(q_idx, dtype=np.float32)
    w_idx = np.ascontiguousarray(w_idx, dtype=np.float32)
    k_idx = np.ascontiguousarray(k_idx, dtype=np.float32)
    B, Tq, Hi, di = q_idx.shape
    S = k_idx.shape[1]
    pos0 = np.ascontiguousarray(np.asarray(pos0, dtype=np.int32))
    rows = _rows(rows, B * Tq)
    idx = np.zeros((len(rows), k), dtype=np.int32)
    kth = np.zeros(len(rows), dtype=np.float64)
    _check(_load().orc_dsa_topk(_ptr(q_idx), _ptr(w_idx), _ptr(k_idx), B, Tq, S, Hi, di, k,
                                int(block), _ptr(pos0), _ptr(rows), len(rows), _ptr(idx),
                                _ptr(kth)),
           "dsa_topk")
    return idx, kth


def sparse_attn(q, k_lat, idx, v_lat=None, *, dqk=None, dv=None, scale=None, q_lat=None,
                w_gate=None, rows=None):
    """Sparse core attention over the latent rows listed in idx (negative entries skipped).

    q [B,Tq,H,dqk]; k_lat [B,S,k_stride] (key = first dqk entries of a row); v_lat
    [B,S,v_stride] or None for V = K (value = first dv entries); idx [B,Tq,k] int32.
    Returns float64 [n_rows,H,dv].
    """
    q, dtq = _tensor(q)
    B, Tq, H, dq = q.shape
    k_lat, dtk = _tensor(k_lat)
    if v_lat is None:
        v_lat, dtv = k_lat, dtk
    else:
        v_lat, dtv = _tensor(v_lat)
    assert dtk == dtv
    S, k_stride = k_lat.shape[1], k_lat.shape[2]
    v_stride = v_lat.shape[2]
    dqk = dq if dqk is None else dqk
    dv = v_stride if dv is None else dv
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    k = idx.shape[-1]
    ql, dtg = _tensor(q_lat)
    wg, dtg2 = _tensor(w_gate)
    d_lat = 0 if ql is None else ql.shape[-1]
    rows = _rows(rows, B * Tq)
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    out = np.zeros((len(rows), H, dv), dtype=np.float64)
    rc = _load().orc_sparse_attn(_ptr(q), dtq, B, Tq, H, dqk, dv, _ptr(k_lat), k_stride,
                                 _ptr(v_lat), v_stride, dtk, S, _ptr(idx), k, float(scale),
                                 _ptr(ql), _ptr(wg), dtg, d_lat, _ptr(rows), len(rows),
                                 _ptr(out))
    _check(rc, "sparse_attn")
    return out


def csa_attn(q, pos0, k, v, q_idx, w_idx, k_idx, k_top, *, block=4, scale=None, q_lat=None,
             w_gate=None, rows=None):
    """Compressed sparse attention (the variant of [blog 2.1] that compresses history, then
    attends to a sparse part of it), in the steps the pages name, taken as the other layers
    take them: K, V and the indexer keys are mean-pooled over complete blocks of `block`
    tokens (hca_compress); the indexer scores the compressed entries a query can see (its
    block complete) and keeps the top k_top (dsa_topk with block); softmax attention runs over
    the kept entries (sparse_attn, values distinct from keys), gated when q_lat is given.

    q [B,T,H,d]; k, v [B,T,d] (the layer's keys and values of every position; rows beyond the
    last complete block are ignored); q_idx [B,T,Hi,64]; w_idx [B,T,Hi]; k_idx [B,T,64].
    Returns (float64 out [n_rows,H,d], idx [n_rows,k_top], kth [n_rows], compressed keys,
    compressed values, compressed indexer keys as float32).
    """
    kc = hca_compress(k, block)
    vc = hca_compress(v, block)
    kic = hca_compress(k_idx, block).astype(np.float32)
    B, T = np.asarray(q_idx).shape[:2]
    rows = _rows(rows, B * T)
    idx, kth = dsa_topk(q_idx, w_idx, kic, pos0, k_top, rows=rows, block=block)
    full = np.full((B, T, k_top), -1, np.int32)
    for j, r in enumerate(rows):
        full[r // T, r % T] = idx[j]
    out = sparse_attn(q, kc, full, v_lat=vc, scale=scale, q_lat=q_lat, w_gate=w_gate,
                      rows=rows)
    return out, idx, kth, kc, vc, kic
