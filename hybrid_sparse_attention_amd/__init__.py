"""Python binding of liblgsa.so, the gfx950 Latent-Gated Sparse Attention forward library.

Argument marshalling only: every step of the computation runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  The names and arguments mirror
``include/lgsa.h`` (ERNIE 5.5 Flash Base release blog, section 2.1 "Latent-Gated Sparse
Attention" defines what the calls compute).

If the library has not been built (``python -m hybrid_sparse_attention_amd.build``) every
call raises ``LibraryMissing``: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblgsa.so")

LGSA_OK, LGSA_EINVAL, LGSA_EUNSUPPORTED, LGSA_EWORKSPACE, LGSA_EHIP = 0, -1, -2, -3, -4
LGSA_F32, LGSA_BF16 = 0, 1

EXPORTS = ["lgsa_last_error", "hca_compress", "latent_gate", "hca_attn_fwd",
           "hca_attn_fwd_workspace", "hca_attn_fwd_static", "dsa_index_topk", "dsa_index_topk_workspace",
           "sparse_attn_fwd", "sparse_attn_fwd_workspace", "hca_cache_append",
           "dsa_cache_append", "vha_mix", "latent_gate_bwd", "latent_gate_bwd_workspace",
           "hca_attn_bwd", "hca_attn_bwd_workspace",
           "sparse_attn_bwd", "sparse_attn_bwd_workspace", "sparse_gather_probe"]


class LibraryMissing(RuntimeError):
    pass


class LgsaError(RuntimeError):
    def __init__(self, name, code, msg):
        super().__init__("%s failed with status %d: %s" % (name, code, msg))
        self.code = code


_P, _I, _SZ, _F, _LL = (ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float,
                        ctypes.c_longlong)


class HcaArgs(ctypes.Structure):
    _fields_ = [("dt", _I), ("B", _I), ("Tq", _I), ("H", _I), ("d", _I), ("q", _P),
                ("pos0", _P), ("max_pos", _I), ("k_win", _P), ("v_win", _P),
                ("win_len", _I), ("window", _I), ("kc", _P), ("vc", _P), ("n_cap", _I),
                ("block", _I), ("scale", _F), ("q_lat", _P), ("w_gate", _P), ("d_lat", _I),
                ("out", _P), ("workspace", _P), ("workspace_bytes", _SZ), ("lse", _P),
                ("vha_u", _P), ("vha_v", _P), ("vha_rank", _I)]


class HcaBwdArgs(ctypes.Structure):
    _fields_ = [("dt", _I), ("B", _I), ("T", _I), ("H", _I), ("d", _I), ("q", _P), ("k", _P),
                ("v", _P), ("kc", _P), ("vc", _P), ("out", _P), ("lse", _P), ("dout", _P),
                ("window", _I), ("block", _I), ("scale", _F), ("dq", _P), ("dk", _P),
                ("dv", _P), ("workspace", _P), ("workspace_bytes", _SZ)]


class IndexArgs(ctypes.Structure):
    _fields_ = [("B", _I), ("Tq", _I), ("S", _I), ("Hi", _I), ("di", _I), ("k", _I),
                ("q_idx", _P), ("w_idx", _P), ("k_idx", _P), ("pos0", _P), ("max_pos", _I),
                ("idx_out", _P), ("workspace", _P), ("workspace_bytes", _SZ), ("block", _I)]


class SparseArgs(ctypes.Structure):
    _fields_ = [("dt", _I), ("B", _I), ("Tq", _I), ("H", _I), ("d_qk", _I), ("d_v", _I),
                ("S", _I), ("k", _I), ("q", _P), ("k_lat", _P), ("k_row_stride", _LL),
                ("v_lat", _P), ("v_row_stride", _LL), ("idx", _P), ("scale", _F),
                ("q_lat", _P), ("w_gate", _P), ("d_lat", _I), ("out", _P),
                ("workspace", _P), ("workspace_bytes", _SZ), ("lse", _P),
                ("vha_u", _P), ("vha_v", _P), ("vha_rank", _I)]


class SparseBwdArgs(ctypes.Structure):
    _fields_ = [("dt", _I), ("B", _I), ("Tq", _I), ("H", _I), ("d_qk", _I), ("d_v", _I),
                ("S", _I), ("k", _I), ("q", _P), ("k_lat", _P), ("k_row_stride", _LL),
                ("v_lat", _P), ("v_row_stride", _LL), ("idx", _P), ("scale", _F),
                ("out", _P), ("lse", _P), ("dout", _P), ("dq", _P), ("dk", _P), ("dv", _P),
                ("workspace", _P), ("workspace_bytes", _SZ)]


class HcaAppendArgs(ctypes.Structure):
    _fields_ = [("dt", _I), ("B", _I), ("d", _I), ("pos", _P), ("k_new", _P), ("v_new", _P),
                ("k_win", _P), ("v_win", _P), ("win_len", _I), ("kc", _P), ("vc", _P),
                ("n_cap", _I), ("block", _I)]


class DsaAppendArgs(ctypes.Structure):
    _fields_ = [("dt", _I), ("B", _I), ("S", _I), ("pos", _P), ("k_idx_new", _P),
                ("k_idx", _P), ("di", _I), ("kv_new", _P), ("kv_lat", _P), ("row", _I),
                ("kv_row_stride", _LL)]


_lib = None


def load():
    """Load liblgsa.so (raises LibraryMissing if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing("%s is not built: run python -m hybrid_sparse_attention_amd.build"
                                 % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        lib.lgsa_last_error.restype = ctypes.c_char_p
        lib.lgsa_last_error.argtypes = []
        lib.hca_compress.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P]
        lib.latent_gate.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _P]
        for name, st in (("hca_attn_fwd", HcaArgs), ("dsa_index_topk", IndexArgs),
                         ("sparse_attn_fwd", SparseArgs), ("hca_attn_bwd", HcaBwdArgs),
                         ("sparse_attn_bwd", SparseBwdArgs)):
            getattr(lib, name).argtypes = [ctypes.POINTER(st), _P]
            getattr(lib, name + "_workspace").argtypes = [ctypes.POINTER(st),
                                                          ctypes.POINTER(_SZ)]
        lib.hca_attn_fwd_static.argtypes = [ctypes.POINTER(HcaArgs), _P]
        lib.sparse_gather_probe.argtypes = [_P, _LL, _I, _P, _I, _I, _P, _P]
        lib.vha_mix.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P]
        lib.latent_gate_bwd.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _SZ,
                                        _P]
        lib.latent_gate_bwd_workspace.argtypes = [_I, _I, _I, _I, ctypes.POINTER(_SZ)]
        lib.hca_cache_append.argtypes = [ctypes.POINTER(HcaAppendArgs), _P]
        lib.dsa_cache_append.argtypes = [ctypes.POINTER(DsaAppendArgs), _P]
        for name in EXPORTS[1:]:
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def last_error() -> str:
    return load().lgsa_last_error().decode()


def _check(name, rc):
    if rc != LGSA_OK:
        raise LgsaError(name, rc, last_error())


# ----------------------------------------------------------------------------- torch helpers
def _torch():
    import torch

    return torch


def _dt(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return LGSA_BF16
    if t.dtype == torch.float32:
        return LGSA_F32
    raise TypeError("tensors must be bfloat16 or float32, got %s" % t.dtype)


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(nbytes, device):
    torch = _torch()
    if nbytes == 0:
        return None, 0
    buf = torch.empty(int(nbytes), dtype=torch.uint8, device=device)
    return buf, int(nbytes)


# ----------------------------------------------------------------------------- calls
def hca_compress(k, v, kc=None, vc=None, block=128, stream=None):
    """Mean of each complete block of `block` rows: k, v [B,T,d] -> kc, vc [B,T//block,d]."""
    torch = _torch()
    B, T, d = k.shape
    if kc is None:
        kc = torch.empty((B, T // block, d), dtype=k.dtype, device=k.device)
    if vc is None:
        vc = torch.empty((B, T // block, d), dtype=v.dtype, device=v.device)
    rc = load().hca_compress(_dev(k, "k"), _dev(v, "v"), _dev(kc, "kc"), _dev(vc, "vc"), B, T,
                             d, block, _dt(k), _stream(stream))
    _check("hca_compress", rc)
    return kc, vc


def latent_gate(q_lat, w_gate, o, out=None, stream=None):
    """out = o * sigmoid(q_lat @ w_gate) with q_lat [M,d_lat], w_gate [d_lat,N], o [M,N]."""
    torch = _torch()
    M, d_lat = q_lat.shape
    N = w_gate.shape[1]
    if out is None:
        out = torch.empty_like(o)
    rc = load().latent_gate(_dev(q_lat, "q_lat"), _dev(w_gate, "w_gate"), _dev(o, "o"),
                            _dev(out, "out"), M, d_lat, N, _dt(o), _stream(stream))
    _check("latent_gate", rc)
    return out


def hca_args(q, pos0, k_win, v_win, kc=None, vc=None, *, max_pos, window=128, block=128,
             scale=None, q_lat=None, w_gate=None, out=None):
    B, Tq, H, d = q.shape
    a = HcaArgs()
    a.dt = _dt(q)
    a.B, a.Tq, a.H, a.d = B, Tq, H, d
    a.q = _dev(q, "q")
    a.pos0 = _dev(pos0, "pos0")
    a.max_pos = int(max_pos)
    a.k_win, a.v_win = _dev(k_win, "k_win"), _dev(v_win, "v_win")
    a.win_len = k_win.shape[1]
    a.window = window
    a.kc = _dev(kc, "kc")
    a.vc = _dev(vc, "vc")
    a.n_cap = 0 if kc is None else kc.shape[1]
    a.block = block
    a.scale = 1.0 / math.sqrt(d) if scale is None else scale
    a.q_lat = _dev(q_lat, "q_lat")
    a.w_gate = _dev(w_gate, "w_gate")
    a.d_lat = 0 if q_lat is None else q_lat.shape[-1]
    a.out = _dev(out, "out")
    return a


def hca_attn_fwd(q, pos0, k_win, v_win, kc=None, vc=None, *, max_pos, window=128, block=128,
                 scale=None, q_lat=None, w_gate=None, out=None, workspace=None, stream=None,
                 lse=None, vha_u=None, vha_v=None):
    """Heavily Compressed Attention forward (optionally gated, then optionally mixed across
    heads by VHA with factors vha_u, vha_v [H, r]); see include/lgsa.h.  lse: an optional
    [B, Tq, H] fp32 tensor receiving each row's log-sum-exp (for hca_attn_bwd)."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(q)
    a = hca_args(q, pos0, k_win, v_win, kc, vc, max_pos=max_pos, window=window, block=block,
                 scale=scale, q_lat=q_lat, w_gate=w_gate, out=out)
    a.lse = _dev(lse, "lse")
    _set_vha(a, vha_u, vha_v)
    need = hca_attn_fwd_workspace(a)
    if workspace is None:
        workspace, _ = _workspace(need, q.device)
    a.workspace = None if workspace is None else workspace.data_ptr()
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("hca_attn_fwd", load().hca_attn_fwd(ctypes.byref(a), _stream(stream)))
    return out


def hca_attn_fwd_static(q, pos0, k_win, v_win, kc=None, vc=None, *, max_pos, window=128,
                        block=128, scale=None, q_lat=None, w_gate=None, out=None, stream=None,
                        lse=None):
    """hca_attn_fwd without a workspace: the library's per-GPU static scratch serves the
    decode partials (see include/lgsa.h).  Allocates only `out` when it is not given."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(q)
    a = hca_args(q, pos0, k_win, v_win, kc, vc, max_pos=max_pos, window=window, block=block,
                 scale=scale, q_lat=q_lat, w_gate=w_gate, out=out)
    a.lse = _dev(lse, "lse")
    _check("hca_attn_fwd_static", load().hca_attn_fwd_static(ctypes.byref(a), _stream(stream)))
    return out


def hca_attn_fwd_workspace(a) -> int:
    n = _SZ(0)
    _check("hca_attn_fwd_workspace", load().hca_attn_fwd_workspace(ctypes.byref(a),
                                                                   ctypes.byref(n)))
    return n.value


def index_args(q_idx, w_idx, k_idx, pos0, k, *, max_pos, idx_out=None, block=1):
    B, Tq, Hi, di = q_idx.shape
    a = IndexArgs()
    a.block = int(block)
    a.B, a.Tq, a.S, a.Hi, a.di, a.k = B, Tq, k_idx.shape[1], Hi, di, k
    a.q_idx, a.w_idx, a.k_idx = _dev(q_idx, "q_idx"), _dev(w_idx, "w_idx"), _dev(k_idx, "k_idx")
    a.pos0 = _dev(pos0, "pos0")
    a.max_pos = int(max_pos)
    a.idx_out = _dev(idx_out, "idx_out")
    return a


def dsa_index_topk_workspace(a) -> int:
    n = _SZ(0)
    _check("dsa_index_topk_workspace", load().dsa_index_topk_workspace(ctypes.byref(a),
                                                                       ctypes.byref(n)))
    return n.value


def dsa_index_topk(q_idx, w_idx, k_idx, pos0, k, *, max_pos, idx_out=None, workspace=None,
                   stream=None, block=1):
    """Indexer scores + per-query top-k keys (ascending, -1 padded); see lgsa.h.  block > 1:
    key s is the compressed entry of positions block*s .. block*s + block - 1."""
    torch = _torch()
    B, Tq = q_idx.shape[:2]
    if idx_out is None:
        idx_out = torch.empty((B, Tq, k), dtype=torch.int32, device=q_idx.device)
    a = index_args(q_idx, w_idx, k_idx, pos0, k, max_pos=max_pos, idx_out=idx_out, block=block)
    if workspace is None:
        workspace, _ = _workspace(dsa_index_topk_workspace(a), q_idx.device)
    a.workspace = None if workspace is None else workspace.data_ptr()
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_index_topk", load().dsa_index_topk(ctypes.byref(a), _stream(stream)))
    return idx_out


def sparse_args(q, k_lat, idx, v_lat=None, *, scale=None, q_lat=None, w_gate=None, out=None,
                d_qk=None, d_v=None):
    B, Tq, H, dq = q.shape
    if v_lat is None:
        v_lat = k_lat
    a = SparseArgs()
    a.dt = _dt(q)
    a.B, a.Tq, a.H = B, Tq, H
    a.d_qk = dq if d_qk is None else d_qk
    a.d_v = v_lat.shape[-1] if d_v is None else d_v
    a.S = k_lat.shape[1]
    a.k = idx.shape[-1]
    a.q = _dev(q, "q")
    a.k_lat, a.k_row_stride = _dev(k_lat, "k_lat"), k_lat.shape[-1]
    a.v_lat, a.v_row_stride = _dev(v_lat, "v_lat"), v_lat.shape[-1]
    a.idx = _dev(idx, "idx")
    a.scale = 1.0 / math.sqrt(a.d_qk) if scale is None else scale
    a.q_lat = _dev(q_lat, "q_lat")
    a.w_gate = _dev(w_gate, "w_gate")
    a.d_lat = 0 if q_lat is None else q_lat.shape[-1]
    a.out = _dev(out, "out")
    return a


def sparse_attn_fwd_workspace(a) -> int:
    n = _SZ(0)
    _check("sparse_attn_fwd_workspace", load().sparse_attn_fwd_workspace(ctypes.byref(a),
                                                                         ctypes.byref(n)))
    return n.value


def _set_vha(a, vha_u, vha_v):
    """The optional head mix (VHA) factors [H, r] of an attention call."""
    a.vha_u, a.vha_v = _dev(vha_u, "vha_u"), _dev(vha_v, "vha_v")
    a.vha_rank = 0 if vha_u is None else vha_u.shape[-1]


def sparse_attn_fwd(q, k_lat, idx, v_lat=None, *, scale=None, q_lat=None, w_gate=None,
                    out=None, lse=None, workspace=None, stream=None, vha_u=None, vha_v=None):
    """DSA sparse core attention over the latent rows listed in idx (optionally gated, then
    optionally mixed across heads by VHA with factors vha_u, vha_v [H, r]); lse [B,Tq,H] fp32,
    when given, receives each row's log-sum-exp for sparse_attn_bwd."""
    torch = _torch()
    B, Tq, H, _ = q.shape
    dv = (k_lat if v_lat is None else v_lat).shape[-1]
    if out is None:
        out = torch.empty((B, Tq, H, dv), dtype=q.dtype, device=q.device)
    a = sparse_args(q, k_lat, idx, v_lat, scale=scale, q_lat=q_lat, w_gate=w_gate, out=out)
    a.lse = _dev(lse, "lse")
    _set_vha(a, vha_u, vha_v)
    if workspace is None:
        workspace, _ = _workspace(sparse_attn_fwd_workspace(a), q.device)
    a.workspace = None if workspace is None else workspace.data_ptr()
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("sparse_attn_fwd", load().sparse_attn_fwd(ctypes.byref(a), _stream(stream)))
    return out


def _sparse_bwd_args(q, k_lat, idx, out, lse, dout, v_lat, scale, dq, dk, dv):
    B, Tq, H, d_qk = q.shape
    vl = k_lat if v_lat is None else v_lat
    a = SparseBwdArgs()
    a.dt = _dt(q)
    a.B, a.Tq, a.H, a.d_qk, a.d_v = B, Tq, H, d_qk, dout.shape[-1]
    a.S, a.k = k_lat.shape[1], idx.shape[-1]
    a.q = _dev(q, "q")
    a.k_lat, a.k_row_stride = _dev(k_lat, "k_lat"), k_lat.shape[-1]
    a.v_lat, a.v_row_stride = _dev(vl, "v_lat"), vl.shape[-1]
    a.idx = _dev(idx, "idx")
    a.scale = 1.0 / math.sqrt(d_qk) if scale is None else scale
    a.out, a.lse, a.dout = _dev(out, "out"), _dev(lse, "lse"), _dev(dout, "dout")
    a.dq, a.dk, a.dv = _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv")
    return a


def sparse_attn_bwd(q, k_lat, idx, out, lse, dout, v_lat=None, *, scale=None, dq=None,
                    dk=None, dv=None, workspace=None, stream=None):
    """Backward of sparse_attn_fwd: returns (dq [B,Tq,H,256], dk [B,S,256], dv [B,S,256] or None
    when v_lat is None, in which case dk holds the key and value gradients of the shared latent
    rows); see include/lgsa.h.  out and lse are the forward's (ungated) output and
    log-sum-exp.  A workspace smaller than sparse_attn_bwd_workspace_bytes() makes the call
    take fewer query rows at a time."""
    torch = _torch()
    B, Tq, H, d_qk = q.shape
    S = k_lat.shape[1]
    dq = torch.empty_like(q) if dq is None else dq
    if dk is None:
        dk = torch.empty((B, S, d_qk), dtype=q.dtype, device=q.device)
    if v_lat is not None and dv is None:
        dv = torch.empty((B, S, dout.shape[-1]), dtype=q.dtype, device=q.device)
    a = _sparse_bwd_args(q, k_lat, idx, out, lse, dout, v_lat, scale, dq, dk, dv)
    if workspace is None:
        n = _SZ(0)
        _check("sparse_attn_bwd_workspace", load().sparse_attn_bwd_workspace(ctypes.byref(a),
                                                                             ctypes.byref(n)))
        workspace, _ = _workspace(n.value, q.device)
    a.workspace = None if workspace is None else workspace.data_ptr()
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("sparse_attn_bwd", load().sparse_attn_bwd(ctypes.byref(a), _stream(stream)))
    return dq, dk, dv


def sparse_attn_bwd_workspace_bytes(q, k_lat, idx, out, lse, dout, v_lat=None) -> int:
    """Default workspace of sparse_attn_bwd for these tensors (gradients assumed separate for
    distinct values)."""
    a = _sparse_bwd_args(q, k_lat, idx, out, lse, dout, v_lat, None, q, q,
                         None if v_lat is None else q)
    n = _SZ(0)
    _check("sparse_attn_bwd_workspace", load().sparse_attn_bwd_workspace(ctypes.byref(a),
                                                                         ctypes.byref(n)))
    return n.value


def hca_attn_bwd(q, k, v, kc, vc, out, lse, dout, *, window=128, block=128, scale=None,
                 dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Backward of hca_attn_fwd in prefill (sequences from position 0, window rows = k, v):
    returns (dq [B,T,H,d], dk [B,T,d], dv [B,T,d]); see include/lgsa.h.  out and lse are the
    forward's (ungated) output and log-sum-exp."""
    torch = _torch()
    B, T, H, d = q.shape
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    a = HcaBwdArgs()
    a.dt = _dt(q)
    a.B, a.T, a.H, a.d = B, T, H, d
    a.q, a.k, a.v = _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    a.kc, a.vc = _dev(kc, "kc"), _dev(vc, "vc")
    a.out, a.lse, a.dout = _dev(out, "out"), _dev(lse, "lse"), _dev(dout, "dout")
    a.window, a.block = window, block
    a.scale = 1.0 / math.sqrt(d) if scale is None else scale
    a.dq, a.dk, a.dv = _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv")
    n = _SZ(0)
    _check("hca_attn_bwd_workspace", load().hca_attn_bwd_workspace(ctypes.byref(a),
                                                                   ctypes.byref(n)))
    if workspace is None:
        workspace, _ = _workspace(n.value, q.device)
    a.workspace = None if workspace is None else workspace.data_ptr()
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("hca_attn_bwd", load().hca_attn_bwd(ctypes.byref(a), _stream(stream)))
    return dq, dk, dv


def latent_gate_bwd(q_lat, w_gate, o, dout, d_o=None, dq_lat=None, dw_gate=None, *,
                    workspace=None, stream=None):
    """Backward of latent_gate: (d_o, dq_lat, dw_gate) for the loss gradient dout with respect
    to out = o * sigmoid(q_lat @ w_gate); see include/lgsa.h."""
    torch = _torch()
    M, d_lat = q_lat.shape
    N = w_gate.shape[1]
    if d_o is None:
        d_o = torch.empty_like(o)
    if dq_lat is None:
        dq_lat = torch.empty_like(q_lat)
    if dw_gate is None:
        dw_gate = torch.empty_like(w_gate)
    n = _SZ(0)
    _check("latent_gate_bwd_workspace",
           load().latent_gate_bwd_workspace(M, d_lat, N, _dt(o), ctypes.byref(n)))
    if workspace is None:
        workspace, _ = _workspace(n.value, o.device)
    rc = load().latent_gate_bwd(_dev(q_lat, "q_lat"), _dev(w_gate, "w_gate"), _dev(o, "o"),
                                _dev(dout, "dout"), _dev(d_o, "d_o"), _dev(dq_lat, "dq_lat"),
                                _dev(dw_gate, "dw_gate"), M, d_lat, N, _dt(o),
                                None if workspace is None else workspace.data_ptr(),
                                0 if workspace is None else
                                workspace.numel() * workspace.element_size(), _stream(stream))
    _check("latent_gate_bwd", rc)
    return d_o, dq_lat, dw_gate


def csa_attn_fwd(q, pos0, k, v, q_idx, w_idx, k_idx, k_top, *, max_pos, block=4, q_lat=None,
                 w_gate=None, out=None, stream=None):
    """Compressed sparse attention, the variant of the release blog's section 2.1 that
    compresses history `block`x and attends to a sparse part of it, composed from three library
    calls: hca_compress pools K, V (bf16, [B,T,256]) and the indexer keys (fp32, [B,T,64]) over
    complete blocks; dsa_index_topk with `block` scores the entries each query can see (its
    block complete) and keeps the top k_top; sparse_attn_fwd attends to the kept entries (values
    distinct from keys), gated when q_lat is given.  q [B,Tq,H,256] sits at positions pos0[b] +
    i; every T >= block.  Returns (out [B,Tq,H,256], idx [B,Tq,k_top])."""
    if k.shape[1] < block:
        raise ValueError("csa_attn_fwd: the sequence (%d) holds no complete block of %d"
                         % (k.shape[1], block))
    kc, vc = hca_compress(k, v, block=block, stream=stream)
    kic, _ = hca_compress(k_idx, k_idx, block=block, stream=stream)
    idx = dsa_index_topk(q_idx, w_idx, kic, pos0, k_top, max_pos=max_pos, block=block,
                         stream=stream)
    out = sparse_attn_fwd(q, kc, idx, v_lat=vc, q_lat=q_lat, w_gate=w_gate, out=out,
                          stream=stream)
    return out, idx


def hca_cache_append(pos, k_new, v_new, k_win, v_win, kc=None, vc=None, *, block=128,
                     stream=None):
    """Decode-time HCA cache update for each sequence's new token at position pos[b]: ring rows
    k_win / v_win [B,win_len,d] and, on a block's last token, the entry kc / vc [B,n_cap,d]
    (updated in place); see include/lgsa.h."""
    B, d = k_new.shape
    a = HcaAppendArgs()
    a.dt = _dt(k_new)
    a.B, a.d = B, d
    a.pos = _dev(pos, "pos")
    a.k_new, a.v_new = _dev(k_new, "k_new"), _dev(v_new, "v_new")
    a.k_win, a.v_win = _dev(k_win, "k_win"), _dev(v_win, "v_win")
    a.win_len = k_win.shape[1]
    a.kc, a.vc = _dev(kc, "kc"), _dev(vc, "vc")
    a.n_cap = 0 if kc is None else kc.shape[1]
    a.block = block
    _check("hca_cache_append", load().hca_cache_append(ctypes.byref(a), _stream(stream)))


def dsa_cache_append(pos, k_idx_new, k_idx, kv_new, kv_lat, stream=None):
    """Decode-time DSA cache append: k_idx[b,pos[b]] = k_idx_new[b] ([B,S,di] fp32) and
    kv_lat[b,pos[b],:row] = kv_new[b] (kv_lat [B,S,stride]), in place; see include/lgsa.h."""
    B, di = k_idx_new.shape
    a = DsaAppendArgs()
    a.dt = _dt(kv_new)
    a.B, a.S = B, k_idx.shape[1]
    a.pos = _dev(pos, "pos")
    a.k_idx_new, a.k_idx = _dev(k_idx_new, "k_idx_new"), _dev(k_idx, "k_idx")
    a.di = di
    a.kv_new, a.kv_lat = _dev(kv_new, "kv_new"), _dev(kv_lat, "kv_lat")
    a.row = kv_new.shape[1]
    a.kv_row_stride = kv_lat.shape[2]
    _check("dsa_cache_append", load().dsa_cache_append(ctypes.byref(a), _stream(stream)))


def vha_mix(o, u, v, out=None, stream=None):
    """Virtual Head Attention mixing step: out = o + U V^T o over the heads of each token, with
    o [M,H,d] (or [B,T,H,d]) and u, v [H,r]; out may be o; see include/lgsa.h."""
    torch = _torch()
    H, d = o.shape[-2], o.shape[-1]
    M = o.numel() // (H * d)
    r = u.shape[1]
    if out is None:
        out = torch.empty_like(o)
    rc = load().vha_mix(_dev(o, "o"), _dev(u, "u"), _dev(v, "v"), _dev(out, "out"), M, H, d, r,
                        _dt(o), _stream(stream))
    _check("vha_mix", rc)
    return out


def sparse_gather_probe(rows, idx, sums=None, stream=None):
    """Measurement helper: the gathers of sparse_attn_fwd alone (see include/lgsa.h).
    rows [S, stride] bf16; idx [n_lists, k] int32.  Returns sums [n_lists, 2] uint32 (as int32)."""
    torch = _torch()
    n_lists, k = idx.shape
    if sums is None:
        sums = torch.empty((n_lists, 2), dtype=torch.int32, device=idx.device)
    _check("sparse_gather_probe",
           load().sparse_gather_probe(_dev(rows, "rows"), rows.shape[-1], rows.shape[0],
                                      _dev(idx, "idx"), n_lists, k, _dev(sums, "sums"),
                                      _stream(stream)))
    return sums
