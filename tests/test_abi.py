"""The C-ABI library loads, exports every symbol include/lgsa.h declares, and rejects bad
arguments on the host with the documented status codes before touching the GPU.

These run without a GPU: every call here is made with arguments that fail validation (or is a
workspace query, which is host arithmetic only), so no kernel is ever enqueued.
"""
import ctypes
import os
import re

import pytest

import hybrid_sparse_attention_amd as lgsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lgsa.h")
FAKE = 0x10000  # a 16-byte aligned non-NULL address; never dereferenced on these paths
FAKE_ODD = 0x10002


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lgsa.LIB_PATH):
        from hybrid_sparse_attention_amd import build

        build.build()
    return lgsa.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(?:lgsa_status|const char\*)\s+(\w+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = _declared()
    for n in ("hca_compress", "hca_attn_fwd", "dsa_index_topk", "sparse_attn_fwd",
              "latent_gate"):
        assert n in names
    assert sorted(names) == sorted(lgsa.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    # and the binding declares argument lists for all of them
    for name in lgsa.EXPORTS:
        assert getattr(lib, name).argtypes is not None or name == "lgsa_last_error"


def _status(rc):
    return rc, lgsa.last_error()


def test_compress_validation(lib):
    f = lib.hca_compress
    assert _status(f(None, FAKE, FAKE, FAKE, 1, 256, 512, 128, 1, None))[0] == lgsa.LGSA_EINVAL
    assert "non-NULL" in lgsa.last_error()
    assert f(FAKE, FAKE, None, FAKE, 1, 256, 512, 128, 1, None) == lgsa.LGSA_EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 256, 512, 128, 7, None) == lgsa.LGSA_EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 256, 512, 0, 1, None) == lgsa.LGSA_EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 256, 12, 128, 1, None) == lgsa.LGSA_EUNSUPPORTED
    assert f(FAKE_ODD, FAKE, FAKE, FAKE, 1, 256, 512, 128, 1, None) == lgsa.LGSA_EINVAL
    assert "aligned" in lgsa.last_error()


def test_gate_validation(lib):
    f = lib.latent_gate
    assert f(FAKE, FAKE, FAKE, FAKE, 10, 0, 64, 1, None) == lgsa.LGSA_EINVAL
    assert f(FAKE, None, FAKE, FAKE, 10, 64, 64, 1, None) == lgsa.LGSA_EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, 10, 100, 64, 1, None) == lgsa.LGSA_EUNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, 10, 64, 24, 1, None) == lgsa.LGSA_EUNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, 10, 64, 64, 5, None) == lgsa.LGSA_EINVAL
    # the bf16 kernels read o and write out 16 bytes at a time: an 8-byte aligned view is refused
    FAKE8 = FAKE + 8
    assert f(FAKE, FAKE, FAKE8, FAKE, 10, 64, 64, 1, None) == lgsa.LGSA_EINVAL
    assert "aligned" in lgsa.last_error()
    assert f(FAKE, FAKE, FAKE, FAKE8, 10, 64, 64, 1, None) == lgsa.LGSA_EINVAL


def _hca(**kw):
    a = lgsa.HcaArgs()
    vals = dict(dt=1, B=1, Tq=256, H=64, d=512, q=FAKE, pos0=FAKE, max_pos=255, k_win=FAKE,
                v_win=FAKE, win_len=256, window=128, kc=FAKE, vc=FAKE, n_cap=2, block=128,
                scale=0.0441941738, q_lat=FAKE, w_gate=FAKE, d_lat=1024, out=FAKE,
                workspace=None, workspace_bytes=0)
    vals.update(kw)
    for k, v in vals.items():
        setattr(a, k, v)
    return a


def _call(lib, name, a):
    return getattr(lib, name)(ctypes.byref(a), None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(B=0), lgsa.LGSA_EINVAL, "must be >= 1"),
    (dict(q=None), lgsa.LGSA_EINVAL, "non-NULL"),
    (dict(window=300, max_pos=300, win_len=256), lgsa.LGSA_EINVAL, "window + Tq - 1"),
    # a multi-row call over a ring of window rows: its rows' windows would alias in the ring
    (dict(Tq=32, win_len=128, window=128, max_pos=1031, n_cap=8), lgsa.LGSA_EINVAL,
     "window + Tq - 1"),
    # a chunk-only window (win_len = Tq) at a later position reaches back before the chunk
    (dict(Tq=256, win_len=256, max_pos=1279, n_cap=9), lgsa.LGSA_EINVAL, "window + Tq - 1"),
    (dict(block=0), lgsa.LGSA_EINVAL, "block"),
    (dict(kc=None), lgsa.LGSA_EINVAL, "kc and vc"),
    (dict(max_pos=10), lgsa.LGSA_EINVAL, "max_pos"),
    (dict(w_gate=None), lgsa.LGSA_EINVAL, "both NULL"),
    (dict(scale=float("inf")), lgsa.LGSA_EINVAL, "scale"),
    (dict(dt=3), lgsa.LGSA_EINVAL, "dt"),
    (dict(d=256), lgsa.LGSA_EUNSUPPORTED, "d == 512"),
    (dict(d_lat=1000), lgsa.LGSA_EUNSUPPORTED, "d_lat"),
    (dict(dt=0, d=600), lgsa.LGSA_EUNSUPPORTED, "d <= 512"),
    (dict(q=FAKE_ODD), lgsa.LGSA_EINVAL, "aligned"),
])
def test_hca_validation(lib, kw, code, msg):
    a = _hca(**kw)
    assert _call(lib, "hca_attn_fwd", a) == code
    assert msg in lgsa.last_error()
    n = ctypes.c_size_t(0)
    assert lib.hca_attn_fwd_workspace(ctypes.byref(a), ctypes.byref(n)) == code


def test_hca_workspace_queries(lib):
    n = ctypes.c_size_t(123)
    # prefill needs no workspace
    assert lib.hca_attn_fwd_workspace(ctypes.byref(_hca()), ctypes.byref(n)) == 0
    assert n.value == 0
    # decode of one long sequence is split over workgroups: partial (m, l, O) per split
    a = _hca(B=1, Tq=1, max_pos=131071, win_len=128, n_cap=1024)
    assert lib.hca_attn_fwd_workspace(ctypes.byref(a), ctypes.byref(n)) == 0
    assert n.value > 0 and n.value % (64 * 4) == 0
    # a decode call without that workspace is refused before any launch
    assert _call(lib, "hca_attn_fwd", a) == lgsa.LGSA_EWORKSPACE
    a.workspace, a.workspace_bytes = FAKE, n.value - 1
    assert _call(lib, "hca_attn_fwd", a) == lgsa.LGSA_EWORKSPACE


def test_hca_static_scratch_limit(lib):
    # decode of 160 sequences x 64 heads needs 42,106,880 bytes of split partials, more than the
    # library's static scratch (40 MiB): refused before anything touches the GPU
    a = _hca(B=160, Tq=1, max_pos=131071, win_len=128, n_cap=1024)
    assert _call(lib, "hca_attn_fwd_static", a) == lgsa.LGSA_EWORKSPACE
    assert "LGSA_STATIC_SCRATCH_BYTES" in lgsa.last_error()
    # arguments are validated exactly as by hca_attn_fwd
    assert _call(lib, "hca_attn_fwd_static", _hca(B=0)) == lgsa.LGSA_EINVAL
    assert _call(lib, "hca_attn_fwd_static", _hca(q=FAKE_ODD)) == lgsa.LGSA_EINVAL


def test_gather_probe_validation(lib):
    f = lib.sparse_gather_probe
    assert f(None, 256, 10, FAKE, 4, 32, FAKE, None) == lgsa.LGSA_EINVAL
    assert f(FAKE, 256, 0, FAKE, 4, 32, FAKE, None) == lgsa.LGSA_EINVAL
    assert f(FAKE, 200, 10, FAKE, 4, 32, FAKE, None) == lgsa.LGSA_EUNSUPPORTED
    assert f(FAKE_ODD, 256, 10, FAKE, 4, 32, FAKE, None) == lgsa.LGSA_EINVAL
    assert "aligned" in lgsa.last_error()


def _idx(**kw):
    a = lgsa.IndexArgs()
    vals = dict(B=1, Tq=4096, S=4096, Hi=4, di=64, k=2048, q_idx=FAKE, w_idx=FAKE, k_idx=FAKE,
                pos0=FAKE, max_pos=4095, idx_out=FAKE, workspace=None, workspace_bytes=0)
    vals.update(kw)
    for k, v in vals.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,code,msg", [
    (dict(S=0), lgsa.LGSA_EINVAL, ">= 1"),
    (dict(k=0), lgsa.LGSA_EINVAL, ">= 1"),
    (dict(max_pos=4096), lgsa.LGSA_EINVAL, "every visible key must exist"),
    (dict(max_pos=4096 * 4 + 3, block=4), lgsa.LGSA_EINVAL, "every visible key must exist"),
    (dict(block=-1), lgsa.LGSA_EINVAL, "block must be >= 0"),
    (dict(max_pos=100), lgsa.LGSA_EINVAL, "max_pos"),
    (dict(idx_out=None), lgsa.LGSA_EINVAL, "non-NULL"),
    (dict(di=128), lgsa.LGSA_EUNSUPPORTED, "di"),
    (dict(Hi=8), lgsa.LGSA_EUNSUPPORTED, "Hi"),
    (dict(k=5000), lgsa.LGSA_EUNSUPPORTED, "k must"),
    (dict(q_idx=FAKE_ODD), lgsa.LGSA_EINVAL, "aligned"),
])
def test_index_validation(lib, kw, code, msg):
    a = _idx(**kw)
    assert _call(lib, "dsa_index_topk", a) == code
    assert msg in lgsa.last_error()


def test_index_block_bounds_the_keys(lib):
    """With block 4, (max_pos + 1) / 4 keys must exist: S = 1024 serves max_pos up to 4098
    (the call then only lacks its workspace), and the recommended workspace holds the scores of
    that many keys per query chunk."""
    n4, n1 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    a4 = _idx(S=1024, max_pos=4098, block=4)
    assert _call(lib, "dsa_index_topk", a4) == lgsa.LGSA_EWORKSPACE
    assert lib.dsa_index_topk_workspace(ctypes.byref(a4), ctypes.byref(n4)) == lgsa.LGSA_OK
    a1 = _idx(S=4096, max_pos=4095)
    assert lib.dsa_index_topk_workspace(ctypes.byref(a1), ctypes.byref(n1)) == lgsa.LGSA_OK
    assert n4.value * 4 == n1.value


def test_index_workspace(lib):
    n = ctypes.c_size_t(0)
    a = _idx()
    assert lib.dsa_index_topk_workspace(ctypes.byref(a), ctypes.byref(n)) == 0
    assert n.value >= 4096 * 4  # at least one row of scores
    assert _call(lib, "dsa_index_topk", a) == lgsa.LGSA_EWORKSPACE
    d = _idx(B=8, Tq=1, S=1 << 20, max_pos=(1 << 20) - 1)
    assert lib.dsa_index_topk_workspace(ctypes.byref(d), ctypes.byref(n)) == 0
    # decode: candidate lists of 64 segments of 16384 positions (k keys, k positions, a count
    # and the segment's bound each), then 16 filtered lists of 4 segments (4k keys, 4k
    # positions and a count each)
    seg, grp = 8 * 64, 8 * 16
    assert n.value == seg * (2048 * 8 + 8) + grp * (4 * 2048 * 8 + 4)


def _sp(**kw):
    a = lgsa.SparseArgs()
    vals = dict(dt=1, B=1, Tq=16, H=64, d_qk=256, d_v=256, S=4096, k=2048, q=FAKE, k_lat=FAKE,
                k_row_stride=256, v_lat=FAKE, v_row_stride=256, idx=FAKE, scale=0.0625,
                q_lat=None, w_gate=None, d_lat=0, out=FAKE, workspace=None, workspace_bytes=0)
    vals.update(kw)
    for k, v in vals.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,code,msg", [
    (dict(k=0), lgsa.LGSA_EINVAL, ">= 1"),
    (dict(idx=None), lgsa.LGSA_EINVAL, "non-NULL"),
    (dict(k_row_stride=128), lgsa.LGSA_EINVAL, "strides"),
    (dict(q_lat=FAKE), lgsa.LGSA_EINVAL, "both NULL"),
    (dict(dt=0), lgsa.LGSA_EUNSUPPORTED, "bf16"),
    (dict(d_qk=128), lgsa.LGSA_EUNSUPPORTED, "256"),
    (dict(H=48), lgsa.LGSA_EUNSUPPORTED, "multiple of 64"),
    (dict(k_row_stride=260), lgsa.LGSA_EUNSUPPORTED, "multiples of 8"),
    (dict(out=FAKE_ODD), lgsa.LGSA_EINVAL, "aligned"),
])
def test_sparse_validation(lib, kw, code, msg):
    a = _sp(**kw)
    assert _call(lib, "sparse_attn_fwd", a) == code
    assert msg in lgsa.last_error()


def test_sparse_workspace_split_for_few_rows(lib):
    n = ctypes.c_size_t(0)
    assert lib.sparse_attn_fwd_workspace(ctypes.byref(_sp(Tq=4096)), ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.sparse_attn_fwd_workspace(ctypes.byref(_sp(B=8, Tq=1)), ctypes.byref(n)) == 0
    assert n.value > 0
    assert _call(lib, "sparse_attn_fwd", _sp(B=8, Tq=1)) == lgsa.LGSA_EWORKSPACE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(lgsa, "_lib", None)
    monkeypatch.setattr(lgsa, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(lgsa.LibraryMissing):
        lgsa.load()


def _hca_append_args(**kw):
    a = lgsa.HcaAppendArgs()
    base = dict(dt=1, B=2, d=512, pos=FAKE, k_new=FAKE, v_new=FAKE, k_win=FAKE, v_win=FAKE,
                win_len=128, kc=FAKE, vc=FAKE, n_cap=4, block=128)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,code,msg", [
    (dict(dt=5), lgsa.LGSA_EINVAL, "dt"),
    (dict(B=-1), lgsa.LGSA_EINVAL, ">= 0"),
    (dict(win_len=0), lgsa.LGSA_EINVAL, ">= 1"),
    (dict(k_new=None), lgsa.LGSA_EINVAL, "non-NULL"),
    (dict(kc=None), lgsa.LGSA_EINVAL, "kc and vc"),
    (dict(win_len=64), lgsa.LGSA_EINVAL, "whole block"),
    (dict(d=12), lgsa.LGSA_EUNSUPPORTED, "multiple of 8"),
    (dict(v_win=FAKE_ODD), lgsa.LGSA_EINVAL, "aligned"),
])
def test_hca_append_validation(lib, kw, code, msg):
    assert lib.hca_cache_append(ctypes.byref(_hca_append_args(**kw)), None) == code
    assert msg in lgsa.last_error()


def test_hca_append_without_entries_needs_no_cache(lib):
    # n_cap == 0: kc / vc may be NULL and the ring may be shorter than a block; with B == 0
    # nothing is enqueued, so this runs without a GPU
    a = _hca_append_args(B=0, kc=None, vc=None, n_cap=0, win_len=16)
    assert lib.hca_cache_append(ctypes.byref(a), None) == lgsa.LGSA_OK


def _dsa_append_args(**kw):
    a = lgsa.DsaAppendArgs()
    base = dict(dt=1, B=2, S=1000, pos=FAKE, k_idx_new=FAKE, k_idx=FAKE, di=64, kv_new=FAKE,
                kv_lat=FAKE, row=256, kv_row_stride=256)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,code,msg", [
    (dict(S=0), lgsa.LGSA_EINVAL, ">= 1"),
    (dict(kv_row_stride=128), lgsa.LGSA_EINVAL, "kv_row_stride"),
    (dict(kv_lat=None), lgsa.LGSA_EINVAL, "non-NULL"),
    (dict(di=6), lgsa.LGSA_EUNSUPPORTED, "multiple"),
    (dict(row=252, kv_row_stride=252), lgsa.LGSA_EUNSUPPORTED, "multiple"),
    (dict(k_idx=FAKE_ODD), lgsa.LGSA_EINVAL, "aligned"),
])
def test_dsa_append_validation(lib, kw, code, msg):
    assert lib.dsa_cache_append(ctypes.byref(_dsa_append_args(**kw)), None) == code
    assert msg in lgsa.last_error()


def test_vha_validation(lib):
    f = lib.vha_mix
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 64, 512, 16, 7, None) == lgsa.LGSA_EINVAL
    assert f(None, FAKE, FAKE, FAKE, 4, 64, 512, 16, 1, None) == lgsa.LGSA_EINVAL
    assert "non-NULL" in lgsa.last_error()
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 64, 512, 0, 1, None) == lgsa.LGSA_EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 64, 512, 17, 1, None) == lgsa.LGSA_EUNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 32, 512, 16, 1, None) == lgsa.LGSA_EUNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 64, 320, 16, 1, None) == lgsa.LGSA_EUNSUPPORTED
    assert f(FAKE_ODD, FAKE, FAKE, FAKE, 4, 64, 512, 16, 1, None) == lgsa.LGSA_EINVAL
    assert "aligned" in lgsa.last_error()
    assert f(FAKE, FAKE, FAKE, FAKE, 0, 64, 512, 16, 1, None) == lgsa.LGSA_OK  # M == 0: no work


@pytest.mark.parametrize("kw,code,msg", [
    (dict(dt=7), lgsa.LGSA_EINVAL, "unknown dt"),
    (dict(M=-1), lgsa.LGSA_EINVAL, ">= 0"),
    (dict(dq_lat=None), lgsa.LGSA_EINVAL, "non-NULL"),
    (dict(d_lat=96), lgsa.LGSA_EUNSUPPORTED, "d_lat % 64"),
    (dict(o=FAKE_ODD), lgsa.LGSA_EINVAL, "aligned"),
    (dict(workspace=None), lgsa.LGSA_EWORKSPACE, "workspace"),
    (dict(workspace_bytes=64 * 32 * 2 - 1), lgsa.LGSA_EWORKSPACE, "below"),
])
def test_gate_bwd_validation(lib, kw, code, msg):
    """Invalid arguments are refused before anything is enqueued (the pointers are never
    dereferenced: the calls fail on the host)."""
    a = dict(q_lat=FAKE, w_gate=FAKE, o=FAKE, dout=FAKE, d_o=FAKE, dq_lat=FAKE, dw_gate=FAKE,
             M=64, d_lat=64, N=32, dt=lgsa.LGSA_BF16, workspace=FAKE, workspace_bytes=64 * 32 * 2)
    a.update(kw)
    rc = lib.latent_gate_bwd(a["q_lat"], a["w_gate"], a["o"], a["dout"], a["d_o"], a["dq_lat"],
                             a["dw_gate"], a["M"], a["d_lat"], a["N"], a["dt"], a["workspace"],
                             a["workspace_bytes"], None)
    assert rc == code
    assert msg in lgsa.last_error()


def test_gate_bwd_workspace_size(lib):
    n = ctypes.c_size_t(0)
    assert lib.latent_gate_bwd_workspace(100, 64, 48, lgsa.LGSA_BF16, ctypes.byref(n)) == 0
    assert n.value == 100 * 48 * 2
    assert lib.latent_gate_bwd_workspace(100, 64, 48, lgsa.LGSA_F32, ctypes.byref(n)) == 0
    assert n.value == 100 * 48 * 4


def _hca_bwd(**kw):
    a = lgsa.HcaBwdArgs()
    vals = dict(dt=lgsa.LGSA_BF16, B=1, T=256, H=4, d=512, q=FAKE, k=FAKE, v=FAKE, kc=FAKE,
                vc=FAKE, out=FAKE, lse=FAKE, dout=FAKE, window=128, block=128, scale=0.044,
                dq=FAKE, dk=FAKE, dv=FAKE, workspace=None, workspace_bytes=0)
    vals.update(kw)
    for k, v in vals.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,code,msg", [
    (dict(dt=lgsa.LGSA_F32), lgsa.LGSA_EUNSUPPORTED, "LGSA_BF16"),
    (dict(d=256), lgsa.LGSA_EUNSUPPORTED, "d must be 512"),
    (dict(H=6), lgsa.LGSA_EUNSUPPORTED, "multiple of 4"),
    (dict(window=0), lgsa.LGSA_EINVAL, "window"),
    (dict(window=600), lgsa.LGSA_EINVAL, "window"),
    (dict(lse=None), lgsa.LGSA_EINVAL, "non-NULL"),
    (dict(kc=None), lgsa.LGSA_EINVAL, "kc and vc"),
    (dict(dk=FAKE_ODD), lgsa.LGSA_EINVAL, "aligned"),
    (dict(), lgsa.LGSA_EWORKSPACE, "workspace"),
])
def test_hca_bwd_validation(lib, kw, code, msg):
    a = _hca_bwd(**kw)
    assert _call(lib, "hca_attn_bwd", a) == code
    assert msg in lgsa.last_error()


def test_hca_bwd_short_sequence_needs_no_entries(lib):
    """T below one block: kc and vc may be NULL; the workspace holds no entry gradients."""
    n_short, n_long = ctypes.c_size_t(0), ctypes.c_size_t(0)
    a = _hca_bwd(T=100, kc=None, vc=None)
    assert lib.hca_attn_bwd_workspace(ctypes.byref(a), ctypes.byref(n_short)) == lgsa.LGSA_OK
    b = _hca_bwd(T=100)
    assert lib.hca_attn_bwd_workspace(ctypes.byref(b), ctypes.byref(n_long)) == lgsa.LGSA_OK
    assert n_short.value == n_long.value > 0


FAKE2 = FAKE + 4096


def _sparse_bwd(**kw):
    a = lgsa.SparseBwdArgs()
    vals = dict(dt=lgsa.LGSA_BF16, B=1, Tq=64, H=64, d_qk=256, d_v=256, S=1000, k=128,
                q=FAKE, k_lat=FAKE, k_row_stride=256, v_lat=FAKE, v_row_stride=256, idx=FAKE,
                scale=0.0625, out=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=FAKE, dv=None,
                workspace=None, workspace_bytes=0)
    vals.update(kw)
    for k, v in vals.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,code,msg", [
    (dict(dt=lgsa.LGSA_F32), lgsa.LGSA_EUNSUPPORTED, "LGSA_BF16"),
    (dict(d_qk=128), lgsa.LGSA_EUNSUPPORTED, "256"),
    (dict(H=32), lgsa.LGSA_EUNSUPPORTED, "multiple of 64"),
    (dict(k=0), lgsa.LGSA_EINVAL, ">= 1"),
    (dict(lse=None), lgsa.LGSA_EINVAL, "non-NULL"),
    (dict(v_lat=FAKE2), lgsa.LGSA_EINVAL, "dv may be NULL only"),
    (dict(k_row_stride=260, v_row_stride=260), lgsa.LGSA_EUNSUPPORTED, "multiples of 8"),
    (dict(dq=FAKE_ODD), lgsa.LGSA_EINVAL, "aligned"),
    (dict(), lgsa.LGSA_EWORKSPACE, "workspace"),
])
def test_sparse_bwd_validation(lib, kw, code, msg):
    a = _sparse_bwd(**kw)
    assert _call(lib, "sparse_attn_bwd", a) == code
    assert msg in lgsa.last_error()


def test_sparse_bwd_workspace_sizes(lib):
    """The default workspace holds a whole sequence's contributions up to a budget of about
    8 GiB (bf16 rows of 256 columns, 512 with distinct values); a long prefill is taken in
    chunks; a workspace below the size for one row is refused."""
    def size(**kw):
        n = ctypes.c_size_t(0)
        assert lib.sparse_attn_bwd_workspace(ctypes.byref(_sparse_bwd(**kw)), ctypes.byref(n)) == 0
        return n.value
    small = size(Tq=64, k=128)
    assert small >= 64 * 128 * (256 * 2 + 4)
    big = size(Tq=65536, S=65536, k=2048)
    assert 8 << 30 <= big <= 9 << 30
    assert size(Tq=64, k=128, v_lat=FAKE2, dv=FAKE) > small
    a = _sparse_bwd(Tq=64, k=128, workspace=FAKE, workspace_bytes=1024)
    assert _call(lib, "sparse_attn_bwd", a) == lgsa.LGSA_EWORKSPACE

