"""Benchmark of the Latent-Gated Sparse Attention forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--configs 0,1,2,3,4] [--no-cpu]

A step is one pass of the hot path over one batch of synthetic input of the HCA prefill at
model shape (seq 32768, 64 query heads sharing one KV head, head dim 512, bf16, 256 mean-pooled
compressed entries + 128-token window, gate from the 1024-wide query latent): hca_compress,
then hca_attn_fwd with the gate operands, whose kernel applies the gate in the attention
epilogue.  `value` is its algorithmic TFLOP/s (attention over the visible pairs + the gate
GEMM).  `roofline` describes the kernel that takes the largest share of the step, bounded by
MFMA or HBM according to its algorithmic work.  The decode and MLA-DSA workloads are timed too
and reported under "secondary" in the same JSON line.  Inputs are seeded synthetic data already resident
in HBM when timing starts.  The CPU baseline times the fp64 oracle on a bounded sample of
query rows of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HCA/DSA attention prefill TFLOP/s + decode GB/s; % of MI355X roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (matrix / packed vector)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
ORACLE_TIMING = True        # --no-cpu turns the fp64 oracle timings off


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------- work formulas
def hca_pairs(T, block=128, window=128, n_cap=None):
    """Visible (query, key) pairs per head of an HCA prefill from position 0."""
    t = np.arange(T, dtype=np.int64)
    nc = (t + 1) // block
    if n_cap is not None:
        nc = np.minimum(nc, n_cap)
    return int(np.sum(nc + np.minimum(t + 1, window)))


def hca_prefill_flops(T, H, d=512, d_lat=1024, gated=True):
    att = 4.0 * d * hca_pairs(T) * H
    gate = 2.0 * T * d_lat * H * d if gated else 0.0
    return att, gate


def src_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


# --------------------------------------------------------------------------- timing helpers
class Timer:
    """HIP events recorded on the stream the kernels run on."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def event(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e


def flush_cache(torch, buf):
    """Reads 1 GiB so that the 256 MB Infinity Cache holds none of the inputs.  A read leaves
    no dirty lines behind: evicting with a write (buf.add_) made the timed kernels pay for
    writing the flush buffer back to HBM, about 30 us of a decode step."""
    buf.view(-1, 1 << 20).amax(dim=1)


# --------------------------------------------------------------------------- workloads
def run_c1(torch, lgsa, synth, to_dev, steps, warmup):
    """Step = hca_compress -> hca_attn_fwd with the gate operands, whose gated prefill kernel
    applies sigmoid(q_lat W) in its epilogue (O never goes to memory).  A HIP event between
    the two calls brackets each kernel."""
    T, H, d = 32768, 64, 512
    log("[bench] C1: generating inputs (seq %d, %d heads, d %d)" % (T, H, d))
    x = synth.hca_prefill(1, T=T, H=H, d=d, bf16=True, qkv_scale=1.0 / math.sqrt(512))
    dev = {k: to_dev(v) for k, v in x.items()}
    kc = torch.empty((1, T // 128, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    out = torch.empty_like(dev["q"])
    stream = torch.cuda.current_stream()
    tm = Timer(torch, stream)

    def step(evs=None):
        lgsa.hca_compress(dev["k"], dev["v"], kc, vc)
        if evs is not None:
            evs.append(tm.event())
        lgsa.hca_attn_fwd(dev["q"], dev["pos0"], dev["k"], dev["v"], kc, vc, max_pos=T - 1,
                          q_lat=dev["q_lat"], w_gate=dev["w_gate"], out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log("[bench] C1: timing %d steps" % steps)
    marks = []
    t0 = tm.event()
    for _ in range(steps):
        step(marks)
        marks.append(tm.event())
    t1 = tm.event()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    # marks per step: [after compress, after the gated attention]
    ends = [t0] + marks[1::2][:-1]
    comp_ms = [a.elapsed_time(b) for a, b in zip(ends, marks[0::2])]
    attn_ms = [a.elapsed_time(b) for a, b in zip(marks[0::2], marks[1::2])]
    att, gate = hca_prefill_flops(T, H, d)
    gib = 1 << 30
    # algorithmic bytes: each input read once, each output written once
    fused_bytes = (2 * gib + 2 * gib + 2 * (T * d * 2) + 2 * (T // 128) * d * 2 +
                   T * 1024 * 2 + 1024 * H * d * 2)
    comp_bytes = 2 * T * d * 2 + 2 * (T // 128) * d * 2
    kernels = [
        dict(name="hca_prefill_gated_kernel", call="hca_attn_fwd",
             ms=float(np.mean(attn_ms)), ms_median=float(np.median(attn_ms)), flops=att + gate,
             bytes=fused_bytes, src="hca_bf16.hip"),
        dict(name="compress_kernel", call="hca_compress", ms=float(np.mean(comp_ms)),
             ms_median=float(np.median(comp_ms)), flops=0.0, bytes=comp_bytes,
             src="compress.hip"),
    ]

    # the same step composed of the unfused calls, for comparison: the ungated attention
    # kernel writes O, then latent_gate rescales it in place
    o2 = out.view(T, H * d)
    ql2 = dev["q_lat"].view(T, -1)

    def unfused():
        lgsa.hca_compress(dev["k"], dev["v"], kc, vc)
        lgsa.hca_attn_fwd(dev["q"], dev["pos0"], dev["k"], dev["v"], kc, vc, max_pos=T - 1,
                          out=out)
        lgsa.latent_gate(ql2, dev["w_gate"], o2, out=o2)

    unfused()
    torch.cuda.synchronize()
    a = tm.event()
    for _ in range(5):
        unfused()
    b = tm.event()
    torch.cuda.synchronize()
    unfused_ms = a.elapsed_time(b) / 5
    return dict(ms_per_step=total_ms / steps, flops=att + gate, kernels=kernels, inputs=x,
                step_ms_min=min(a_ + c_ for a_, c_ in zip(attn_ms, comp_ms)),
                unfused_ms=unfused_ms)


def kernel_roofline(k, traffic):
    """Roofline record of one kernel: bound by whichever of MFMA time and HBM time at peak is
    larger for its algorithmic work."""
    t_f = k["flops"] / (PEAK_BF16_TFLOPS * 1e12)
    t_b = k["bytes"] / (PEAK_HBM_GBPS * 1e9)
    sec = k["ms"] * 1e-3
    if t_f >= t_b:
        ach, peak, unit, bound = k["flops"] / sec / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma"
    else:
        ach, peak, unit, bound = k["bytes"] / sec / 1e9, PEAK_HBM_GBPS, "GB/s", "hbm"
    return dict(bound=bound, achieved=round(ach, 2), peak=peak, unit=unit,
                frac=round(ach / peak, 4), traffic=traffic, kernel=k["name"],
                entry_point=k["call"], launch_ms=round(k["ms"], 4),
                launch_ms_median=round(k.get("ms_median", k["ms"]), 4),
                flops_per_launch=k["flops"], bytes_per_launch=k["bytes"])


def run_copy(torch, steps):
    """A plain 1 GiB device-to-device copy, the calibration kernel of the traffic counters."""
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps(dict(copy_bytes_read=4 * n, copy_bytes_written=4 * n, launches=steps)))


def oracle_seconds(fn, repeats=1):
    """Best wall time of `repeats` calls of an oracle computation on the host cores (None when
    the oracle timings are off)."""
    if not ORACLE_TIMING:
        return None
    best = None
    for _ in range(repeats):
        t0 = time.perf_counter()
        fn()
        dt = time.perf_counter() - t0
        best = dt if best is None else min(best, dt)
    return best


def run_c0(torch, lgsa, synth, to_dev, iters):
    """The tiny fp32 HCA prefill: seq 1024, 4 heads, d 512, 8 entries, gated (W 1024 x 2048);
    step = hca_compress + gated hca_attn_fwd.  Also the fp64 oracle on the whole workload,
    best of 3."""
    import oracle

    T, H, d = 1024, 4, 512
    x = synth.hca_prefill(0, T=T, H=H, bf16=False)
    dev = {k: to_dev(v) for k, v in x.items()}
    tm = Timer(torch, torch.cuda.current_stream())

    def step():
        kc, vc = lgsa.hca_compress(dev["k"], dev["v"])
        return lgsa.hca_attn_fwd(dev["q"], dev["pos0"], dev["k"], dev["v"], kc, vc,
                                 max_pos=T - 1, q_lat=dev["q_lat"], w_gate=dev["w_gate"])

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    ms = []
    for _ in range(iters):
        a = tm.event()
        step()
        b = tm.event()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    att, gate = hca_prefill_flops(T, H, d)
    oracle.build(force=False)

    def orc():
        kc = oracle.hca_compress(x["k"])
        vc = oracle.hca_compress(x["v"])
        oracle.hca_attn(x["q"], x["pos0"], x["k"], x["v"], kc, vc, q_lat=x["q_lat"],
                        w_gate=x["w_gate"])

    secs = oracle_seconds(orc, 3)
    orec = None if secs is None else dict(
        seconds=round(secs, 4), TFLOPs=(att + gate) / secs / 1e12, cores=oracle.max_threads(),
        kind="oracle", sample="whole workload (1024 rows, 4 heads, gated), best of 3")
    return dict(ms=float(np.median(ms)), ms_min=float(np.min(ms)), flops=att + gate,
                oracle=orec)


def run_c2(torch, lgsa, synth, to_dev, iters):
    B, ctx, H, d = 64, 131072, 64, 512
    log("[bench] C2: generating inputs (batch %d, context %d)" % (B, ctx))
    x = synth.hca_decode(2, B=B, context=ctx, H=H)
    dev = {k: to_dev(v) for k, v in x.items()}
    # five copies of the inputs (1.13 GB) in rotation: each call reads the copy used five calls
    # before, with more than the 256 MB Infinity Cache read since
    sets = [dev] + [{k: v.clone() for k, v in dev.items()} for _ in range(4)]
    outs = [torch.empty_like(dev["q"]) for _ in sets]
    tm = Timer(torch, torch.cuda.current_stream())

    def step(i):
        d = sets[i % len(sets)]
        lgsa.hca_attn_fwd(d["q"], d["pos0"], d["k_win"], d["v_win"], d["kc"], d["vc"],
                          max_pos=ctx - 1, q_lat=d["q_lat"], w_gate=d["w_gate"],
                          out=outs[i % len(sets)])

    for i in range(len(sets)):
        step(i)
    torch.cuda.synchronize()
    ms = []
    for i in range(iters):
        a = tm.event()
        step(i)
        b = tm.event()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    del sets, outs
    nbytes = sum(int(v.nbytes) for k, v in x.items() if k != "pos0") + int(x["q"].nbytes)
    import oracle

    oracle.build(force=False)
    secs = oracle_seconds(lambda: oracle.hca_attn(x["q"], x["pos0"], x["k_win"], x["v_win"],
                                                  x["kc"], x["vc"], q_lat=x["q_lat"],
                                                  w_gate=x["w_gate"]))
    orec = None if secs is None else dict(
        seconds=round(secs, 3), GBps=nbytes / secs / 1e9, cores=oracle.max_threads(),
        kind="oracle", sample="all 64 sequences, all heads, gated")
    return dict(ms=float(np.median(ms)), ms_min=float(np.min(ms)), bytes=nbytes, oracle=orec)


def run_c3(torch, lgsa, synth, to_dev, iters):
    T, H, d, k = 65536, 64, 256, 2048
    log("[bench] C3: generating inputs (seq %d, top-%d)" % (T, k))
    xi = synth.dsa_index(3, B=1, Tq=T, S=T)
    xs = synth.dsa_sparse(3, B=1, Tq=T, S=T, H=H, d=d)
    di = {k_: to_dev(v) for k_, v in xi.items()}
    ds = {k_: to_dev(v) for k_, v in xs.items()}
    idx = torch.empty((1, T, k), dtype=torch.int32, device="cuda")
    out = torch.empty_like(ds["q"])
    tm = Timer(torch, torch.cuda.current_stream())

    def step(evs):
        evs.append(tm.event())
        lgsa.dsa_index_topk(di["q_idx"], di["w_idx"], di["k_idx"], di["pos0"], k,
                            max_pos=T - 1, idx_out=idx)
        evs.append(tm.event())
        lgsa.sparse_attn_fwd(ds["q"], ds["kv_lat"], idx, q_lat=ds["q_lat"],
                             w_gate=ds["w_gate"], out=out)
        evs.append(tm.event())

    step([])
    torch.cuda.synchronize()
    idx_ms, sp_ms = [], []
    for _ in range(iters):
        e = []
        step(e)
        torch.cuda.synchronize()
        idx_ms.append(e[0].elapsed_time(e[1]))
        sp_ms.append(e[1].elapsed_time(e[2]))

    # the same gated sparse attention followed by the head mix (VHA, rank 16), fused into its
    # epilogue (the gate factors computed first)
    vu = to_dev(synth.normal(62, (H, 16), 0.02, True))
    vv = to_dev(synth.normal(63, (H, 16), 0.02, True))

    def mixed():
        lgsa.sparse_attn_fwd(ds["q"], ds["kv_lat"], idx, q_lat=ds["q_lat"], w_gate=ds["w_gate"],
                             out=out, vha_u=vu, vha_v=vv)

    mixed()
    torch.cuda.synchronize()
    mix_ms = []
    for _ in range(iters):
        a = tm.event()
        mixed()
        b = tm.event()
        torch.cuda.synchronize()
        mix_ms.append(a.elapsed_time(b))
    pairs = int(sum(min(k, t + 1) for t in range(T)))
    sp_flops = 4.0 * d * pairs * H + 2.0 * T * 1024 * H * d
    ind_pairs = T * (T + 1) // 2
    ind_flops = ind_pairs * (4 * 2 * 64 + 8)

    # backward of the sparse attention over the same lists: an ungated forward that also
    # writes the log-sum-exp, an N(0,1) output gradient, then sparse_attn_bwd (the latent rows
    # serve as keys and values, so dk holds both gradients); 10 d flops per (row, key, head)
    lse = torch.empty((1, T, H), dtype=torch.float32, device="cuda")
    o_ung = lgsa.sparse_attn_fwd(ds["q"], ds["kv_lat"], idx, lse=lse)
    g = torch.Generator(device="cuda").manual_seed(13)
    dout = torch.randn(1, T, H, d, device="cuda", generator=g).to(torch.bfloat16)
    dq = torch.empty_like(ds["q"])
    dk = torch.empty((1, T, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(lgsa.sparse_attn_bwd_workspace_bytes(ds["q"], ds["kv_lat"], idx, o_ung, lse,
                                                          dout), dtype=torch.uint8, device="cuda")

    def bwd():
        lgsa.sparse_attn_bwd(ds["q"], ds["kv_lat"], idx, o_ung, lse, dout, dq=dq, dk=dk,
                             workspace=ws)

    bwd()
    torch.cuda.synchronize()
    bwd_ms = []
    for _ in range(iters):
        a = tm.event()
        bwd()
        b = tm.event()
        torch.cuda.synchronize()
        bwd_ms.append(a.elapsed_time(b))
    del ws, dq, dk, dout, o_ung, lse

    # the gathers alone: the same top-k lists over the 32 MiB table of 512-byte latent rows,
    # the sparse kernel's DMA pattern with no arithmetic (the bound of its data movement)
    lists = idx.view(T, k)
    table = ds["kv_lat"].view(T, d)
    lgsa.sparse_gather_probe(table, lists)
    torch.cuda.synchronize()
    g_ms = []
    for _ in range(iters):
        a = tm.event()
        lgsa.sparse_gather_probe(table, lists)
        b = tm.event()
        torch.cuda.synchronize()
        g_ms.append(a.elapsed_time(b))
    gathered = float(pairs) * d * 2

    # the fp64 oracle on a bounded sample: top-k of 64 evenly spaced rows, gated sparse
    # attention of 128 evenly spaced rows over the GPU's own lists
    import oracle

    oracle.build(force=False)
    rows_i = np.linspace(0, T - 1, 64).astype(np.int64)
    rows_s = np.linspace(0, T - 1, 128).astype(np.int64)
    idx_h = idx.cpu().numpy()
    t_i = oracle_seconds(lambda: oracle.dsa_topk(xi["q_idx"], xi["w_idx"], xi["k_idx"],
                                                 xi["pos0"], k, rows=rows_i))
    t_s = oracle_seconds(lambda: oracle.sparse_attn(xs["q"], xs["kv_lat"], idx_h,
                                                    q_lat=xs["q_lat"], w_gate=xs["w_gate"],
                                                    rows=rows_s))
    i_fl = float(np.sum((rows_i + 1) * (4 * 2 * 64 + 8)))
    s_fl = float(np.sum(np.minimum(k, rows_s + 1))) * 4 * d * H + 2.0 * len(rows_s) * 1024 * H * d
    orec = None if t_i is None else dict(
        indexer_seconds=round(t_i, 3), indexer_TFLOPs=i_fl / t_i / 1e12,
        sparse_seconds=round(t_s, 3), sparse_TFLOPs=s_fl / t_s / 1e12,
        cores=oracle.max_threads(), kind="oracle",
        sample="top-k of 64 and gated sparse attention of 128 evenly spaced query rows (all "
               "64 heads)")
    return dict(index_ms=float(np.median(idx_ms)), sparse_ms=float(np.median(sp_ms)),
                sparse_flops=sp_flops, index_flops=float(ind_flops),
                bwd_ms=float(np.median(bwd_ms)), bwd_flops=10.0 * d * pairs * H,
                gather_ms=float(np.median(g_ms)), gather_bytes=gathered, oracle=orec,
                sparse_vha_ms=float(np.median(mix_ms)))


def run_csa(torch, lgsa, synth, to_dev, iters):
    """The compressed sparse attention variant at the DSA prefill shape: 65536 positions, 64
    heads, d 256 (bf16), keys and values pooled 4x (16384 entries), the indexer (4 heads x 64,
    fp32) over the entries each query can see, top-2048, gated.  One step = the three library
    calls of csa_attn_fwd."""
    T, H, d, k, block = 65536, 64, 256, 2048, 4
    log("[bench] CSA: generating inputs (seq %d, block %d, top-%d)" % (T, block, k))
    x = synth.csa(5, B=1, T=T, H=H)
    dx = {k_: to_dev(v) for k_, v in x.items()}
    tm = Timer(torch, torch.cuda.current_stream())

    def step():
        return lgsa.csa_attn_fwd(dx["q"], dx["pos0"], dx["kv_lat"], dx["v_lat"], dx["q_idx"],
                                 dx["w_idx"], dx["k_idx"], k, max_pos=T - 1, block=block,
                                 q_lat=dx["q_lat"], w_gate=dx["w_gate"])

    step()
    torch.cuda.synchronize()
    ms = []
    for _ in range(iters):
        a = tm.event()
        step()
        b = tm.event()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    ne = [(t + 1) // block for t in range(T)]
    att_pairs = float(sum(min(k, n) for n in ne))
    ind_pairs = float(sum(ne))
    flops = 4.0 * d * att_pairs * H + 2.0 * T * 1024 * H * d + ind_pairs * (4 * 2 * 64 + 8)
    return dict(ms=float(np.median(ms)), flops=flops)


def run_gate_bwd(torch, lgsa, iters):
    """Backward of the gate at the HCA prefill model shape (32768 rows x 32768 channels, d_lat
    1024, bf16): the recomputed gate with the elementwise gradients, then dq_lat = dG W^T and
    dW = q_lat^T dG.  Inputs are device-side N(0,1) draws from a seeded generator (W scaled by
    0.02), the shapes of the forward's."""
    M, N, d_lat = 32768, 32768, 1024
    g = torch.Generator(device="cuda").manual_seed(7)
    bf = torch.bfloat16
    ql = torch.randn(M, d_lat, device="cuda", generator=g).to(bf)
    w = (torch.randn(d_lat, N, device="cuda", generator=g) * 0.02).to(bf)
    o = torch.randn(M, N, device="cuda", generator=g).to(bf)
    dout = torch.randn(M, N, device="cuda", generator=g).to(bf)
    d_o, dq, dw = torch.empty_like(o), torch.empty_like(ql), torch.empty_like(w)
    ws = torch.empty(M * N * 2, dtype=torch.uint8, device="cuda")
    tm = Timer(torch, torch.cuda.current_stream())
    lgsa.latent_gate_bwd(ql, w, o, dout, d_o, dq, dw, workspace=ws)
    torch.cuda.synchronize()
    a = tm.event()
    for _ in range(iters):
        lgsa.latent_gate_bwd(ql, w, o, dout, d_o, dq, dw, workspace=ws)
    b = tm.event()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / iters
    flops = 3 * 2.0 * M * N * d_lat
    del ql, w, o, dout, d_o, dq, dw, ws
    return dict(ms=round(ms, 3), TFLOPs=round(flops / (ms * 1e-3) / 1e12, 1),
                mfma_frac=round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4))


def run_hca_bwd(torch, lgsa, iters):
    """Backward of HCA prefill at the model shape (seq 32768, 64 heads, d 512, bf16, block 128,
    window 128), after an ungated forward that also writes the log-sum-exp.  Inputs are
    device-side seeded N(0,1) draws scaled as the forward's (q, k, v / sqrt(512)); the output
    gradient is N(0,1).  Algorithmic work: 10 d flops per visible (row, key) pair (S, dP, dQ,
    dK, dV)."""
    T, H, d, W, blk = 32768, 64, 512, 128, 128
    g = torch.Generator(device="cuda").manual_seed(11)
    bf = torch.bfloat16
    sc = 1.0 / math.sqrt(d)
    q = (torch.randn(1, T, H, d, device="cuda", generator=g) * sc).to(bf)
    k = (torch.randn(1, T, d, device="cuda", generator=g) * sc).to(bf)
    v = (torch.randn(1, T, d, device="cuda", generator=g) * sc).to(bf)
    kc, vc = lgsa.hca_compress(k, v, block=blk)
    lse = torch.empty(1, T, H, dtype=torch.float32, device="cuda")
    pos0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = lgsa.hca_attn_fwd(q, pos0, k, v, kc, vc, max_pos=T - 1, window=W, block=blk, lse=lse)
    dout = torch.randn(1, T, H, d, device="cuda", generator=g).to(bf)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step():
        lgsa.hca_attn_bwd(q, k, v, kc, vc, out, lse, dout, window=W, block=blk, dq=dq, dk=dk,
                          dv=dv)

    step()
    torch.cuda.synchronize()
    tm = Timer(torch, torch.cuda.current_stream())
    a = tm.event()
    for _ in range(iters):
        step()
    b = tm.event()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / iters
    pairs = sum(min(T // blk, (t + 1) // blk) + min(W, t + 1) for t in range(T))
    flops = 10.0 * d * pairs * H
    del q, k, v, out, dout, dq, dk, dv, lse
    return dict(ms=round(ms, 3), TFLOPs=round(flops / (ms * 1e-3) / 1e12, 1),
                mfma_frac=round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4))


def run_c4(torch, lgsa, synth, to_dev, iters):
    B, ctx, H = 8, 1 << 20, 64
    log("[bench] C4: generating inputs (batch %d, context %d)" % (B, ctx))
    xh = synth.hca_decode(4, B=B, context=ctx, H=H)
    xi = synth.dsa_index(4, B=B, Tq=1, S=ctx, pos0=[ctx - 1] * B)
    xs = synth.dsa_sparse(4, B=B, Tq=1, S=ctx, H=H, qname="q_dsa", latname="q_lat_dsa",
                          wname="w_gate_dsa")
    dh = {k: to_dev(v) for k, v in xh.items()}
    di = {k: to_dev(v) for k, v in xi.items()}
    ds = {k: to_dev(v) for k, v in xs.items()}
    # four copies of all inputs (9.6 GB) in rotation: each step reads the copy used four steps
    # before, with far more than the 256 MB Infinity Cache read since
    n_rot = 4
    sets = [(dh, di, ds)] + [tuple({k: v.clone() for k, v in d.items()} for d in (dh, di, ds))
                             for _ in range(n_rot - 1)]
    outs = [(torch.empty_like(dh["q"]), torch.empty_like(ds["q"]),
             torch.empty((B, 1, 2048), dtype=torch.int32, device="cuda")) for _ in range(n_rot)]
    tm = Timer(torch, torch.cuda.current_stream())

    def step(evs, it):
        h, i_, s_ = sets[it % n_rot]
        out_h, out_s, idx = outs[it % n_rot]
        evs.append(tm.event())
        lgsa.hca_attn_fwd(h["q"], h["pos0"], h["k_win"], h["v_win"], h["kc"], h["vc"],
                          max_pos=ctx - 1, q_lat=h["q_lat"], w_gate=h["w_gate"], out=out_h)
        evs.append(tm.event())
        lgsa.dsa_index_topk(i_["q_idx"], i_["w_idx"], i_["k_idx"], i_["pos0"], 2048,
                            max_pos=ctx - 1, idx_out=idx)
        evs.append(tm.event())
        lgsa.sparse_attn_fwd(s_["q"], s_["kv_lat"], idx, q_lat=s_["q_lat"],
                             w_gate=s_["w_gate"], out=out_s)
        evs.append(tm.event())

    for it in range(n_rot):
        step([], it)
    torch.cuda.synchronize()
    tot, ind = [], []
    for it in range(iters):
        e = []
        step(e, it)
        torch.cuda.synchronize()
        tot.append(e[0].elapsed_time(e[3]))
        ind.append(e[1].elapsed_time(e[2]))
    del sets, outs
    hbytes = sum(int(v.nbytes) for k, v in xh.items() if k != "pos0") + int(xh["q"].nbytes)
    ibytes = sum(int(v.nbytes) for k, v in xi.items() if k != "pos0") + B * 2048 * 4
    sbytes = (sum(int(v.nbytes) for k_, v in xs.items() if k_ != "kv_lat") +
              B * 2048 * 256 * 2 + int(xs["q"].nbytes))
    # the fp64 oracle on the whole step: HCA of the 8 sequences, their top-k, then the gated
    # sparse attention over the oracle's own lists
    import oracle

    oracle.build(force=False)
    def orc():
        oracle.hca_attn(xh["q"], xh["pos0"], xh["k_win"], xh["v_win"], xh["kc"], xh["vc"],
                        q_lat=xh["q_lat"], w_gate=xh["w_gate"])
        o_idx, _ = oracle.dsa_topk(xi["q_idx"], xi["w_idx"], xi["k_idx"], xi["pos0"], 2048)
        oracle.sparse_attn(xs["q"], xs["kv_lat"], o_idx.reshape(B, 1, 2048), q_lat=xs["q_lat"],
                           w_gate=xs["w_gate"])

    secs = oracle_seconds(orc)
    nb = hbytes + ibytes + sbytes
    orec = None if secs is None else dict(
        seconds=round(secs, 3), GBps=nb / secs / 1e9, cores=oracle.max_threads(),
        kind="oracle", sample="whole step: all 8 sequences, both layers, gated")
    return dict(ms=float(np.median(tot)), index_ms=float(np.median(ind)),
                bytes=nb, index_bytes=ibytes, oracle=orec)


def run_vha(torch, lgsa, synth, to_dev, iters):
    """The Virtual Head Attention mixing step at the prefill model shape: 32768 tokens x 64
    heads x 512 channels (bf16), rank 16, in place; it reads and writes the output once."""
    M, H, d, r = 32768, 64, 512, 16
    o = torch.randn((M, H, d), device="cuda").to(torch.bfloat16)
    u = to_dev(synth.normal(60, (H, r), 0.02, True))
    v = to_dev(synth.normal(61, (H, r), 0.02, True))
    tm = Timer(torch, torch.cuda.current_stream())
    lgsa.vha_mix(o, u, v, out=o)
    torch.cuda.synchronize()
    a = tm.event()
    for _ in range(iters):
        lgsa.vha_mix(o, u, v, out=o)
    b = tm.event()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / iters
    nbytes = 2 * M * H * d * 2 + 2 * H * r * 2
    flops = 2.0 * 2 * M * H * r * d
    return dict(ms=round(ms, 4), bytes=nbytes, GBps=round(nbytes / (ms * 1e-3) / 1e9, 1),
                hbm_frac=round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4), flops=flops)


def run_append(torch, lgsa, synth, to_dev, iters):
    """Decode-time cache appends at the decode workloads' shapes: the HCA append for 64
    sequences (ring of 128 rows, 1024 entries, d 512, bf16) at a block's last token, which also
    writes the block's entry, and mid-block; the DSA append for 8 sequences (indexer key 64 fp32,
    latent row 256 bf16, 1M positions)."""
    B, d, W, n_cap = 64, 512, 128, 1024
    kw = to_dev(synth.normal(50, (B, W, d), 1.0, True))
    vw = to_dev(synth.normal(51, (B, W, d), 1.0, True))
    kc = torch.zeros((B, n_cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kn = to_dev(synth.normal(52, (B, d), 1.0, True))
    vn = to_dev(synth.normal(53, (B, d), 1.0, True))
    Bd, S = 8, 1 << 20
    ki = torch.zeros((Bd, S, 64), dtype=torch.float32, device="cuda")
    kv = torch.zeros((Bd, S, 256), dtype=torch.bfloat16, device="cuda")
    kin = to_dev(synth.normal(54, (Bd, 64)))
    kvn = to_dev(synth.normal(55, (Bd, 256), 1.0, True))
    flush = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
    tm = Timer(torch, torch.cuda.current_stream())

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(iters):
            flush_cache(torch, flush)
            a = tm.event()
            fn()
            b = tm.event()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return float(np.median(ms))

    res = {}
    for name, t in (("hca_block_end", 131071), ("hca_mid_block", 131070)):
        pos = torch.full((B,), t, dtype=torch.int32, device="cuda")
        ms = timed(lambda: lgsa.hca_cache_append(pos, kn, vn, kw, vw, kc, vc))
        # new rows read + ring rows written; at a block's end also the block's other rows read
        # and the entry written
        nbytes = 2 * B * d * 2 * 2 + (2 * B * (W - 1) * d * 2 + 2 * B * d * 2 if t % 128 == 127
                                      else 0)
        res[name] = dict(us=round(ms * 1e3, 2), bytes=nbytes,
                         GBps=round(nbytes / (ms * 1e-3) / 1e9, 1))
    posd = torch.full((Bd,), S - 1, dtype=torch.int32, device="cuda")
    ms = timed(lambda: lgsa.dsa_cache_append(posd, kin, ki, kvn, kv))
    nbytes = 2 * Bd * (64 * 4 + 256 * 2)
    res["dsa"] = dict(us=round(ms * 1e3, 2), bytes=nbytes,
                      GBps=round(nbytes / (ms * 1e-3) / 1e9, 1))
    return res


# --------------------------------------------------------------------------- CPU baseline
def cpu_baseline(x, budget_s=15.0):
    """The fp64 oracle on a bounded, evenly spread sample of query rows of the C1 workload."""
    import oracle

    oracle.build(force=False)
    T, H, d = 32768, 64, 512
    kc = oracle.hca_compress(x["k"])
    vc = oracle.hca_compress(x["v"])

    def run(rows):
        t0 = time.perf_counter()
        oracle.hca_attn(x["q"], x["pos0"], x["k"], x["v"], kc, vc, q_lat=x["q_lat"],
                        w_gate=x["w_gate"], rows=rows)
        return time.perf_counter() - t0

    probe = np.arange(0, T, T // 16)
    dt = run(probe)
    n = int(max(16, min(T, budget_s / max(dt / len(probe), 1e-6))))
    rows = np.unique(np.linspace(0, T - 1, n).astype(np.int64))
    secs = run(rows)
    t = rows
    pairs = np.sum((t + 1) // 128 + np.minimum(t + 1, 128))
    flops = 4.0 * d * pairs * H + 2.0 * len(rows) * 1024 * H * d
    return dict(value=flops / secs / 1e12, unit="TFLOP/s", cores=oracle.max_threads(),
                kind="oracle",
                sample="%d of %d query rows (all %d heads, gated), evenly spaced; %.1f s"
                       % (len(rows), T, H, secs))


def kernel_sources_sha(src):
    """Hash of a kernel's source file and the shared device header it includes."""
    h = hashlib.sha256()
    for f in (src, "common.h"):
        with open(os.path.join(ROOT, "hybrid_sparse_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_record(k):
    """HBM bytes per launch of kernel k from the committed rocprofv3 counter summary (FETCH_SIZE
    + WRITE_SIZE, scaled by the copy-kernel calibration), or None when that summary was taken on
    another version of the kernel's source."""
    path = os.path.join(ROOT, "profiles", "hca_prefill_c1_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get("kernels", {}).get(k["name"])
    if not rec or rec.get("source_sha") != kernel_sources_sha(k["src"]):
        return None
    return float(rec["bytes_per_launch"])


# --------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--configs", default="0,1,2,3,4",
                    help="workloads to run; 1 is the headline, 0 and 2-4 are reported as "
                         "secondary")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--copy", action="store_true",
                    help="only run a 1 GiB device copy (calibrates the HBM traffic counters)")
    args = ap.parse_args()
    global ORACLE_TIMING
    ORACLE_TIMING = not args.no_cpu
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy:
        run_copy(torch, args.steps)
        return

    import hybrid_sparse_attention_amd as lgsa
    from hybrid_sparse_attention_amd import synth

    lgsa.load()  # fails loudly if the library is not built

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    cfgs = [int(c) for c in args.configs.split(",") if c]
    r1 = run_c1(torch, lgsa, synth, to_dev, args.steps, args.warmup)
    value = r1["flops"] / (r1["ms_per_step"] * 1e-3) / 1e12
    kern = [kernel_roofline(k, traffic_record(k)) for k in r1["kernels"]]
    dom = max(range(len(kern)), key=lambda i: r1["kernels"][i]["ms"])
    roofline = kern[dom]
    secondary = dict(c1_kernels=[kern[i] for i in range(len(kern)) if i != dom],
                     c1_unfused_step_ms=round(r1["unfused_ms"], 4))
    cpu = None
    if not args.no_cpu:
        log("[bench] CPU baseline: fp64 oracle on a sample of C1 rows")
        cpu = cpu_baseline(r1["inputs"])
    del r1["inputs"]
    if 0 in cfgs:
        log("[bench] C0: tiny fp32 HCA prefill")
        r0 = run_c0(torch, lgsa, synth, to_dev, 20)
        tf0 = r0["flops"] / (r0["ms"] * 1e-3) / 1e12
        secondary["c0_hca_prefill_f32"] = dict(
            ms=round(r0["ms"], 4), ms_min=round(r0["ms_min"], 4), TFLOPs=round(tf0, 2),
            fp32_frac=round(tf0 / PEAK_FP32_TFLOPS, 4), oracle=r0["oracle"])
    if 2 in cfgs:
        r2 = run_c2(torch, lgsa, synth, to_dev, 200)
        gbps = r2["bytes"] / (r2["ms"] * 1e-3) / 1e9
        secondary["c2_hca_decode"] = dict(ms=round(r2["ms"], 4), ms_min=round(r2["ms_min"], 4),
                                          GBps=round(gbps, 1),
                                          hbm_frac=round(gbps / PEAK_HBM_GBPS, 4),
                                          bytes=r2["bytes"], oracle=r2["oracle"])
    secondary["vha_mix_prefill"] = run_vha(torch, lgsa, synth, to_dev, 10)
    secondary["gate_bwd_prefill"] = run_gate_bwd(torch, lgsa, 3)
    secondary["hca_bwd_prefill"] = run_hca_bwd(torch, lgsa, 3)
    if 2 in cfgs or 4 in cfgs:
        secondary["decode_cache_append"] = run_append(torch, lgsa, synth, to_dev, 50)
    if 3 in cfgs:
        r3 = run_c3(torch, lgsa, synth, to_dev, 20)
        sp_tf = r3["sparse_flops"] / (r3["sparse_ms"] * 1e-3) / 1e12
        ix_tf = r3["index_flops"] / (r3["index_ms"] * 1e-3) / 1e12
        secondary["c3_dsa_prefill"] = dict(
            sparse_gate_ms=round(r3["sparse_ms"], 3), sparse_gate_TFLOPs=round(sp_tf, 1),
            sparse_mfma_frac=round(sp_tf / PEAK_BF16_TFLOPS, 4),
            indexer_ms=round(r3["index_ms"], 3), indexer_TFLOPs=round(ix_tf, 1),
            indexer_fp32_frac=round(ix_tf / PEAK_FP32_TFLOPS, 4),
            sparse_gate_vha_ms=round(r3["sparse_vha_ms"], 3),
            gather_probe=dict(ms=round(r3["gather_ms"], 3), bytes=r3["gather_bytes"],
                              TBps=round(r3["gather_bytes"] / (r3["gather_ms"] * 1e-3) / 1e12,
                                         2)),
            oracle=r3["oracle"])
        bw_tf = r3["bwd_flops"] / (r3["bwd_ms"] * 1e-3) / 1e12
        secondary["sparse_bwd_prefill"] = dict(ms=round(r3["bwd_ms"], 3), TFLOPs=round(bw_tf, 1),
                                               mfma_frac=round(bw_tf / PEAK_BF16_TFLOPS, 4))
    if 3 in cfgs:
        rc = run_csa(torch, lgsa, synth, to_dev, 20)
        tf = rc["flops"] / (rc["ms"] * 1e-3) / 1e12
        secondary["csa_prefill"] = dict(ms=round(rc["ms"], 3), TFLOPs=round(tf, 1))
    if 4 in cfgs:
        r4 = run_c4(torch, lgsa, synth, to_dev, 200)
        gbps = r4["bytes"] / (r4["ms"] * 1e-3) / 1e9
        igbps = r4["index_bytes"] / (r4["index_ms"] * 1e-3) / 1e9
        secondary["c4_mixed_decode"] = dict(ms=round(r4["ms"], 4), GBps=round(gbps, 1),
                                            hbm_frac=round(gbps / PEAK_HBM_GBPS, 4),
                                            indexer_ms=round(r4["index_ms"], 4),
                                            indexer_GBps=round(igbps, 1), bytes=r4["bytes"],
                                            oracle=r4["oracle"])
    line = dict(
        metric=METRIC, value=round(value, 2), unit="TFLOP/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=round(r1["ms_per_step"], 4), higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload="HCA prefill at model shape: seq 32768, 64 query heads + 1 shared "
                             "KV head, head dim 512, bf16, 256 mean-pooled entries + 128-token "
                             "window, low-rank sigmoid gate (W_gate 1024x32768) fused into the "
                             "attention epilogue; step = hca_compress + gated hca_attn_fwd",
                    seq_len=32768, heads=64, head_dim=512, batch=1, parallelism="none"),
        roofline=roofline, cpu_baseline=cpu, secondary=secondary)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
