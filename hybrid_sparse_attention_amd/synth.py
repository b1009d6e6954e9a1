"""Seeded synthetic inputs shaped like the ERNIE 5.5 Flash attention layers.

This module holds no arithmetic of the method: it only draws seeded random numbers and rounds
them to bfloat16.  Both the HIP path and the oracle are fed from it.

Shapes follow the pages: 64 attention heads and hidden size 4096, so the query latent is
4096 / 4 = 1024 wide; HCA heads are 512 wide and MLA heads 256 wide; one HCA cache entry per
128 tokens and a 128-token raw window; contexts up to 1,048,576 tokens (ERNIE 5.5 Flash Base
release blog, sections 2 and 2.1; xenospectrum.com article on ERNIE 5.5 Flash Base, section
on the long-context mechanism).

Recipe: numpy ``Generator(PCG64(seed))`` with ``seed = 1000 * config + tensor_id``.  Normals
are drawn in float32 chunk by chunk from one generator per tensor, scaled, and for bfloat16
configurations rounded to nearest-even bfloat16 (stored as uint16 bit patterns).
"""
from __future__ import annotations

import numpy as np

# tensor ids of the seed recipe
TID = dict(q=1, k=2, v=3, q_lat=4, w_gate=5, kc=6, vc=7, k_win=8, v_win=9, q_idx=10,
           k_idx=11, w_idx=12, kv_lat=13, v_lat=14, q_dsa=15, q_lat_dsa=16, w_gate_dsa=17,
           idx=18)

HIDDEN, HEADS, D_LAT = 4096, 64, 1024
D_HCA, D_MLA, BLOCK, WINDOW = 512, 256, 128, 128
HI, DI, TOPK = 4, 64, 2048

_CHUNK = 1 << 24  # elements per generation chunk


def seed_of(config: int, name: str) -> int:
    return 1000 * int(config) + TID[name]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to nearest-even bfloat16; returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(seed: int, shape, scale: float = 1.0, bf16: bool = False) -> np.ndarray:
    """N(0, scale^2) draws in float32 (or bfloat16 bits), generated chunk by chunk."""
    g = np.random.Generator(np.random.PCG64(seed))
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    buf = np.empty(min(n, _CHUNK), dtype=np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        b = buf[: e - s]
        g.standard_normal(out=b, dtype=np.float32)
        if scale != 1.0:
            b *= np.float32(scale)
        out[s:e] = round_bf16(b) if bf16 else b
    return out.reshape(shape)


def uniform(seed: int, shape) -> np.ndarray:
    """U(0, 1) draws in float32."""
    g = np.random.Generator(np.random.PCG64(seed))
    return g.random(size=shape, dtype=np.float32)


# --------------------------------------------------------------------------- configurations
CONFIGS = {
    0: "HCA prefill, tiny: B=1, T=1024, H=4, 1 KV head, d=512, fp32, 8 compressed entries, "
       "window 128, gate from a 1024-wide query latent",
    1: "HCA prefill, model shape: B=1, T=32768, H=64, 1 KV head, d=512, bf16, 256 compressed "
       "entries, window 128, gate W 1024x32768",
    2: "HCA decode: B=64, context 131072 (1024 compressed entries + 128-row ring), H=64, "
       "d=512, bf16",
    3: "MLA-DSA prefill: B=1, T=65536, H=64, d=256, bf16 latent rows (V = K), indexer 4x64 "
       "fp32, top-2048, gate W 1024x16384",
    4: "mixed long-context decode: B=8, context 1048576; HCA 8192 entries + 128 ring, d=512; "
       "DSA indexer over 1048576 fp32 keys, top-2048, sparse attention d=256",
}


def hca_prefill(config: int, T: int, H: int, d: int = D_HCA, bf16: bool = True,
                qkv_scale: float = 1.0, d_lat: int = D_LAT, gated: bool = True):
    """Inputs of an HCA prefill: q [1,T,H,d], k, v [1,T,d], q_lat [1,T,d_lat], w [d_lat,H*d]."""
    x = dict(
        q=normal(seed_of(config, "q"), (1, T, H, d), qkv_scale, bf16),
        k=normal(seed_of(config, "k"), (1, T, d), qkv_scale, bf16),
        v=normal(seed_of(config, "v"), (1, T, d), qkv_scale, bf16),
        pos0=np.zeros(1, dtype=np.int32),
    )
    if gated:
        x["q_lat"] = normal(seed_of(config, "q_lat"), (1, T, d_lat), 1.0, bf16)
        x["w_gate"] = normal(seed_of(config, "w_gate"), (d_lat, H * d), 0.02, bf16)
    return x


def hca_decode(config: int, B: int, context: int, H: int, d: int = D_HCA,
               block: int = BLOCK, window: int = WINDOW, d_lat: int = D_LAT,
               contexts=None, gated: bool = True):
    """Inputs of an HCA decode step: one query per sequence at t = context - 1.

    The caches are seeded directly (N(0,1) bf16): kc, vc [B, context//block, d] and a
    `window`-row ring k_win, v_win [B, window, d] where position p sits in row p % window.
    `contexts` may give a different context per sequence (the cache is sized for the max).
    """
    if contexts is None:
        contexts = [context] * B
    n_cap = max(contexts) // block
    x = dict(
        q=normal(seed_of(config, "q"), (B, 1, H, d), 1.0, True),
        kc=normal(seed_of(config, "kc"), (B, n_cap, d), 1.0, True),
        vc=normal(seed_of(config, "vc"), (B, n_cap, d), 1.0, True),
        k_win=normal(seed_of(config, "k_win"), (B, window, d), 1.0, True),
        v_win=normal(seed_of(config, "v_win"), (B, window, d), 1.0, True),
        pos0=np.asarray([c - 1 for c in contexts], dtype=np.int32),
    )
    if gated:
        x["q_lat"] = normal(seed_of(config, "q_lat"), (B, 1, d_lat), 1.0, True)
        x["w_gate"] = normal(seed_of(config, "w_gate"), (d_lat, H * d), 0.02, True)
    return x


def dsa_index(config: int, B: int, Tq: int, S: int, Hi: int = HI, di: int = DI, pos0=None):
    """Indexer inputs: q_idx [B,Tq,Hi,di], k_idx [B,S,di] ~ N(0,1), w_idx [B,Tq,Hi] ~ U(0,1)."""
    x = dict(
        q_idx=normal(seed_of(config, "q_idx"), (B, Tq, Hi, di)),
        k_idx=normal(seed_of(config, "k_idx"), (B, S, di)),
        w_idx=uniform(seed_of(config, "w_idx"), (B, Tq, Hi)),
    )
    x["pos0"] = (np.zeros(B, dtype=np.int32) if pos0 is None
                 else np.asarray(pos0, dtype=np.int32))
    return x


def dsa_sparse(config: int, B: int, Tq: int, S: int, H: int, d: int = D_MLA,
               d_lat: int = D_LAT, distinct_v: bool = False, gated: bool = True,
               qname: str = "q", latname: str = "q_lat", wname: str = "w_gate"):
    """Sparse-attention inputs: q [B,Tq,H,d], kv_lat [B,S,d] (bf16, N(0,1)), optional v_lat."""
    x = dict(
        q=normal(seed_of(config, qname), (B, Tq, H, d), 1.0, True),
        kv_lat=normal(seed_of(config, "kv_lat"), (B, S, d), 1.0, True),
    )
    if distinct_v:
        x["v_lat"] = normal(seed_of(config, "v_lat"), (B, S, d), 1.0, True)
    if gated:
        x["q_lat"] = normal(seed_of(config, latname), (B, Tq, d_lat), 1.0, True)
        x["w_gate"] = normal(seed_of(config, wname), (d_lat, H * d), 0.02, True)
    return x


def csa(config: int, B: int, T: int, H: int, d: int = D_MLA, gated: bool = True):
    """Compressed sparse attention inputs for T positions per sequence: the sparse-attention
    draws with distinct values (q, kv_lat as the keys, v_lat as the values, the gate) and the
    indexer draws (q_idx, w_idx, k_idx per position), pos0 = 0."""
    x = dsa_sparse(config, B, T, T, H, d, distinct_v=True, gated=gated)
    x.update(dsa_index(config, B, Tq=T, S=T))
    return x


def random_topk(config: int, B: int, Tq: int, S: int, k: int, pos0):
    """A seeded index list per query: k distinct causal positions (all when t+1 <= k),
    ascending, -1 padded.  Stands in for an indexer output when sparse attention is tested
    by itself."""
    g = np.random.Generator(np.random.PCG64(seed_of(config, "idx")))
    idx = np.full((B, Tq, k), -1, dtype=np.int32)
    for b in range(B):
        for i in range(Tq):
            t = int(pos0[b]) + i
            n = min(t + 1, S)
            if n <= k:
                idx[b, i, :n] = np.arange(n, dtype=np.int32)
            else:
                idx[b, i] = np.sort(g.choice(n, size=k, replace=False)).astype(np.int32)
    return idx


def stratified_topk(config: int, B: int, Tq: int, S: int, k: int, pos0):
    """A seeded index list per query row shaped like an indexer's output, cheap at any size:
    row t keeps every causal position when t + 1 <= k; otherwise [0, t] is cut into k strata
    at the integer boundaries floor(j (t+1) / k) and one position is drawn uniformly from each,
    which gives k distinct positions in ascending order.  Unused slots hold -1."""
    g = np.random.Generator(np.random.PCG64(seed_of(config, "idx")))
    idx = np.full((B, Tq, k), -1, dtype=np.int32)
    j = np.arange(k + 1, dtype=np.int64)
    for b in range(B):
        for i0 in range(0, Tq, 1024):
            i1 = min(Tq, i0 + 1024)
            t = int(pos0[b]) + np.arange(i0, i1, dtype=np.int64)
            n = np.minimum(t + 1, S)
            short = n <= k
            bounds = (j[None, :] * n[:, None]) // k              # [rows, k+1]
            width = bounds[:, 1:] - bounds[:, :-1]               # >= 1 when n >= k
            u = g.random((i1 - i0, k))
            pick = bounds[:, :-1] + np.floor(u * width).astype(np.int64)
            blk = pick.astype(np.int32)
            if short.any():
                rows = np.nonzero(short)[0]
                ar = np.arange(k, dtype=np.int64)[None, :]
                full = np.where(ar < n[rows, None], ar, -1).astype(np.int32)
                blk[rows] = full
            idx[b, i0:i1] = blk
    return idx
