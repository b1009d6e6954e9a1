// Heavily Compressed Attention forward, bfloat16, 512-wide heads, for gfx950.
//
// ERNIE 5.5 Flash Base release blog, section 2.1 "Latent-Gated Sparse Attention": each HCA
// layer keeps one cache entry per 128 tokens and attends densely to all completed entries plus
// a short window of recent raw tokens (128 tokens per the xenospectrum.com article on ERNIE 5.5
// Flash Base, long-context section); HCA heads are 512 wide; every layer multiplies the
// attention output by a gate computed from the low-rank query latent.  Visibility is
// closed-form: position t sees compressed entry e iff e < (t + 1) / block, raw position s iff
// t - window + 1 <= s <= t.
//
// On-chip budget for 512-wide heads.  A wave owns 16 query rows over the whole head: Q in 64
// registers and O in 128, which leaves room for two waves per SIMD (a wave of 32 rows would
// need 384 registers for Q and O alone).  Each wave forms the full scores of its rows, so no
// partial results are exchanged between waves.
//
// Data movement.  Key and value tiles (32 rows x 1 KiB) go from global memory to LDS by LDS
// DMA (global_load_lds_dwordx4: one 1 KiB row per wave instruction), never through registers.
// Rows are padded by 32 bytes so that the fragment reads are bank-conflict free (a 16-byte pad
// leaves the row-wise K reads conflicting) and every fragment address is the lane's base plus
// an immediate.  V stays row-major; the MFMA operand V^T is read with the transposing LDS read
// (ds_read_b64_tr_b16).  K and V are both double buffered: tile ti + 1 streams in while tile
// ti is used, with one workgroup barrier per tile.
//
// Products on v_mfma_f32_16x16x32_bf16, transposed (S^T = K Q^T, O^T = V^T P^T): the tile in
// LDS is the A operand, the query rows in registers the B operand; a lane owns one query row
// for all its accumulators, and the P fragment of the second product is the S^T accumulator
// of the first (the two transposed reads pick the key rows that lane group's accumulator
// holds, so no data moves between lanes).
//
// Prefill: one workgroup of 8 waves per (32 query tokens, 4 heads).  Decode: one workgroup of
// 4 waves (the 64 heads of one token) per (sequence, key split); partial (max, sum, O) of a
// split go to the workspace and a combine kernel merges them.  When gated, the gate GEMM then
// multiplies sigmoid(q_lat W) into O in place.
#include "common.h"
#include "kernels.h"

namespace lgsa {

namespace {

constexpr int D = 512;
constexpr int KT = 32;                 // keys per tile
constexpr int ROWB = 1024;             // bytes of one 512-wide bf16 row in memory
constexpr int KLD = ROWB + 32;         // LDS row of a key tile (32-byte pad: no bank conflicts)
constexpr int VLD = ROWB + 32;         // LDS row of a value tile
constexpr int KTILE = KT * KLD;
constexpr int VTILE = KT * VLD;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LAZY = 8.0f;           // rescale O only when the max grows by more (log2)

// Masked logits take this finite sentinel instead of -inf, which keeps the online softmax
// free of special cases: while a row has seen no visible key its running max is the
// sentinel, whatever it accumulated is scaled by 2^(sentinel - real max) = 0 as soon as a
// visible key arrives, and a row that never sees one is written as zeros.
constexpr float NEG_BIG = -1.0e30f;

struct Tile {
  int kind, start, count;  // kind 0: compressed entries start.., kind 1: raw positions start..
  int row0;                // buffer row of key 0 (entry index, or position % win_len)
  bool full;               // every key of the tile is visible to every row of the workgroup
};

struct Src {
  const char* kc;
  const char* vc;
  const char* kw;
  const char* vw;
  int win_len;
  __device__ __forceinline__ size_t row(const Tile& t, int j) const {
    if (j >= t.count) j = 0;  // rows past the tile end repeat its first row (masked later)
    int r = t.row0 + j;
    if (t.kind == 1 && r >= win_len) r -= win_len;  // a 32-key tile wraps the ring at most once
    return (size_t)r;
  }
};

// The calling wave DMAs rows KT / n_waves * wave .. of one tile (K or V), a run of consecutive
// rows.  A full tile that does not wrap the window ring is consecutive in memory too: one
// wave-uniform base then serves all the wave's rows through immediate offsets, and the lane
// adds a 32-bit offset made opaque at the point of use, so no per-lane pointer stays live
// across the key loop.  Other tiles (the last, partial one, or one that wraps the ring) form
// each row's address separately.
__device__ __forceinline__ void dma_rows(const Src& src, const Tile& t, bool is_v, char* dst,
                                         int ld, int wave, int n_waves, int lane) {
  const char* base = t.kind == 0 ? (is_v ? src.vc : src.kc) : (is_v ? src.vw : src.kw);
  const int n = KT / n_waves;  // rows per wave
  const int j0 = wave * n;
  if (t.count == KT && (t.kind == 0 || t.row0 + KT <= src.win_len)) {
    const char* rowp = base + (size_t)(t.row0 + j0) * ROWB;
    const uint32_t lo = (uint32_t)opaque(16 * lane);
#pragma unroll
    for (int u = 0; u < n; ++u) lds_dma16(rowp + u * ROWB + lo, dst + (j0 + u) * ld);
  } else {
#pragma unroll
    for (int u = 0; u < n; ++u) {
      const char* rowp = base + src.row(t, j0 + u) * ROWB;
      lds_dma16(rowp + (uint32_t)opaque(16 * lane), dst + (j0 + u) * ld);
    }
  }
}

// Positions of a wave's 32 query rows, all fields wave-uniform: row r (= 16nb + l16) is at
// position t0 + step * r when r < n_rows and has no position (sees nothing) otherwise.
// Prefill rows are consecutive tokens (step 1); decode rows are heads of one token (step 0).
// The lane's own row is formed where it is needed, so no per-lane row state stays live.
struct RowPos {
  int t0, n_rows, step, window, block;
};

__device__ __forceinline__ int row_t(const RowPos& rp, int r) {
  return r < rp.n_rows ? rp.t0 + rp.step * r : -1;
}

// Key j of tile t is visible to a row at position tr: compressed entry e when its block is
// complete (block * e + block - 1 <= tr), raw position s when tr - window + 1 <= s <= tr.
__device__ __forceinline__ bool visible(const Tile& t, int j, int tr, const RowPos& rp) {
  const int s = t.start + j;
  const bool in_set = t.kind == 0 ? (rp.block * s + rp.block - 1 <= tr)
                                  : ((s <= tr) & (s + rp.window - 1 >= tr));
  return (j < t.count) & in_set;
}

// Whether a tile is visible in full to rows at positions [t_lo, t_hi] (all valid).
__device__ __forceinline__ bool tile_full(const Tile& t, int t_lo, int t_hi, int window,
                                          int block) {
  if (t.count != KT || t_lo < 0) return false;
  if (t.kind == 0) return t.start + KT <= (t_lo + 1) / block;
  return t.start + KT - 1 <= t_lo && t.start >= t_hi - window + 1;
}

// 1 / l for the final normalisation; 0 for a row that never saw a visible key
__device__ __forceinline__ float final_scale(float m, float l_total) {
  return (m > 0.5f * NEG_BIG && l_total > 0.f) ? 1.f / l_total : 0.f;
}

__device__ __forceinline__ void store4(uint16_t* dst, const f32x4_t& v) {
  uint2 r;
  r.x = pack_bf16x2(v[0], v[1]);
  r.y = pack_bf16x2(v[2], v[3]);
  *(uint2*)dst = r;
}

// ------------------------------------------------------------------------- the key loop
// A wave owns 16 query rows over the whole head dimension: Q in 64 registers, O in 128.  No
// partial scores are exchanged; K and V tiles are both double buffered, so one barrier per
// tile remains.
struct RowState {
  f32x4_t o[32];  // o[cb][r] = O[row l16][16cb + 4g + r]
  float m;        // reference max (log2 domain): p = 2^(x - m) <= 2^LAZY
  float l;        // running partial sum of this lane's keys
};

__shared__ __attribute__((aligned(1024))) char pf_k0[KTILE];
__shared__ __attribute__((aligned(1024))) char pf_k1[KTILE];
__shared__ __attribute__((aligned(1024))) char pf_v0[VTILE];
__shared__ __attribute__((aligned(1024))) char pf_v1[VTILE];

// S^T of one key tile over the whole head dimension for the wave's 16 rows: A = key row
// 16mb + l16 with dims 32kk + 8g .. +7, B = query row l16 with the same dims.
__device__ __forceinline__ void row_scores(f32x4_t (&s)[2], const Frag8 (&qf)[16],
                                           const char* ks, int lane) {
  const int l16 = lane & 15, g = lane >> 4;
  s[0] = s[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const char* a0 = ks + l16 * KLD + 16 * g;
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) {
    Frag8 ka[2];
    ka[0].u = *(const uint4*)(a0 + 64 * kk);
    ka[1].u = *(const uint4*)(a0 + 64 * kk + 16 * KLD);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) s[mb] = mfma_16x16x32(ka[mb], qf[kk], s[mb]);
  }
}

// Online softmax of one tile's scores (masked unless the tile is fully visible), then
// O += V^T P^T over all 32 column blocks of the head.
__device__ __forceinline__ void row_softmax_pv(RowState& st, const f32x4_t (&s)[2],
                                               const char* vs, const Tile& t,
                                               const RowPos& rp, float scale_log2, int lane) {
  const int l16 = lane & 15, g = lane >> 4;
  float x[2][4];  // [mb][r]: key 16mb + 4g + r
  if (t.full) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) x[mb][r] = s[mb][r] * scale_log2;
  } else {
    const int tr = row_t(rp, opaque(l16));
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        x[mb][r] = visible(t, 16 * mb + 4 * g + r, tr, rp) ? s[mb][r] * scale_log2 : NEG_BIG;
  }
  float mx = x[0][0];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, x[mb][r]);
  const float m_new = fmaxf(st.m, wave_max16(mx));
  // lazy rescale: keep the reference max unless some row's max grew by more than LAZY
  if (__any(m_new > st.m + LAZY)) {
    const float alpha = fast_exp2(st.m - m_new);
    st.m = m_new;
    st.l *= alpha;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) st.o[cb] *= alpha;
  }
  float pr[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[mb][r] = fast_exp2(x[mb][r] - st.m);
      st.l += pr[mb][r];
    }
  Frag8 pf;
  pf.u = make_uint4(pack_bf16x2(pr[0][0], pr[0][1]), pack_bf16x2(pr[0][2], pr[0][3]),
                    pack_bf16x2(pr[1][0], pr[1][1]), pack_bf16x2(pr[1][2], pr[1][3]));
  // V^T fragment of column block cb: transposed reads of rows 4g + a (slots 8g..8g+3) and
  // 16 + 4g + a (slots 8g+4..8g+7), a = l16 / 4, columns 16cb + 4(l16 % 4) + 0..3.
  const char* v0 = vs + (4 * g + (l16 >> 2)) * VLD + 8 * (l16 & 3);
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) {
    Frag8 va;
    const uint2 lo = lds_read_tr16(v0 + 32 * cb);
    const uint2 hi = lds_read_tr16(v0 + 32 * cb + 16 * VLD);
    va.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
    st.o[cb] = mfma_16x16x32(va, pf, st.o[cb]);
  }
}

// Key loop shared by prefill and decode, unrolled by two so that every LDS access names its
// buffer: tile ti is read from (k0, v0) or (k1, v1) while tile ti + 1 streams into the other
// pair by LDS DMA.  The four buffers are separate LDS objects: the compiler can then prove that
// reading one pair does not touch the transfers into the other and does not wait for them.
template <class TileOf>
__device__ __forceinline__ void row_key_loop(RowState& st, const Frag8 (&qf)[16],
                                             const RowPos& rp, const Src& src,
                                             const TileOf& tile_of, int n_tiles, int wave,
                                             int n_waves, int lane, float scale_log2) {
  if (n_tiles > 0) {
    const Tile t0 = tile_of(0);
    dma_rows(src, t0, false, pf_k0, KLD, wave, n_waves, lane);
    dma_rows(src, t0, true, pf_v0, VLD, wave, n_waves, lane);
  }
  wait_all();
  __syncthreads();
  auto body = [&](int ti, const char* kcur, const char* vcur, char* knxt, char* vnxt) {
    const Tile t = tile_of(ti);
    if (ti + 1 < n_tiles) {
      const Tile tn = tile_of(ti + 1);
      dma_rows(src, tn, false, knxt, KLD, wave, n_waves, lane);
      dma_rows(src, tn, true, vnxt, VLD, wave, n_waves, lane);
    }
    f32x4_t s[2];
    row_scores(s, qf, kcur, lane);
    row_softmax_pv(st, s, vcur, t, rp, scale_log2, lane);
    wait_all();  // this wave's transfers of tile ti + 1 have landed
    __syncthreads();
  };
  for (int ti = 0; ti < n_tiles; ti += 2) {
    body(ti, pf_k0, pf_v0, pf_k1, pf_v1);
    if (ti + 1 < n_tiles) body(ti + 1, pf_k1, pf_v1, pf_k0, pf_v0);
  }
}

__device__ __forceinline__ void init_row_state(RowState& st) {
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) st.o[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  st.m = NEG_BIG;
  st.l = 0.f;
}

// ------------------------------------------------------------------------------- prefill
// One workgroup of 8 waves per (32 query tokens, 4 heads); wave w owns head 4 * hg + (w & 3)
// for rows 16 * (w >> 2) .. +15 of the token tile.  Workgroups are ordered XCD-aware:
// consecutive ids go to different XCDs (round robin), so the head groups of one token tile get
// ids that share an XCD and its key tiles are served from that XCD's L2.
__global__ __launch_bounds__(512, 1) void hca_prefill_kernel(HcaParams p) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int hw = wave & 3, rh = wave >> 2;  // head within the group, half of the token tile
  const int n_hg = (p.H + 3) / 4;
  const int n_qt = (p.Tq + 31) / 32;
  const int n_units = p.B * n_qt;
  const int xcd = blockIdx.x % 8, jj = blockIdx.x / 8;
  int unit = (jj / n_hg) * 8 + xcd;
  int hgi = jj % n_hg;
  if ((int)gridDim.x % (8 * n_hg) != 0 || unit >= n_units) {  // ragged grid: plain order
    unit = blockIdx.x / n_hg;
    hgi = blockIdx.x % n_hg;
  }
  const int b = unit / n_qt, qt = unit % n_qt;
  const int h_raw = hgi * 4 + hw;
  const bool h_ok = h_raw < p.H;  // a head count that is not a multiple of 4 leaves waves idle
  const int h = h_ok ? h_raw : p.H - 1;
  const int pos = p.pos0[b];
  const int i_first = qt * 32;
  const int i_end = min(p.Tq, i_first + 32);
  const int t_first = pos + i_first, t_last = pos + i_end - 1;
  const bool all_rows = i_end - i_first == 32;

  const int ne = t_last >= 0 ? min(p.n_cap, (t_last + 1) / p.block) : 0;
  const int s_lo = max(0, t_first - p.window + 1);
  const int nw = max(0, t_last - s_lo + 1);
  const int tiles_c = (ne + KT - 1) / KT, tiles_w = (nw + KT - 1) / KT;
  const int n_tiles = tiles_c + tiles_w;
  auto tile_of = [&](int ti) {
    Tile t;
    if (ti < tiles_c) {
      t.kind = 0;
      t.start = KT * ti;
      t.count = min(KT, ne - t.start);
      t.row0 = t.start;
    } else {
      t.kind = 1;
      t.start = s_lo + KT * (ti - tiles_c);
      t.count = min(KT, t_last - t.start + 1);
      t.row0 = t.start % p.win_len;
    }
    t.full = all_rows && tile_full(t, t_first, t_last, p.window, p.block);
    return t;
  };
  Src src;
  src.kc = (const char*)p.kc + (size_t)b * p.n_cap * ROWB;
  src.vc = (const char*)p.vc + (size_t)b * p.n_cap * ROWB;
  src.kw = (const char*)p.k_win + (size_t)b * p.win_len * ROWB;
  src.vw = (const char*)p.v_win + (size_t)b * p.win_len * ROWB;
  src.win_len = p.win_len;

  const int r_first = i_first + 16 * rh;  // token of the wave's row 0
  RowPos rp;
  rp.t0 = pos + r_first;
  rp.n_rows = i_end - r_first;  // may be <= 0: the wave's rows all lie past the end
  rp.step = 1;
  rp.window = p.window;
  rp.block = p.block;
  Frag8 qf[16];
  {
    const int i = r_first + l16;
    const int ic = min(i, i_end - 1);  // rows past the end read the last row, never stored
    const uint16_t* qr = (const uint16_t*)p.q + (((size_t)b * p.Tq + ic) * p.H + h) * D;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) qf[kk].u = *(const uint4*)(qr + 32 * kk + 8 * g);
  }
  RowState st;
  init_row_state(st);
  row_key_loop(st, qf, rp, src, tile_of, n_tiles, wave, 8, lane, p.scale * LOG2E);

  const int i = r_first + l16;
  const float inv = final_scale(st.m, wave_sum16(st.l));
  if (i < i_end && h_ok) {
    uint16_t* orow = (uint16_t*)p.out + (((size_t)b * p.Tq + i) * p.H + h) * D;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) store4(orow + 16 * cb + 4 * g, st.o[cb] * inv);
  }
}

// ------------------------------------------------------------------------------- decode
// One workgroup of 4 waves (16 heads each: the 64 heads of a group) per (sequence, key split).
// Keys of a sequence: compressed entries 0..ne-1, then raw positions s_lo..t; every row is at
// position t.  A split writes its partial (max, sum, O) unless it is the only one.
__global__ __launch_bounds__(256, 1) void hca_decode_kernel(HcaParams p, int n_split, int chunk,
                                                            float* part_o, float* part_ml) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int n_hg = p.H / 64;
  const int hg = blockIdx.x % n_hg;
  const int sp = (blockIdx.x / n_hg) % n_split;
  const int b = blockIdx.x / (n_hg * n_split);
  const int t = p.pos0[b];
  const int ne = t >= 0 ? min(p.n_cap, (t + 1) / p.block) : 0;
  const int s_lo = max(0, t - p.window + 1);
  const int nw = t >= 0 ? t - s_lo + 1 : 0;
  const int k_begin = sp * chunk, k_end = min(ne + nw, k_begin + chunk);
  const int c_end = min(k_end, ne), w_begin = max(k_begin, ne);
  const int tiles_c = k_begin < c_end ? (c_end - k_begin + KT - 1) / KT : 0;
  const int tiles_w = w_begin < k_end ? (k_end - w_begin + KT - 1) / KT : 0;
  auto tile_of = [&](int ti) {
    Tile tl;
    if (ti < tiles_c) {
      tl.kind = 0;
      tl.start = k_begin + KT * ti;
      tl.count = min(KT, c_end - tl.start);
      tl.row0 = tl.start;
    } else {
      tl.kind = 1;
      const int k0 = w_begin + KT * (ti - tiles_c);
      tl.start = s_lo + (k0 - ne);
      tl.count = min(KT, k_end - k0);
      tl.row0 = tl.start % p.win_len;
    }
    tl.full = tile_full(tl, t, t, p.window, p.block);
    return tl;
  };
  Src src;
  src.kc = (const char*)p.kc + (size_t)b * p.n_cap * ROWB;
  src.vc = (const char*)p.vc + (size_t)b * p.n_cap * ROWB;
  src.kw = (const char*)p.k_win + (size_t)b * p.win_len * ROWB;
  src.vw = (const char*)p.v_win + (size_t)b * p.win_len * ROWB;
  src.win_len = p.win_len;

  const int h = hg * 64 + 16 * wave + l16;  // this lane's head (MFMA column)
  RowPos rp;
  rp.t0 = t;
  rp.n_rows = 16;
  rp.step = 0;
  rp.window = p.window;
  rp.block = p.block;
  Frag8 qf[16];
  {
    const uint16_t* qr = (const uint16_t*)p.q + ((size_t)b * p.H + h) * D;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) qf[kk].u = *(const uint4*)(qr + 32 * kk + 8 * g);
  }
  RowState st;
  init_row_state(st);
  row_key_loop(st, qf, rp, src, tile_of, tiles_c + tiles_w, wave, 4, lane, p.scale * LOG2E);

  const float lt = wave_sum16(st.l);
  if (n_split == 1) {
    const float inv = final_scale(st.m, lt);
    uint16_t* orow = (uint16_t*)p.out + ((size_t)b * p.H + h) * D;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) store4(orow + 16 * cb + 4 * g, st.o[cb] * inv);
    return;
  }
  const size_t pr = ((size_t)b * n_split + sp) * p.H + h;
  float* po = part_o + pr * D;
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) *(f32x4_t*)(po + 16 * cb + 4 * g) = st.o[cb];
  if (g == 0) {
    part_ml[pr * 2 + 0] = st.m;
    part_ml[pr * 2 + 1] = lt;
  }
}

__global__ __launch_bounds__(128) void hca_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          uint16_t* __restrict__ out, int H,
                                                          int n_split) {
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh % H;
  float mt = NEG_BIG;
  for (int s = 0; s < n_split; ++s)
    mt = fmaxf(mt, part_ml[(((size_t)b * n_split + s) * H + h) * 2]);
  float lt = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < n_split; ++s) {
    const size_t pr = ((size_t)b * n_split + s) * H + h;
    const float a = fast_exp2(part_ml[pr * 2] - mt);  // an empty split carries the sentinel
    lt += a * part_ml[pr * 2 + 1];
    const float4 v = *(const float4*)(part_o + pr * D + 4 * threadIdx.x);
    acc[0] += a * v.x;
    acc[1] += a * v.y;
    acc[2] += a * v.z;
    acc[3] += a * v.w;
  }
  const float inv = final_scale(mt, lt);
  uint2 r;
  r.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  r.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *(uint2*)(out + (size_t)bh * D + 4 * threadIdx.x) = r;
}

void decode_plan(const HcaParams& p, int& n_split, int& chunk) {
  const long long mp = p.max_pos;
  const long long ne = std::min<long long>(p.n_cap, (mp + 1) / p.block);
  const long long nk = ne + std::min<long long>(p.window, mp + 1);
  const long long groups = (long long)p.B * (p.H / 64);
  const long long want = (256 + groups - 1) / groups;  // one workgroup per CU or more
  const long long max_split = (nk + KT - 1) / KT;
  n_split = (int)std::max<long long>(1, std::min(want, max_split));
  long long c = (nk + n_split - 1) / n_split;
  c = (c + KT - 1) / KT * KT;
  chunk = (int)std::max<long long>(c, KT);
  n_split = (int)std::max<long long>(1, (nk + chunk - 1) / chunk);
}

// the decode kernel takes one query row per sequence and whole groups of 64 heads; the
// prefill kernel takes groups of 4 heads and any number of rows
bool use_decode(const HcaParams& p) { return p.Tq == 1 && p.H % 64 == 0; }

}  // namespace

size_t hca_bf16_workspace(const HcaParams& p) {
  if (!use_decode(p)) return 0;
  int n_split, chunk;
  decode_plan(p, n_split, chunk);
  if (n_split == 1) return 0;
  const size_t rows = (size_t)p.B * n_split * p.H;
  return rows * D * sizeof(float) + rows * 2 * sizeof(float);
}

hipError_t launch_hca_bf16(const HcaParams& p, hipStream_t stream) {
  hipError_t e;
  if (use_decode(p)) {
    int n_split, chunk;
    decode_plan(p, n_split, chunk);
    float* part_o = (float*)p.ws;
    float* part_ml = part_o ? part_o + (size_t)p.B * n_split * p.H * D : nullptr;
    const long long grid = (long long)p.B * (p.H / 64) * n_split;
    hipLaunchKernelGGL(hca_decode_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p,
                       n_split, chunk, part_o, part_ml);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (n_split > 1) {
      hipLaunchKernelGGL(hca_combine_kernel, dim3(p.B * p.H), dim3(128), 0, stream, part_o,
                         part_ml, (uint16_t*)p.out, p.H, n_split);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  } else {
    const long long grid = (long long)p.B * ((p.Tq + 31) / 32) * ((p.H + 3) / 4);
    hipLaunchKernelGGL(hca_prefill_kernel, dim3((unsigned)grid), dim3(512), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.q_lat != nullptr)  // the gate GEMM multiplies sigmoid(q_lat W) into O in place
    return launch_gate(p.q_lat, p.w_gate, p.out, p.out, p.B * p.Tq, p.d_lat, p.H * D, DT_BF16,
                       stream);
  return hipSuccess;
}

}  // namespace lgsa
