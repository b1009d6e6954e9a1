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
// Prefill, ungated: one workgroup of 8 waves per (32 query tokens, 4 heads).  Prefill, gated:
// one workgroup of 8 waves per (128 query tokens, 1 head) that applies the gate in its epilogue.
// Decode: one workgroup of 4 waves (the 64 heads of one token) per (sequence, key split);
// partial (max, sum, O) of a split go to the workspace and a second kernel merges them.  When
// gated, that kernel is the gate's: it streams W once, 64 channels of every row per workgroup,
// and multiplies sigmoid(q_lat W) into the merged O of those channels.
#include <type_traits>

#include "common.h"
#include "gate_skinny.h"
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
// 16mb + l16 with dims 32kk + 8g .. +7, B = query row l16 with the same dims.  The even and
// odd contraction steps accumulate separately and are summed at the end: four independent
// chains of 8 products instead of two of 16.
__device__ __forceinline__ void row_scores(f32x4_t (&s)[2], const Frag8 (&qf)[16],
                                           const char* ks, int lane) {
  const int l16 = lane & 15, g = lane >> 4;
  s[0] = s[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t s_odd[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  const char* a0 = ks + l16 * KLD + 16 * g;
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) {
    Frag8 ka[2];
    ka[0].u = *(const uint4*)(a0 + 64 * kk);
    ka[1].u = *(const uint4*)(a0 + 64 * kk + 16 * KLD);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      if (kk & 1) s_odd[mb] = mfma_16x16x32(ka[mb], qf[kk], s_odd[mb]);
      else s[mb] = mfma_16x16x32(ka[mb], qf[kk], s[mb]);
    }
  }
  s[0] += s_odd[0];
  s[1] += s_odd[1];
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
    // the keys j of the tile that the lane's row (position tr) sees form one range
    // [j_lo, j_hi], the rule of visible() solved for j once per tile
    const int tr = row_t(rp, opaque(l16));
    int j_lo, j_hi;
    if (t.kind == 0) {  // entries: block (s + 1) <= tr + 1
      j_lo = 0;
      j_hi = tr >= 0 ? (tr + 1) / rp.block - 1 - t.start : -1;
    } else {  // raw positions: tr - window + 1 <= s <= tr
      j_lo = tr - rp.window + 1 - t.start;
      j_hi = tr - t.start;
    }
    j_hi = min(j_hi, t.count - 1);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * mb + 4 * g + r;
        x[mb][r] = (j >= j_lo && j <= j_hi) ? s[mb][r] * scale_log2 : NEG_BIG;
      }
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
// WITH_V = false streams the key tiles alone.
template <bool WITH_V = true, class TileOf, class Consume>
__device__ __forceinline__ void tile_key_loop(const Src& src, const TileOf& tile_of, int n_tiles,
                                              int wave, int n_waves, int lane,
                                              const Consume& consume) {
  if (n_tiles > 0) {
    const Tile t0 = tile_of(0);
    dma_rows(src, t0, false, pf_k0, KLD, wave, n_waves, lane);
    if (WITH_V) dma_rows(src, t0, true, pf_v0, VLD, wave, n_waves, lane);
  }
  wait_all();
  __syncthreads();
  auto body = [&](int ti, const char* kcur, const char* vcur, char* knxt, char* vnxt) {
    const Tile t = tile_of(ti);
    if (ti + 1 < n_tiles) {
      const Tile tn = tile_of(ti + 1);
      dma_rows(src, tn, false, knxt, KLD, wave, n_waves, lane);
      if (WITH_V) dma_rows(src, tn, true, vnxt, VLD, wave, n_waves, lane);
    }
    consume(t, kcur, vcur);
    wait_all();  // this wave's transfers of tile ti + 1 have landed
    __syncthreads();
  };
  for (int ti = 0; ti < n_tiles; ti += 2) {
    body(ti, pf_k0, pf_v0, pf_k1, pf_v1);
    if (ti + 1 < n_tiles) body(ti + 1, pf_k1, pf_v1, pf_k0, pf_v0);
  }
}

template <class TileOf>
__device__ __forceinline__ void row_key_loop(RowState& st, const Frag8 (&qf)[16],
                                             const RowPos& rp, const Src& src,
                                             const TileOf& tile_of, int n_tiles, int wave,
                                             int n_waves, int lane, float scale_log2) {
  tile_key_loop(src, tile_of, n_tiles, wave, n_waves, lane,
                [&](const Tile& t, const char* kcur, const char* vcur) {
                  f32x4_t s[2];
                  row_scores(s, qf, kcur, lane);
                  row_softmax_pv(st, s, vcur, t, rp, scale_log2, lane);
                });
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
  const float lt = wave_sum16(st.l);
  const float inv = final_scale(st.m, lt);
  if (i < i_end && h_ok) {
    uint16_t* orow = (uint16_t*)p.out + (((size_t)b * p.Tq + i) * p.H + h) * D;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) store4(orow + 16 * cb + 4 * g, st.o[cb] * inv);
    // ln sum_j exp(scale s_j) = (m + log2 l) ln 2 in the log2 domain of the key loop
    if (p.lse != nullptr && g == 0)
      p.lse[((size_t)b * p.Tq + i) * p.H + h] =
          inv > 0.f ? (st.m + __log2f(lt)) * 0.69314718055994531f : -INFINITY;
  }
}

// ------------------------------------------------------------------ gated prefill (fused)
// The gate is applied in the epilogue of the attention, so O never goes to memory: the HBM
// traffic of the gated step is Q in and out once.  One workgroup of 8 waves per (sequence,
// 128 query tokens, head): wave w owns tokens 16w .. 16w + 15 of the tile over the whole
// 512-wide head, with the key loop above.  The workgroup streams the union of its waves' key
// tiles; each wave computes only the tiles holding a key that one of its rows sees (5 of the 8
// window tiles of a whole tile) and skips the masking of tiles its rows see in full.
//
// Then the gate G = q_lat W for the tile's 128 rows and the head's 512 channels, sliced by
// channel: wave w computes G^T for channels 64w .. 64w + 63 and all 128 rows, so each W^T
// fragment feeds 8 products.  Each contraction step of 32 brings a 32-row slice of the head's
// W columns (its transposed reads give W^T) and the 128 q_lat rows' 32 columns to LDS by LDS
// DMA, through a four-stage ring, three steps ahead of the one being read (the stages reuse
// the key/value buffers, 160 KiB of LDS in all).  Meanwhile O waits in the registers as packed bfloat16 (the value the unfused path
// would store).  sigmoid(G), rounded to bfloat16, crosses to the row layout of O through LDS;
// each wave writes out = O * sigmoid(G) over it and stores its 16 rows whole, 1 KiB per
// instruction.
constexpr int FQ = 128;  // query tokens per workgroup of the gated prefill kernel

// Whether tile t holds a key visible to some row at positions [t_lo, t_hi] (all valid).
__device__ __forceinline__ bool tile_touches(const Tile& t, int t_lo, int t_hi, int window,
                                             int block) {
  if (t.kind == 0) return block * t.start + block - 1 <= t_hi;
  return t.start <= t_hi && t.start + t.count - 1 >= t_lo - window + 1;
}

// The gate loop's transfers are issued in inline assembly (LDS DMA, global_load_lds_dwordx4:
// lane l's 16 bytes land at M0 + 16 l).  The compiler then does not see them and does not make
// every LDS read wait for the transfers in flight into the other stages; the loop waits for
// its own transfers (wait_vm) before the barrier that precedes their reads.  The instruction
// writes no register, so nothing the compiler allocates is written late.
// M0 is named as clobbered (the compiler warns that it keeps no value of its own there across
// the statement; no code after these transfers relies on one).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_asm(const char* base, uint32_t lane_off, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %0"
      :
      : "s"(base), "v"(lane_off), "s"(lds)
      : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// W stage of the gate: 32 tile rows of 1 KiB, unpadded; the 16-byte chunk c of tile row r sits
// at position c ^ gw_sw(r), which keeps the transposing reads free of bank conflicts (measured
// as fast as rows padded by 32 bytes) and leaves room in LDS for a fourth stage.
constexpr int GROW = 1024;
__device__ __forceinline__ int gw_sw(int r) { return 2 * (r & 7) + 16 * ((r >> 3) & 1); }

// Step k0 of the gate contraction into one stage: rows k0 + 4 wave .. + 3 of the head's W
// slice (1 KiB each) into the stage's W tile, contraction index k0 + 8c + 4h + a (c, h, a
// < 4, 2, 4) at tile row 16h + 4c + a (lane l fetching chunk l ^ gw_sw of that row), and the
// wave's 16 q_lat rows, columns k0 .. k0 + 31 (64 bytes each), into its own 1 KiB block qdst
// of the stage's q_lat tile, which holds the workgroup's 128 rows in 8 such blocks:
// chunk-major within a block, lane l fetching 16-byte chunk l / 16 of row l % 16, so that a
// fragment read (chunk g of rows l16) is 1 KiB read contiguously by the 64 lanes, which the
// LDS serves without bank conflicts.  Five transfers per wave.
// ql_wave is the q_lat row of the wave's first row and q_off the lane's byte offset from it
// (its row, clamped to the last row, and its chunk).
__device__ __forceinline__ void gate_dma(const char* w_head, size_t ldw, const char* ql_wave,
                                         uint32_t q_off, int k0, char* wdst, char* qdst,
                                         int wave, int lane) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {  // index 4 wave + u: c = wave / 2, h = wave % 2, a = u
    const int tr = 16 * (wave & 1) + 4 * (wave >> 1) + u;
    dma16_asm(w_head + (size_t)(k0 + 4 * wave + u) * ldw,
              (uint32_t)opaque(16 * (lane ^ gw_sw(tr))), lds_addr(wdst + tr * GROW));
  }
  dma16_asm(ql_wave + 2 * k0, (uint32_t)opaque((int)q_off), lds_addr(qdst));
}

// One contraction step of 32 for the wave's 64 channels (64 wave .. + 63 of the head) and all
// 128 rows of the tile: G^T = W^T q_lat^T, acc[i][j] = G^T of channels 64 wave + 16 i .. and
// rows 16 j ..  W^T comes from the stage's W tile through the transposing read of tile rows
// 4g + a and 16 + 4g + a, which hold contraction indices 8g + a and 8g + 4 + a: slots
// 8g .. 8g + 7 take indices 8g .. 8g + 7 in order, so the q_lat^T fragment of a lane is one
// 16-byte chunk of its q_lat row (qblk(j): the stage's block of rows 16j ..).  Each W^T
// fragment feeds 8 products and each q_lat fragment 4.
template <class QBlk>
__device__ __forceinline__ void gate_step(f32x4_t (&acc)[4][8], const char* ws, const QBlk& qblk,
                                          int wave, int lane) {
  const int l16 = lane & 15, g = lane >> 4;
  const int r = 4 * g + (l16 >> 2);  // tile row of the lo read; the hi read is row r + 16
  const int fx = gw_sw(r);           // = gw_sw(r + 16)
  const char* wr = ws + r * GROW + 8 * (l16 & 1);
  const int cl = (l16 & 3) >> 1;
  Frag8 wa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const char* a = wr + 16 * ((8 * wave + 2 * i + cl) ^ fx);
    const uint2 lo = lds_read_tr16(a);
    const uint2 hi = lds_read_tr16(a + 16 * GROW);
    wa[i].u = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    Frag8 qf;
    qf.u = *(const uint4*)(qblk(j) + 256 * g + 16 * l16);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][j] = mfma_16x16x32(wa[i], qf, acc[i][j]);
  }
}

__shared__ __attribute__((aligned(1024))) char pf_q0[8 * 1024];
__shared__ __attribute__((aligned(1024))) char pf_q1[8 * 1024];
__shared__ __attribute__((aligned(1024))) char pf_q2[8 * 1024];
// the fourth q_lat stage: blocks 0..3 in the 1 KiB past the W tile in each key/value buffer,
// blocks 4..7 here
__shared__ __attribute__((aligned(1024))) char pf_q3h[4 * 1024];

__global__ __launch_bounds__(512, 1) void hca_prefill_gated_kernel(HcaParams p) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int n_qt = (p.Tq + FQ - 1) / FQ;
  // XCD-aware order (consecutive ids go to the 8 XCDs in turn): XCD x takes the heads
  // x H/8 .. x H/8 + H/8 - 1 of every token tile, token tiles in descending order (longer key
  // lists first) from a starting point of its own, and the heads of a tile one after another.
  // The ~32 workgroups an XCD holds at once are then 4 token tiles x 8 heads: each key/value
  // tile is read by 8 of them from the XCD's L2, and each head's W slice by 4.
  int qt, h, b;
  if (p.H % 8 == 0) {
    const int hx = p.H / 8, idx = blockIdx.x / 8;
    h = (blockIdx.x % 8) * hx + idx % hx;
    const int tt = idx / hx;  // (sequence, rank of the token tile in the order below)
    b = tt / n_qt;
    // descending from a starting tile that differs by XCD (x n_qt / 8), wrapping around: the
    // workgroups of one XCD stay in step (they share W slices and key tiles in its L2), while
    // the 8 XCDs are at different points of the order, so their Q loads and out stores spread
    // over the launch instead of all CUs moving Q or out at the same moment
    const int u = tt % n_qt;
    qt = n_qt - 1 - (u + (int)(blockIdx.x % 8) * (n_qt / 8)) % n_qt;
  } else {
    qt = n_qt - 1 - (int)blockIdx.x % n_qt;
    h = (blockIdx.x / n_qt) % p.H;
    b = blockIdx.x / (n_qt * p.H);
  }
  const int pos = p.pos0[b];
  const int i_first = qt * FQ;
  const int i_end = min(p.Tq, i_first + FQ);
  const int t_first = pos + i_first, t_last = pos + i_end - 1;

  const int ne = t_last >= 0 ? min(p.n_cap, (t_last + 1) / p.block) : 0;
  const int s_lo = max(0, t_first - p.window + 1);
  const int nw = max(0, t_last - s_lo + 1);
  const int tiles_c = (ne + KT - 1) / KT, tiles_w = (nw + KT - 1) / KT;
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
    t.full = false;  // decided per wave
    return t;
  };
  Src src;
  src.kc = (const char*)p.kc + (size_t)b * p.n_cap * ROWB;
  src.vc = (const char*)p.vc + (size_t)b * p.n_cap * ROWB;
  src.kw = (const char*)p.k_win + (size_t)b * p.win_len * ROWB;
  src.vw = (const char*)p.v_win + (size_t)b * p.win_len * ROWB;
  src.win_len = p.win_len;

  const int r_first = i_first + 16 * wave;  // token of the wave's row 0
  const int n_valid = max(0, min(16, i_end - r_first));
  RowPos rp;
  rp.t0 = pos + r_first;
  rp.n_rows = i_end - r_first;
  rp.step = 1;
  rp.window = p.window;
  rp.block = p.block;
  const int tw_lo = pos + r_first, tw_hi = pos + r_first + n_valid - 1;
  Frag8 qf[16];
  {
    // rows past the end read the last row and are never stored
    const int i_row = min(r_first + l16, i_end - 1);
    const uint16_t* qr = (const uint16_t*)p.q + (((size_t)b * p.Tq + i_row) * p.H + h) * D;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) qf[kk].u = *(const uint4*)(qr + 32 * kk + 8 * g);
  }
  RowState st;
  init_row_state(st);
  const float scale_log2 = p.scale * LOG2E;
  tile_key_loop(src, tile_of, tiles_c + tiles_w, wave, 8, lane,
                [&](const Tile& t0, const char* kcur, const char* vcur) {
                  if (n_valid == 0 || tw_lo < 0 ||
                      !tile_touches(t0, tw_lo, tw_hi, p.window, p.block))
                    return;
                  Tile t = t0;
                  t.full = n_valid == 16 && tile_full(t, tw_lo, tw_hi, p.window, p.block);
                  f32x4_t s[2];
                  row_scores(s, qf, kcur, lane);
                  row_softmax_pv(st, s, vcur, t, rp, scale_log2, lane);
                });

  const int i = r_first + l16;
  const float lt = wave_sum16(st.l);
  const float inv = final_scale(st.m, lt);
  if (p.lse != nullptr && g == 0 && i < i_end)
    p.lse[((size_t)b * p.Tq + i) * p.H + h] =
        inv > 0.f ? (st.m + __log2f(lt)) * 0.69314718055994531f : -INFINITY;
  uint2 ob[32];  // O rounded to bfloat16, as the unfused path stores it
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) {
    ob[cb].x = pack_bf16x2(st.o[cb][0] * inv, st.o[cb][1] * inv);
    ob[cb].y = pack_bf16x2(st.o[cb][2] * inv, st.o[cb][3] * inv);
    // pins the packing here: left to itself the compiler sinks it to the epilogue and keeps
    // the fp32 O (twice the registers) live through the gate loop
    asm volatile("" : "+v"(ob[cb].x), "+v"(ob[cb].y));
  }

  // ------------------------------------------------------------------ gate
  // Four stages (W tile + q_lat tile), three steps in flight ahead of the one being read.
  const size_t ldw = (size_t)p.H * D * 2;  // bytes of one W row
  const size_t ldq = (size_t)p.d_lat * 2;  // bytes of one q_lat row
  const char* w_head = (const char*)p.w_gate + (size_t)h * ROWB;
  // the wave's first q_lat row; rows past the end read the last row (and are never stored)
  const int r_dma = min(r_first, i_end - 1);
  const char* ql_wave = (const char*)p.q_lat + ((size_t)b * p.Tq + r_dma) * ldq;
  const uint32_t q_off = (uint32_t)((min(r_first + (lane & 15), i_end - 1) - r_dma) * (int)ldq +
                                    16 * (lane >> 4));
  const int nk = p.d_lat / KT;  // contraction steps of 32
  f32x4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // stage st: W tile in key/value buffer st, q_lat blocks in pf_q<st> (st < 3) or split over
  // the four buffers' last KiB and pf_q3h (st = 3)
  auto wst = [](int st) { return st == 0 ? pf_k0 : (st == 1 ? pf_v0 : (st == 2 ? pf_k1 : pf_v1)); };
  auto qblk = [&](int st, int j) -> char* {
    if (st < 3) return (st == 0 ? pf_q0 : (st == 1 ? pf_q1 : pf_q2)) + 1024 * j;
    return j < 4 ? wst(j) + 32 * GROW : pf_q3h + 1024 * (j - 4);
  };
  auto issue = [&](int step, int st) {
    gate_dma(w_head, ldw, ql_wave, q_off, step * KT, wst(st), qblk(st, wave), wave, lane);
  };
  // the key loop ended with a barrier: every stage is free
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  if (nk > 2) issue(2, 2);
  if (nk > 2) wait_vm<10>(); else if (nk > 1) wait_vm<5>(); else wait_vm<0>();
  lds_barrier();
  // step s on stage ST = s % 4; step s + 3 goes into the stage step s - 1 read (free since the
  // barrier that ended it); at the end, step s + 1 must have landed while the transfers of
  // steps s + 2 and s + 3 (5 each, when they exist) may still fly
  auto one = [&](int s, auto stc) {
    constexpr int ST = decltype(stc)::value;
    if (s + 3 < nk) issue(s + 3, (ST + 3) & 3);
    gate_step(acc, wst(ST), [&](int j) { return qblk(ST, j); }, wave, lane);
    const int later = min(nk - 1, s + 3) - (s + 1);
    if (later >= 2) wait_vm<10>(); else if (later == 1) wait_vm<5>(); else wait_vm<0>();
    lds_barrier();
  };
  for (int s = 0; s < nk; s += 4) {
    one(s, std::integral_constant<int, 0>());
    if (s + 1 < nk) one(s + 1, std::integral_constant<int, 1>());
    if (s + 2 < nk) one(s + 2, std::integral_constant<int, 2>());
    if (s + 3 < nk) one(s + 3, std::integral_constant<int, 3>());
  }

  // sigmoid(G) as bfloat16 into LDS, rows of the tile 32 to a buffer (pitch VLD): the last
  // step ended with a barrier, so every buffer is free
  auto sbuf = [](int q4) { return q4 == 0 ? pf_k0 : (q4 == 1 ? pf_v0 : (q4 == 2 ? pf_k1 : pf_v1)); };
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    char* rowp = sbuf(j >> 1) + (16 * (j & 1) + l16) * VLD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint2 v;
      v.x = pack_bf16x2(sigmoidf_fast(acc[i][j][0]), sigmoidf_fast(acc[i][j][1]));
      v.y = pack_bf16x2(sigmoidf_fast(acc[i][j][2]), sigmoidf_fast(acc[i][j][3]));
      *(uint2*)(rowp + 2 * (64 * wave + 16 * i + 4 * g)) = v;
    }
  }
  lds_barrier();
  // out = O * sigmoid(G) for the wave's own rows, in the layout of O, written over the gate
  // factors it replaces; then the wave stores its 16 rows whole, 1 KiB per instruction
  char* tile = sbuf(wave >> 1) + 16 * (wave & 1) * VLD;
  {
    char* srow = tile + l16 * VLD + 8 * g;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      const uint2 sg = *(const uint2*)(srow + 32 * cb);
      const float o0 = __uint_as_float(ob[cb].x << 16), o1 = __uint_as_float(ob[cb].x & 0xFFFF0000u);
      const float o2 = __uint_as_float(ob[cb].y << 16), o3 = __uint_as_float(ob[cb].y & 0xFFFF0000u);
      uint2 r;
      r.x = pack_bf16x2(o0 * __uint_as_float(sg.x << 16), o1 * __uint_as_float(sg.x & 0xFFFF0000u));
      r.y = pack_bf16x2(o2 * __uint_as_float(sg.y << 16), o3 * __uint_as_float(sg.y & 0xFFFF0000u));
      *(uint2*)(srow + 32 * cb) = r;
    }
  }
  char* orow0 = (char*)p.out + (((size_t)b * p.Tq + r_first) * p.H + h) * ROWB + 16 * lane;
  const size_t ldo = (size_t)p.H * ROWB;
#pragma unroll
  for (int rr = 0; rr < 16; ++rr)
    if (r_first + rr < i_end)
      *(uint4*)(orow0 + rr * ldo) = *(const uint4*)(tile + rr * VLD + 16 * lane);
}

// ------------------------------------------------------------------------------- decode
// One workgroup of 4 waves (16 heads each: the 64 heads of a group) per (sequence, key split).
// Keys of a sequence: compressed entries 0..ne-1, then raw positions s_lo..t; every row is at
// position t.  A split writes its partial (max, sum, O) to the workspace, unless it is the
// only one and no gate follows (then it writes the output).
// One key split of one sequence for the 64 heads of a group (the decode kernel's attention).
__device__ __forceinline__ void decode_split(const HcaParams& p, int n_split, int chunk,
                                             float* part_o, float* part_ml, bool partials,
                                             int wave, int lane) {
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
  if (!partials) {  // the only split, not gated here: the output directly
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

__global__ __launch_bounds__(256, 1) void hca_decode_kernel(HcaParams p, int n_split, int chunk,
                                                            float* part_o, float* part_ml,
                                                            bool partials) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  decode_split(p, n_split, chunk, part_o, part_ml, partials, wave, lane);
}

// splits whose partials the decode gate kernel loads before its K loop
constexpr int MERGE_PRE = 4;

// The merged O of the decode splits for the gate tile's epilogue (gate_skinny.h): the lane's
// row b and its four 4-channel groups n .. n + 3 + 48 of head h.  The partials of the first
// PRE splits are loaded before the gate's K loop, the others in the epilogue.  Values are
// rounded to bfloat16, as the output stores O.
template <int PRE>
struct MergedO {
  const float* part_o;
  const float* part_ml;
  int H, n_split;
  size_t base;  // partial row (b, split 0, h) times D, plus the channel
  size_t ml0;   // (b, split 0, h) in part_ml pairs
  float2 ml[PRE];
  float4 v[4][PRE];

  __device__ __forceinline__ void fetch(int b, int n) {
    const int h = n / D, j = n % D;
    base = (((size_t)b * n_split) * H + h) * D + j;
    ml0 = ((size_t)b * n_split) * H + h;
#pragma unroll
    for (int s = 0; s < PRE; ++s) {
      if (s < n_split) {
        ml[s] = *(const float2*)(part_ml + (ml0 + (size_t)s * H) * 2);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          v[cb][s] = *(const float4*)(part_o + base + (size_t)s * H * D + 16 * cb);
      }
    }
  }
  __device__ __forceinline__ float4 value(int cb) const {
    float mt = NEG_BIG;
#pragma unroll
    for (int s = 0; s < PRE; ++s)
      if (s < n_split) mt = fmaxf(mt, ml[s].x);
    for (int s = PRE; s < n_split; ++s) mt = fmaxf(mt, part_ml[(ml0 + (size_t)s * H) * 2]);
    float lt = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
    auto add = [&](float m, float l, float4 x) {
      const float a = fast_exp2(m - mt);  // an empty split carries the sentinel
      lt += a * l;
      acc[0] += a * x.x;
      acc[1] += a * x.y;
      acc[2] += a * x.z;
      acc[3] += a * x.w;
    };
#pragma unroll
    for (int s = 0; s < PRE; ++s)
      if (s < n_split) add(ml[s].x, ml[s].y, v[cb][s]);
    for (int s = PRE; s < n_split; ++s) {
      const float2 q = *(const float2*)(part_ml + (ml0 + (size_t)s * H) * 2);
      add(q.x, q.y, *(const float4*)(part_o + base + (size_t)s * H * D + 16 * cb));
    }
    const float inv = final_scale(mt, lt);
    auto rb = [](float x) { return __uint_as_float(pack_bf16x2(x, 0.f) << 16); };
    return make_float4(rb(acc[0] * inv), rb(acc[1] * inv), rb(acc[2] * inv), rb(acc[3] * inv));
  }
};

// Gated decode, second kernel: the gate tile of gate_skinny.h over channels 64 blockIdx .. + 63
// of every sequence (rows of q_lat), whose epilogue merges the splits of those channels and
// multiplies them: out = bf16(O) * sigmoid(q_lat W), what the gate GEMM does to a stored O.
__shared__ __attribute__((aligned(1024))) char dg_st0[gate_skinny::STAGE];
__shared__ __attribute__((aligned(1024))) char dg_st1[gate_skinny::STAGE];
__shared__ __attribute__((aligned(1024))) char dg_st2[gate_skinny::STAGE];
__shared__ __attribute__((aligned(1024))) char dg_st3[gate_skinny::STAGE];

__global__ __launch_bounds__(256) void hca_decode_gate_kernel(HcaParams p, int n_split,
                                                              const float* __restrict__ part_o,
                                                              const float* __restrict__ part_ml) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto stage = [](int i) -> char* {
    return i == 0 ? dg_st0 : i == 1 ? dg_st1 : i == 2 ? dg_st2 : dg_st3;
  };
  MergedO<MERGE_PRE> ov;
  ov.part_o = part_o;
  ov.part_ml = part_ml;
  ov.H = p.H;
  ov.n_split = n_split;
  gate_skinny::tile<16>((const uint16_t*)p.q_lat, (const uint16_t*)p.w_gate, ov,
                        (uint16_t*)p.out, p.B, p.H * D, blockIdx.x * gate_skinny::N_TILE, stage,
                        wave, lane);
}

// Merges the splits of one (sequence, head): 128 threads of 4 channels.
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

// Whether the gate kernel of the decode path merges the splits: the tile of gate_skinny.h (at
// most 64 rows, d_lat = 1024), with at most MERGE_PRE splits, whose partials it loads before
// its K loop (more splits, for few long sequences, would be read after it, one after
// another).  Otherwise a combine kernel merges them and the gate GEMM follows.

bool decode_fuses_gate(const HcaParams& p) {
  if (p.q_lat == nullptr || p.B * p.Tq > 64 || p.d_lat != 16 * gate_skinny::K_STEP) return false;
  int n_split, chunk;
  decode_plan(p, n_split, chunk);
  return n_split <= MERGE_PRE;
}

// ------------------------------------------------------------------------------ backward
// Prefill backward (every sequence from position 0).  With P = softmax of the scaled logits
// (rebuilt from the forward's log-sum-exp), dP = dO V^T and D = rowsum(dO * O):
//   dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO
// over the keys of each row.  A compressed entry's gradient reaches each position of its
// block divided by block.  Three stages:
//   hca_bwd_dq_kernel   per (32 query tokens, 4 heads), as the forward: recomputes S and dP
//                       tile by tile, accumulates dQ (two passes of 256 columns: Q, dO and
//                       half of dQ fill the registers), and in its first pass writes P and
//                       scale * dS of every (row, key) pair: for the entries to [rows][ne_pad],
//                       for the window to [rows][window] at column t - s;
//   entry gradients     dKc = dSc^T Q and dVc = Pc^T dO as split-K GEMMs over all rows;
//   hca_bwd_dkv_kernel  per 64 keys: the window gradients as banded products over the query
//                       tokens s .. s + window - 1 of every head, plus dKc / block and
//                       dVc / block of the key's block, written as dK and dV.
__global__ __launch_bounds__(256) void hca_bwd_delta_kernel(const uint16_t* __restrict__ dout,
                                                            const uint16_t* __restrict__ out,
                                                            float* __restrict__ delta,
                                                            long long rows) {
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const uint4 a = *(const uint4*)(dout + r * D + 8 * lane);
  const uint4 o = *(const uint4*)(out + r * D + 8 * lane);
  const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, ow[4] = {o.x, o.y, o.z, o.w};
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sum = fmaf(__uint_as_float(aw[j] << 16), __uint_as_float(ow[j] << 16), sum);
    sum = fmaf(__uint_as_float(aw[j] & 0xFFFF0000u), __uint_as_float(ow[j] & 0xFFFF0000u), sum);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane == 0) delta[r] = sum;
}

struct BwdWs {  // workspace regions of the backward
  float* delta;
  uint16_t* pc;
  uint16_t* dsc;
  uint16_t* pw;
  uint16_t* dsw;
  float* dkc;
  float* dvc;
  float* part;
  int ne_pad, splits;
};

__global__ __launch_bounds__(512, 1) void hca_bwd_dq_kernel(HcaBwdParams bp, BwdWs ws) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int hw = wave & 3, rh = wave >> 2;
  const int n_hg = bp.H / 4;
  const int n_qt = (bp.T + 31) / 32;
  // XCD-aware order as in the forward: the head groups of one token tile share an XCD
  const int n_units = bp.B * n_qt;
  const int xcd = blockIdx.x % 8, jj = blockIdx.x / 8;
  int unit = (jj / n_hg) * 8 + xcd, hgi = jj % n_hg;
  if ((int)gridDim.x % (8 * n_hg) != 0 || unit >= n_units) {  // ragged grid: plain order
    unit = blockIdx.x / n_hg;
    hgi = blockIdx.x % n_hg;
  }
  const int b = unit / n_qt, qt = unit % n_qt;
  const int h = hgi * 4 + hw;
  const int T = bp.T, W = bp.window;
  const int i_first = qt * 32, i_end = min(T, i_first + 32);
  const int t_first = i_first, t_last = i_end - 1;
  const bool all_rows = i_end - i_first == 32;
  const int ne = min(bp.ne, (t_last + 1) / bp.block);
  const int s_lo = max(0, t_first - W + 1);
  const int nw = t_last - s_lo + 1;
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
      t.row0 = t.start;
    }
    t.full = all_rows && tile_full(t, t_first, t_last, W, bp.block);
    return t;
  };
  Src src;
  src.kc = (const char*)bp.kc + (size_t)b * bp.ne * ROWB;
  src.vc = (const char*)bp.vc + (size_t)b * bp.ne * ROWB;
  src.kw = (const char*)bp.k + (size_t)b * T * ROWB;
  src.vw = (const char*)bp.v + (size_t)b * T * ROWB;
  src.win_len = T;

  const int r_first = i_first + 16 * rh;
  RowPos rp;
  rp.t0 = r_first;
  rp.n_rows = i_end - r_first;
  rp.step = 1;
  rp.window = W;
  rp.block = bp.block;
  const int i = r_first + l16;
  const bool row_ok = i < i_end;
  const int ic = min(i, i_end - 1);
  const size_t row = ((size_t)b * T + ic) * bp.H + h;
  Frag8 qf[16], of[16];
  {
    const uint16_t* qr = (const uint16_t*)bp.q + row * D;
    const uint16_t* dr = (const uint16_t*)bp.dout + row * D;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      qf[kk].u = *(const uint4*)(qr + 32 * kk + 8 * g);
      of[kk].u = *(const uint4*)(dr + 32 * kk + 8 * g);
    }
  }
  const float lse2 = bp.lse[row] * LOG2E;
  const float dlt = ws.delta[row];
  const float scale_log2 = bp.scale * LOG2E;
  uint16_t* pc = ws.pc + row * ws.ne_pad;
  uint16_t* dsc = ws.dsc + row * ws.ne_pad;
  uint16_t* pw = ws.pw + row * W;
  uint16_t* dsw = ws.dsw + row * W;

  // dQ^T += K^T (scale dS)^T over 16 column blocks (256 columns, half hf of the head), K read
  // through the transposing read as V is in the forward; the B operand is scale dS rounded to
  // bfloat16, the value the workspace holds
  auto dq_tile = [&](f32x4_t (&dq)[16], const Frag8& pf, const char* kcur, int hf) {
    const char* k0 = kcur + (4 * g + (l16 >> 2)) * KLD + 8 * (l16 & 3) + 512 * hf;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) {
      Frag8 ka;
      const uint2 lo = lds_read_tr16(k0 + 32 * cb);
      const uint2 hi = lds_read_tr16(k0 + 32 * cb + 16 * KLD);
      ka.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
      dq[cb] = mfma_16x16x32(ka, pf, dq[cb]);
    }
  };
  auto store_dq = [&](const f32x4_t (&dq)[16], int hf) {
    if (row_ok) {
      uint16_t* dr = (uint16_t*)bp.dq + row * D + 256 * hf;
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) store4(dr + 16 * cb + 4 * g, dq[cb]);
    }
  };
  {
    // First half: S and dP from K, V and the rows' Q, dO; P and scale dS of every (row, key)
    // to the workspace.
    f32x4_t dq[16];
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) dq[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    tile_key_loop(src, tile_of, n_tiles, wave, 8, lane,
                  [&](const Tile& t, const char* kcur, const char* vcur) {
      f32x4_t sc[2], dp[2];
      row_scores(sc, qf, kcur, lane);
      row_scores(dp, of, vcur, lane);
      const int tr = row_t(rp, opaque(l16));
      float pr[2][4], ds[2][4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool vis = t.full || visible(t, 16 * mb + 4 * g + r, tr, rp);
          pr[mb][r] = vis ? fast_exp2(sc[mb][r] * scale_log2 - lse2) : 0.f;
          ds[mb][r] = pr[mb][r] * (dp[mb][r] - dlt) * bp.scale;
        }
      uint2 dsb[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        dsb[mb] = make_uint2(pack_bf16x2(ds[mb][0], ds[mb][1]), pack_bf16x2(ds[mb][2], ds[mb][3]));
      if (row_ok) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int j0 = t.start + 16 * mb + 4 * g;  // keys j0 .. j0 + 3
          if (t.kind == 0) {
            if (j0 < ws.ne_pad) {
              *(uint2*)(pc + j0) = make_uint2(pack_bf16x2(pr[mb][0], pr[mb][1]),
                                              pack_bf16x2(pr[mb][2], pr[mb][3]));
              *(uint2*)(dsc + j0) = dsb[mb];
            }
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int jj = i - (j0 + r);  // column t - s of the window arrays
              if (jj >= 0 && jj < W) {
                pw[jj] = f32_to_bf16(pr[mb][r]);
                dsw[jj] = (uint16_t)((r & 1 ? (r < 2 ? dsb[mb].x : dsb[mb].y) >> 16
                                            : (r < 2 ? dsb[mb].x : dsb[mb].y)) & 0xFFFFu);
              }
            }
          }
        }
      }
      Frag8 pf;
      pf.u = make_uint4(dsb[0].x, dsb[0].y, dsb[1].x, dsb[1].y);
      dq_tile(dq, pf, kcur, 0);
    });
    store_dq(dq, 0);
  }
  {
    // Second half: scale dS read back from the workspace (this lane wrote it above; 0 where the
    // row does not see the key), so S and dP are not formed again and only K is streamed.
    f32x4_t dq[16];
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) dq[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    tile_key_loop<false>(src, tile_of, n_tiles, wave, 8, lane,
                         [&](const Tile& t, const char* kcur, const char*) {
      uint2 dsb[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int j0 = t.start + 16 * mb + 4 * g;
        dsb[mb] = make_uint2(0u, 0u);
        if (!row_ok) continue;
        if (t.kind == 0) {
          if (j0 < ws.ne_pad) dsb[mb] = *(const uint2*)(dsc + j0);
        } else {
          uint32_t h4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int jj = i - (j0 + r);
            h4[r] = (jj >= 0 && jj < W) ? (uint32_t)dsw[jj] : 0u;
          }
          dsb[mb] = make_uint2(h4[0] | (h4[1] << 16), h4[2] | (h4[3] << 16));
        }
      }
      Frag8 pf;
      pf.u = make_uint4(dsb[0].x, dsb[0].y, dsb[1].x, dsb[1].y);
      dq_tile(dq, pf, kcur, 1);
    });
    store_dq(dq, 1);
  }
  // entries past the workgroup's last tile are invisible to its rows: zeros
  if (row_ok)
    for (int e = tiles_c * KT + 4 * g; e < ws.ne_pad; e += 16) {
      *(uint2*)(pc + e) = make_uint2(0u, 0u);
      *(uint2*)(dsc + e) = make_uint2(0u, 0u);
    }
}

constexpr int BW_CLD = 32 + 8;  // LDS row of a coefficient tile (bf16)
constexpr int BW_NK = 64;       // keys per workgroup of the dkv kernel
constexpr int BW_NKB = BW_NK / 16;

// Window gradients of 64 keys s0 .. s0 + 63 and the final dK, dV.  Wave w owns the dims
// 64w .. 64w + 63.  For every query-token tile of 32 and head h: the coefficient tiles
// C[s][t] = scale dS (or P) of (t, h) at key s when 0 <= t - s < window, and the 32 rows of Q
// (or dO) of head h go to LDS; then dK[s][c] += sum_t C[s][t] Q[t][c] on the MFMA (A = C rows,
// B = Q^T by the transposing read).
// The steps of a workgroup are (head h, token tile t0) pairs, token tiles fastest; the Q and dO
// rows of step i + 1 stream into one pair of LDS buffers by LDS DMA (rows past T repeat the
// last row: their coefficients are 0) and its coefficients into registers while step i's
// products run on the other pair, with one barrier per step.
__shared__ __attribute__((aligned(16))) uint16_t bw_ck0[BW_NK * BW_CLD];
__shared__ __attribute__((aligned(16))) uint16_t bw_cv0[BW_NK * BW_CLD];
__shared__ __attribute__((aligned(16))) uint16_t bw_ck1[BW_NK * BW_CLD];
__shared__ __attribute__((aligned(16))) uint16_t bw_cv1[BW_NK * BW_CLD];

__global__ __launch_bounds__(512, 1) void hca_bwd_dkv_kernel(HcaBwdParams bp, BwdWs ws) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int T = bp.T, W = bp.window, H = bp.H;
  const int n_kt = (T + BW_NK - 1) / BW_NK;
  // XCD-aware order: XCD x takes a contiguous run of key blocks, so the ~32 blocks it holds at
  // once are neighbours, whose token bands overlap (each Q and dO row is needed by about three
  // of them) and are served from its L2
  const int n_blk = (int)gridDim.x;
  const int lin = n_blk % 8 == 0 ? (int)(blockIdx.x % 8) * (n_blk / 8) + (int)blockIdx.x / 8
                                 : (int)blockIdx.x;
  const int b = lin / n_kt, s0 = (lin % n_kt) * BW_NK;
  f32x4_t ak[BW_NKB][4], av[BW_NKB][4];
#pragma unroll
  for (int sb = 0; sb < BW_NKB; ++sb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) ak[sb][cb] = av[sb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // tokens that see one of the keys: s0 .. t_end - 1; steps are (head, token tile) pairs, token
  // tiles fastest, so neighbouring key blocks need the same rows within a few steps
  const int t_end = min(T, s0 + BW_NK - 1 + W);
  const int n_tt = (t_end - s0 + 31) / 32;
  const int n_steps = n_tt * H;
  // Q and dO rows of step i: 64 rows of 1 KiB (32 of Q, then 32 of dO), eight per wave
  auto dma_step = [&](int i, char* dq, char* dd) {
    const int t0 = s0 + 32 * (i % n_tt), h = i / n_tt;
    const uint32_t lo = (uint32_t)opaque(16 * lane);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = 8 * wave + u;  // wave-uniform
      const int rr = row & 31;
      const int t = min(t0 + rr, T - 1);
      const char* src = (const char*)(row < 32 ? bp.q : bp.dout) +
                        ((((size_t)b * T + t) * H + h) * D) * 2;
      lds_dma16(src + lo, (row < 32 ? dq : dd) + rr * KLD);
    }
  };
  // coefficients of keys s0 + sr and tokens t0 + tc, BW_NK / 16 (sr, tc) per thread; the keys
  // run fastest across lanes, so a wave's loads read one token's BW_NK consecutive window
  // offsets (one row of the workspace) instead of one value from each of 32 rows
  uint16_t cfk[BW_NK / 16], cfv[BW_NK / 16];
  auto load_coef = [&](int i) {
    const int t0 = s0 + 32 * (i % n_tt), h = i / n_tt;
#pragma unroll
    for (int u = 0; u < BW_NK / 16; ++u) {
      const int e = tid + 512 * u;  // 0 .. 32 BW_NK - 1
      const int sr = e % BW_NK, tc = e / BW_NK;
      const int s = s0 + sr, t = t0 + tc, jj = t - s;
      cfk[u] = cfv[u] = 0;
      if (t < T && s < T && jj >= 0 && jj < W) {
        const size_t at = (((size_t)b * T + t) * H + h) * W + jj;
        cfk[u] = ws.dsw[at];
        cfv[u] = ws.pw[at];
      }
    }
  };
  auto store_coef = [&](uint16_t* ck, uint16_t* cv) {
#pragma unroll
    for (int u = 0; u < BW_NK / 16; ++u) {
      const int e = tid + 512 * u;
      const int sr = e % BW_NK, tc = e / BW_NK;
      ck[sr * BW_CLD + tc] = cfk[u];
      cv[sr * BW_CLD + tc] = cfv[u];
    }
  };
  // A = coefficient rows (keys 16sb + l16, tokens 8g .. 8g + 7); B = Q^T / dO^T columns
  // 64 wave + 16cb + l16 of tokens 8g .. 8g + 7 (two transposed reads of 4 rows each)
  const int rowa = (8 * g + (l16 >> 2)) * KLD + 2 * (64 * wave + 4 * (l16 & 3));
  auto compute = [&](const char* sq, const char* so, const uint16_t* ck, const uint16_t* cv) {
    Frag8 fk[BW_NKB], fv[BW_NKB];
#pragma unroll
    for (int sb = 0; sb < BW_NKB; ++sb) {
      fk[sb].u = *(const uint4*)(&ck[(16 * sb + l16) * BW_CLD + 8 * g]);
      fv[sb].u = *(const uint4*)(&cv[(16 * sb + l16) * BW_CLD + 8 * g]);
    }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      Frag8 bq, bo;
      const uint2 q0 = lds_read_tr16(sq + rowa + 32 * cb);
      const uint2 q1 = lds_read_tr16(sq + rowa + 32 * cb + 4 * KLD);
      const uint2 o0 = lds_read_tr16(so + rowa + 32 * cb);
      const uint2 o1 = lds_read_tr16(so + rowa + 32 * cb + 4 * KLD);
      bq.u = make_uint4(q0.x, q0.y, q1.x, q1.y);
      bo.u = make_uint4(o0.x, o0.y, o1.x, o1.y);
#pragma unroll
      for (int sb = 0; sb < BW_NKB; ++sb) {
        ak[sb][cb] = mfma_16x16x32(fk[sb], bq, ak[sb][cb]);
        av[sb][cb] = mfma_16x16x32(fv[sb], bo, av[sb][cb]);
      }
    }
  };
  if (n_steps > 0) {
    dma_step(0, pf_k0, pf_v0);
    load_coef(0);
  }
  wait_all();
  store_coef(bw_ck0, bw_cv0);
  __syncthreads();
  // step i reads buffers (q, o, ck, cv) of its parity; step i + 1 fills the other set, whose
  // previous contents step i - 1 read before the barrier that ended it
  auto step = [&](int i, const char* q, const char* o, const uint16_t* ck, const uint16_t* cv,
                  char* qn, char* on, uint16_t* ckn, uint16_t* cvn) {
    const bool more = i + 1 < n_steps;
    if (more) {
      dma_step(i + 1, qn, on);
      load_coef(i + 1);
    }
    compute(q, o, ck, cv);
    wait_all();  // this wave's transfers and coefficients of step i + 1
    if (more) store_coef(ckn, cvn);
    __syncthreads();
  };
  for (int i = 0; i < n_steps; i += 2) {
    step(i, pf_k0, pf_v0, bw_ck0, bw_cv0, pf_k1, pf_v1, bw_ck1, bw_cv1);
    if (i + 1 < n_steps) step(i + 1, pf_k1, pf_v1, bw_ck1, bw_cv1, pf_k0, pf_v0, bw_ck0, bw_cv0);
  }
  // lane holds dK, dV[s = s0 + 16sb + 4g + r][c = 64 wave + 16cb + l16]
  const float inv_blk = 1.0f / (float)bp.block;
#pragma unroll
  for (int sb = 0; sb < BW_NKB; ++sb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = s0 + 16 * sb + 4 * g + r;
      if (s >= T) continue;
      const int e = s / bp.block;
      const bool pooled = e < bp.ne;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int c = 64 * wave + 16 * cb + l16;
        float gk = ak[sb][cb][r], gv = av[sb][cb][r];
        if (pooled) {
          gk += ws.dkc[((size_t)b * ws.ne_pad + e) * D + c] * inv_blk;
          gv += ws.dvc[((size_t)b * ws.ne_pad + e) * D + c] * inv_blk;
        }
        ((uint16_t*)bp.dk)[((size_t)b * T + s) * D + c] = f32_to_bf16(gk);
        ((uint16_t*)bp.dv)[((size_t)b * T + s) * D + c] = f32_to_bf16(gv);
      }
    }
}

BwdWs bwd_layout(const HcaBwdParams& p, size_t* total) {
  BwdWs w;
  const size_t rows = (size_t)p.B * p.T * p.H;
  w.ne_pad = (std::max(p.ne, 1) + 7) / 8 * 8;
  w.splits = (int)std::max<size_t>(1, std::min<size_t>(128, rows / 4096));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) / 256 * 256;
    return at;
  };
  const size_t o_delta = take(rows * 4);
  const size_t o_pc = take(rows * w.ne_pad * 2), o_dsc = take(rows * w.ne_pad * 2);
  const size_t o_pw = take(rows * p.window * 2), o_dsw = take(rows * p.window * 2);
  const size_t o_dkc = take((size_t)p.B * w.ne_pad * D * 4);
  const size_t o_dvc = take((size_t)p.B * w.ne_pad * D * 4);
  const size_t o_part = take((size_t)w.splits * w.ne_pad * D * 4);
  *total = off;
  char* base = (char*)p.ws;
  w.delta = (float*)(base + o_delta);
  w.pc = (uint16_t*)(base + o_pc);
  w.dsc = (uint16_t*)(base + o_dsc);
  w.pw = (uint16_t*)(base + o_pw);
  w.dsw = (uint16_t*)(base + o_dsw);
  w.dkc = (float*)(base + o_dkc);
  w.dvc = (float*)(base + o_dvc);
  w.part = (float*)(base + o_part);
  return w;
}

}  // namespace

size_t hca_bwd_workspace(const HcaBwdParams& p) {
  size_t total = 0;
  bwd_layout(p, &total);
  return total;
}

hipError_t launch_hca_bwd(const HcaBwdParams& p, hipStream_t stream) {
  size_t total = 0;
  const BwdWs w = bwd_layout(p, &total);
  const long long rows = (long long)p.B * p.T * p.H;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(hca_bwd_delta_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                     stream, (const uint16_t*)p.dout, (const uint16_t*)p.out, w.delta, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long grid = (long long)p.B * ((p.T + 31) / 32) * (p.H / 4);
  hipLaunchKernelGGL(hca_bwd_dq_kernel, dim3((unsigned)grid), dim3(512), 0, stream, p, w);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // entry gradients per sequence: dKc = dSc^T Q, dVc = Pc^T dO over its T * H rows
  const long long rows_b = (long long)p.T * p.H;
  for (int b = 0; b < p.B && p.ne > 0; ++b) {
    const size_t ro = (size_t)b * rows_b;
    e = launch_gemm_splitk_f32(w.dsc + ro * w.ne_pad, w.ne_pad, true,
                               (const uint16_t*)p.q + ro * D, D, true,
                               w.dkc + (size_t)b * w.ne_pad * D, w.ne_pad, D, (int)rows_b,
                               w.splits, w.part, stream);
    if (e != hipSuccess) return e;
    e = launch_gemm_splitk_f32(w.pc + ro * w.ne_pad, w.ne_pad, true,
                               (const uint16_t*)p.dout + ro * D, D, true,
                               w.dvc + (size_t)b * w.ne_pad * D, w.ne_pad, D, (int)rows_b,
                               w.splits, w.part, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(hca_bwd_dkv_kernel, dim3((unsigned)(p.B * ((p.T + BW_NK - 1) / BW_NK))),
                     dim3(512),
                     0, stream, p, w);
  return hipGetLastError();
}

size_t hca_bf16_workspace(const HcaParams& p) {
  if (!use_decode(p)) return 0;
  int n_split, chunk;
  decode_plan(p, n_split, chunk);
  if (n_split == 1 && !decode_fuses_gate(p)) return 0;
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
    const bool fuse = decode_fuses_gate(p);
    const long long grid = (long long)p.B * (p.H / 64) * n_split;
    hipLaunchKernelGGL(hca_decode_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p,
                       n_split, chunk, part_o, part_ml, n_split > 1 || fuse);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (fuse) {  // the gate kernel merges the splits and multiplies the gate in
      const int slices = (p.H * D + gate_skinny::N_TILE - 1) / gate_skinny::N_TILE;
      hipLaunchKernelGGL(hca_decode_gate_kernel, dim3(slices), dim3(256), 0, stream, p, n_split,
                         part_o, part_ml);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    } else if (n_split > 1) {
      hipLaunchKernelGGL(hca_combine_kernel, dim3(p.B * p.H), dim3(128), 0, stream, part_o,
                         part_ml, (uint16_t*)p.out, p.H, n_split);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (p.q_lat != nullptr && !fuse) {  // the gate GEMM multiplies sigmoid(q_lat W) into O
      e = launch_gate(p.q_lat, p.w_gate, p.out, p.out, p.B * p.Tq, p.d_lat, p.H * D, DT_BF16,
                      stream);
      if (e != hipSuccess) return e;
    }
  } else if (p.q_lat != nullptr) {  // the gate in the attention epilogue
    const long long grid = (long long)p.B * ((p.Tq + FQ - 1) / FQ) * p.H;
    hipLaunchKernelGGL(hca_prefill_gated_kernel, dim3((unsigned)grid), dim3(512), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    const long long grid = (long long)p.B * ((p.Tq + 31) / 32) * ((p.H + 3) / 4);
    hipLaunchKernelGGL(hca_prefill_kernel, dim3((unsigned)grid), dim3(512), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // the head mix (VHA) of the gated output: a workgroup of these kernels holds one head of a
  // token tile (prefill) or splits the keys (decode), so the mix runs as its own pass in place
  if (p.vha_r > 0)
    return launch_vha(p.out, p.vha_u, p.vha_v, p.out, p.B * p.Tq, p.H, D, p.vha_r, DT_BF16,
                      stream);
  return hipSuccess;
}

}  // namespace lgsa
