// Heavily Compressed Attention forward, bfloat16, 512-wide heads, for gfx950 (v2 kernels).
//
// ERNIE 5.5 Flash Base release blog, section 2.1 "Latent-Gated Sparse Attention": each HCA
// layer keeps one cache entry per 128 tokens and attends densely to all completed entries plus
// a short window of recent raw tokens (128 tokens per the xenospectrum.com article on ERNIE 5.5
// Flash Base, long-context section); HCA heads are 512 wide; every layer multiplies the
// attention output by a gate computed from the low-rank query latent.  Visibility is
// closed-form: position t sees compressed entry e iff e < (t + 1) / block, raw position s iff
// t - window + 1 <= s <= t.
//
// On-chip budget for 512-wide heads.  A wave owns 32 query rows; a 32x512 fp32 accumulator
// plus the 32x512 bf16 query would take 384 of the 512 registers a lane has, so the two waves
// of a pair share 32 rows and split the head dimension: each holds half of Q (64 registers)
// and half of O (128).  Each computes S^T over its half of the dimensions; the partial scores
// are swapped through LDS and summed (both waves form the same sum, so their softmax is
// identical) and each wave then accumulates its half of O.
//
// Data movement.  Key and value tiles (32 rows x 1 KiB) go straight from global memory to
// LDS with buffer-less LDS DMA (global_load_lds_dwordx4, 1 KiB per wave instruction), two
// stages deep, without passing through registers.  Bank conflicts are removed by an XOR
// swizzle of the 16-byte chunks of each row, applied by permuting which chunk every lane
// fetches.  The value tile stays row-major: the MFMA operand V^T is read with the gfx950
// transposing LDS read (ds_read_b64_tr_b16).
//
// Products on v_mfma_f32_16x16x32_bf16, transposed (S^T = K Q^T, O^T = V^T P^T): the tile in
// LDS is the A operand, the query rows in registers the B operand, so a lane owns one query
// row for all its accumulators and the P fragment of the second product is the S^T
// accumulator of the first (keys relabelled so that no data moves between lanes).
//
// Prefill: one workgroup of 8 waves (4 pairs) per 128 query rows: TG token groups of 32 rows
// by 4/TG heads.  The gate logits q_lat . W for the workgroup's rows and channels are
// computed after the key loop with the same scheme (W^T read transposed from row-major LDS
// tiles, q_lat rows from registers) and multiplied into O before the only store.
// Decode: one workgroup of 4 waves (2 pairs = 64 heads) per (sequence, key split); partial
// (max, sum, O) of a split go to the workspace and a combine kernel merges them.
#include "common.h"
#include "kernels.h"

namespace lgsa {

namespace {

constexpr int D = 512;
constexpr int HALF = 256;
constexpr int KT = 32;                   // keys per tile
constexpr int ROWB = 1024;               // bytes of one 512-wide bf16 row
constexpr int TILEB = KT * ROWB;         // 32 KiB
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ int swz_k(int r) { return r & 15; }
__device__ __forceinline__ int swz_v(int r) { return 2 * (r & 7); }
__device__ __forceinline__ int swz_w(int r) { return 2 * (r & 3) + 8 * ((r >> 3) & 1); }


struct Tile {
  int kind, start, count;  // kind 0: compressed entries start.., kind 1: raw positions start..
  int row0;                // buffer row of key 0 (entry index, or position % win_len)
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

// Stage one tile: the calling wave DMAs rows r0, r0 + step, ... of K and of V.
__device__ __forceinline__ void dma_tile(const Src& src, const Tile& t, char* ks, char* vs,
                                         int r0, int step, int lane) {
  for (int j = r0; j < KT; j += step) {
    const size_t row = src.row(t, j);
    const char* kr = (t.kind == 0 ? src.kc : src.kw) + row * ROWB;
    const char* vr = (t.kind == 0 ? src.vc : src.vw) + row * ROWB;
    lds_dma16(kr + 16 * (lane ^ swz_k(j)), ks + j * ROWB);
    lds_dma16(vr + 16 * (lane ^ swz_v(j)), vs + j * ROWB);
  }
}

// Per-wave state: 32 query rows (column blocks nb = 0, 1), one half of the head dimension.
struct HalfState {
  f32x4_t o[16][2];  // o[cb][nb][r] = O[row 16nb + l16][hf*256 + 16cb + 4g + r]
  float m[2];
  float l[2];
};

// Per query row: position t, number of visible compressed entries, first visible raw position
// (a row with t < 0 sees nothing: ncv = 0 and wlo > t).
struct RowVis {
  int t, ncv, wlo;
};

__device__ __forceinline__ RowVis row_vis(int t, int window, int block) {
  RowVis v;
  v.t = t;
  v.ncv = t >= 0 ? (t + 1) / block : 0;
  v.wlo = t >= 0 ? t - window + 1 : t + 1;
  return v;
}

__device__ __forceinline__ bool visible(const Tile& t, int j, const RowVis& v) {
  const int s = t.start + j;
  const bool in_set = t.kind == 0 ? (s < v.ncv) : ((s <= v.t) & (s >= v.wlo));
  return (j < t.count) & in_set;
}

// Masked logits take this finite sentinel instead of -inf, which keeps the online softmax
// free of special cases: while a row has seen no visible key its running max is the
// sentinel, whatever it accumulated is scaled by 2^(sentinel - real max) = 0 as soon as a
// visible key arrives, and a row that never sees one is written as zeros.
constexpr float NEG_BIG = -1.0e30f;

// S^T over this wave's half of the head dimension.  Rows 16mb + l16 carry swizzle l16, and
// the chunk index hf*32 + 4kk + g has the kk bits disjoint from the lane bits, so the address
// of step kk is one XOR of an immediate into the lane's base address.
__device__ __forceinline__ void partial_scores(f32x4_t (&s)[2][2], const Frag8 (&qf)[2][8],
                                               const char* ks, int hf, int lane) {
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) s[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int base = opaque(l16 * ROWB + 16 * ((hf * 32 + g) ^ l16));
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const char* a0 = ks + (base ^ (64 * kk));
    Frag8 ka[2];
    ka[0].u = *(const uint4*)(a0);
    ka[1].u = *(const uint4*)(a0 + 16 * ROWB);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) s[mb][nb] = mfma_16x16x32(ka[mb], qf[nb][kk], s[mb][nb]);
  }
}

// Masked online softmax of the full scores and O-half += V-half^T P^T.
__device__ __forceinline__ void softmax_pv(HalfState& st, const f32x4_t (&s)[2][2],
                                           const char* vs, const Tile& t, const RowVis (&rv)[2],
                                           float scale_log2, int hf, int lane) {
  const int l16 = lane & 15, g = lane >> 4;
  float alpha[2];
  Frag8 pf[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float x[2][4];
    float mx = NEG_BIG;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * mb + 4 * g + r;
        x[mb][r] = visible(t, j, rv[nb]) ? s[mb][nb][r] * scale_log2 : NEG_BIG;
        mx = fmaxf(mx, x[mb][r]);
      }
    mx = wave_max16(mx);
    const float m_new = fmaxf(st.m[nb], mx);
    alpha[nb] = fast_exp2(st.m[nb] - m_new);
    st.m[nb] = m_new;
    float p[2][4], psum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[mb][r] = fast_exp2(x[mb][r] - m_new);
        psum += p[mb][r];
      }
    st.l[nb] = st.l[nb] * alpha[nb] + psum;
    pf[nb].u = make_uint4(pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                          pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3]));
  }
  if (__any((alpha[0] != 1.f) | (alpha[1] != 1.f))) {
#pragma unroll
    for (int cb = 0; cb < 16; ++cb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) st.o[cb][nb] *= alpha[nb];
  }
  // V^T fragment of column block cb: two transposed reads (slots 8g..8g+3 from rows
  // 4g + a, slots 8g+4..8g+7 from rows 16 + 4g + a, a = l16 / 4).  Both rows share the
  // swizzle 2 * ((4g + a) & 7); the cb bits of the chunk index are disjoint from it, so block
  // cb is one XOR of an immediate into the lane's base address.
  const int a = l16 >> 2, c4 = l16 & 3;
  const int r_lo = 4 * g + a;
  const int vbase = opaque(r_lo * ROWB + 16 * ((hf * 32 + (c4 >> 1)) ^ swz_v(r_lo)) +
                           (c4 & 1) * 8);
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) {
    const char* va_lo = vs + (vbase ^ (32 * cb));
    Frag8 va;
    const uint2 lo = lds_read_tr16(va_lo);
    const uint2 hi = lds_read_tr16(va_lo + 16 * ROWB);
    va.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) st.o[cb][nb] = mfma_16x16x32(va, pf[nb], st.o[cb][nb]);
  }
}

__device__ __forceinline__ void init_state(HalfState& st) {
#pragma unroll
  for (int cb = 0; cb < 16; ++cb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) st.o[cb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  st.m[0] = st.m[1] = NEG_BIG;
  st.l[0] = st.l[1] = 0.f;
}

// 1 / l for the final normalisation; 0 for a row that never saw a visible key
__device__ __forceinline__ float final_scale(float m, float l_total) {
  return (m > 0.5f * NEG_BIG && l_total > 0.f) ? 1.f / l_total : 0.f;
}

// partial scores are swapped through LDS: xs[wave][q][lane] f32x4, q = mb * 2 + nb
__device__ __forceinline__ void xs_write(char* xs, int wave, int lane, const f32x4_t (&s)[2][2]) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      *(f32x4_t*)(xs + ((wave * 4 + mb * 2 + nb) * 64 + lane) * 16) = s[mb][nb];
}

__device__ __forceinline__ void xs_add(const char* xs, int wave, int lane, f32x4_t (&s)[2][2]) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      s[mb][nb] += *(const f32x4_t*)(xs + ((wave * 4 + mb * 2 + nb) * 64 + lane) * 16);
}

__device__ __forceinline__ void store4(uint16_t* dst, const f32x4_t& v) {
  uint2 r;
  r.x = pack_bf16x2(v[0], v[1]);
  r.y = pack_bf16x2(v[2], v[3]);
  *(uint2*)dst = r;
}

extern __shared__ __attribute__((aligned(1024))) char hca2_smem[];

// ------------------------------------------------------------------------------- prefill
// LDS: K stages [0, 64K), V stages [64K, 128K), score exchange [128K, 160K).
constexpr int PF_XS = 4 * TILEB;
constexpr size_t PF_SMEM = 5 * TILEB;
constexpr int GK = 64;  // gate contraction step

template <int TG>
__global__ __launch_bounds__(512, 1) void hca_prefill2_kernel(HcaParams p) {
  constexpr int NH = 4 / TG;  // heads per workgroup
  char* smem = hca2_smem;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps derived values scalar
  const int l16 = lane & 15, g = lane >> 4;
  const int pair = wave >> 1, hf = wave & 1;
  const int tg = pair % TG, hh = pair / TG;
  // workgroup -> (sequence, query tile of 32*TG rows, head group of NH heads), heads fastest
  const int n_hg = p.H / NH;
  const int rows_wg = 32 * TG;
  const int n_qt = (p.Tq + rows_wg - 1) / rows_wg;
  const int hgi = blockIdx.x % n_hg;
  const int qt = (blockIdx.x / n_hg) % n_qt;
  const int b = blockIdx.x / (n_hg * n_qt);
  const int h = hgi * NH + hh;
  const int pos = p.pos0[b];
  const int i_first = qt * rows_wg;
  const int i_end = min(p.Tq, i_first + rows_wg);
  const int t_first = pos + i_first, t_last = pos + i_end - 1;

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
    return t;
  };
  Src src;
  src.kc = (const char*)p.kc + (size_t)b * p.n_cap * ROWB;
  src.vc = (const char*)p.vc + (size_t)b * p.n_cap * ROWB;
  src.kw = (const char*)p.k_win + (size_t)b * p.win_len * ROWB;
  src.vw = (const char*)p.v_win + (size_t)b * p.win_len * ROWB;
  src.win_len = p.win_len;

  // this pair's 32 rows
  const int wi0 = i_first + 32 * tg;
  RowVis rv[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int i = wi0 + 16 * nb + l16;
    rv[nb] = row_vis(i < i_end ? pos + i : -1, p.window, p.block);
  }
  const int wa = pos + wi0, wb = pos + min(i_end, wi0 + 32) - 1;
  const bool live = wi0 < i_end && wb >= 0;
  const int wne = live ? (wb + 1) / p.block : 0;

  Frag8 qf[2][8];
  const uint16_t* qb = (const uint16_t*)p.q;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    // rows past the end load the last row: their results are never stored
    const int i = min(wi0 + 16 * nb + l16, i_end - 1);
    const uint16_t* qr = qb + (((size_t)b * p.Tq + i) * p.H + h) * D + hf * HALF;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[nb][kk].u = *(const uint4*)(qr + 32 * kk + 8 * g);
  }
  HalfState st;
  init_state(st);
  const float scale_log2 = p.scale * LOG2E;
  char* xs = smem + PF_XS;

  if (n_tiles > 0) dma_tile(src, tile_of(0), smem, smem + 2 * TILEB, wave, 8, lane);
  wait_all();
  __syncthreads();
  for (int ti = 0; ti < n_tiles; ++ti) {
    const int buf = ti & 1;
    if (ti + 1 < n_tiles)
      dma_tile(src, tile_of(ti + 1), smem + (buf ^ 1) * TILEB, smem + (2 + (buf ^ 1)) * TILEB,
               wave, 8, lane);
    const Tile t = tile_of(ti);
    bool rel = live;
    if (t.kind == 0)
      rel = rel && t.start < wne;
    else
      rel = rel && t.start <= wb && t.start + t.count - 1 >= wa - p.window + 1;
    f32x4_t s[2][2];
    if (rel) {
      partial_scores(s, qf, smem + buf * TILEB, hf, lane);
      xs_write(xs, wave, lane, s);
    }
    __syncthreads();
    if (rel) {
      xs_add(xs, wave ^ 1, lane, s);
      softmax_pv(st, s, smem + (2 + buf) * TILEB, t, rv, scale_log2, hf, lane);
    }
    wait_all();
    __syncthreads();
  }

  float inv[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) inv[nb] = final_scale(st.m[nb], wave_sum16(st.l[nb]));
#pragma unroll
  for (int cb = 0; cb < 16; ++cb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) st.o[cb][nb] *= inv[nb];

  uint16_t* out = (uint16_t*)p.out;
  if (p.q_lat == nullptr) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int i = wi0 + 16 * nb + l16;
      if (i >= i_end) continue;
      uint16_t* orow = out + (((size_t)b * p.Tq + i) * p.H + h) * D + hf * HALF;
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) store4(orow + 16 * cb + 4 * g, st.o[cb][nb]);
    }
    return;
  }

  // ---- fused gate: G^T[n][row] = sum_k W[k][n] q_lat[row][k] for the wave's 256 channels,
  // 128 at a time.  W k-rows are staged row-major in LDS (segments of 128 channels, one per
  // head and half: NH*2 segments of 64 x 128) and read transposed.
  const int N = p.H * D;
  const uint16_t* w = (const uint16_t*)p.w_gate;
  const uint16_t* ql = (const uint16_t*)p.q_lat;
  constexpr int SEGB = GK * 256;            // one segment: 64 k-rows x 256 bytes
  constexpr int STAGEB = NH * 2 * SEGB;     // all segments of one k step
  const int n_k = p.d_lat / GK;
  const int seg = hh * 2 + hf;
  const size_t qrow[2] = {(size_t)b * p.Tq + min(wi0 + l16, i_end - 1),
                          (size_t)b * p.Tq + min(wi0 + 16 + l16, i_end - 1)};
  // DMA of one k step: NH*2 segments x 16 instructions of 4 k-rows; 8 waves share them
  auto dma_w = [&](int cc, int kt, char* dst) {
    for (int ins = wave; ins < NH * 2 * 16; ins += 8) {
      const int sg = ins >> 4, kr = (ins & 15) * 4;      // segment, first k-row
      const int shh = sg >> 1, shf = sg & 1;
      const int r = kr + (lane >> 4);                     // k-row of this lane
      const int col0 = (hgi * NH + shh) * D + shf * HALF + cc * 128;
      const uint16_t* srow = w + (size_t)(kt * GK + r) * N + col0;
      lds_dma16(srow + 8 * ((lane & 15) ^ swz_w(r)), dst + sg * SEGB + kr * 256);
    }
  };
  __syncthreads();  // all waves are done with the key loop's LDS
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    f32x4_t ga[8][2];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) ga[c][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    dma_w(cc, 0, smem);
    uint4 qv[2][2];  // q_lat fragments of the current k step: [nb][ks]
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
        qv[nb][k2] = *(const uint4*)(ql + qrow[nb] * p.d_lat + 32 * k2 + 8 * g);
    wait_all();
    __syncthreads();
    for (int kt = 0; kt < n_k; ++kt) {
      const int buf = kt & 1;
      uint4 qn[2][2];
      if (kt + 1 < n_k) {
        dma_w(cc, kt + 1, smem + (buf ^ 1) * STAGEB);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2)
            qn[nb][k2] = *(const uint4*)(ql + qrow[nb] * p.d_lat + (kt + 1) * GK + 32 * k2 +
                                         8 * g);
      }
      const char* sw = smem + buf * STAGEB + seg * SEGB;
      // W^T fragment (channel block c, k rows 32k2 + 8g + a and + 4): both rows share the
      // swizzle 2a + 8(g & 1); the c bits of the chunk index are disjoint from it.
      const int a = l16 >> 2, c4 = l16 & 3;
      const int wbase = opaque((8 * g + a) * 256 +
                               16 * ((c4 >> 1) ^ (2 * a + 8 * (g & 1))) + (c4 & 1) * 8);
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        Frag8 qb2[2];
        qb2[0].u = qv[0][k2];
        qb2[1].u = qv[1][k2];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const char* wl = sw + (wbase ^ (32 * c)) + k2 * 32 * 256;
          const uint2 lo = lds_read_tr16(wl);
          const uint2 hi = lds_read_tr16(wl + 4 * 256);
          Frag8 wa_;
          wa_.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) ga[c][nb] = mfma_16x16x32(wa_, qb2[nb], ga[c][nb]);
        }
      }
      if (kt + 1 < n_k) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) qv[nb][k2] = qn[nb][k2];
      }
      wait_all();
      __syncthreads();
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int i = wi0 + 16 * nb + l16;
      if (i >= i_end) continue;
      uint16_t* orow = out + (((size_t)b * p.Tq + i) * p.H + h) * D + hf * HALF + cc * 128;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        f32x4_t v = st.o[cc * 8 + c][nb];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] *= sigmoidf_fast(ga[c][nb][r]);
        store4(orow + 16 * c + 4 * g, v);
      }
    }
  }
}

// ------------------------------------------------------------------------------- decode
// One workgroup of 4 waves = 2 pairs (heads 0..31, 32..63 of a 64-head group) per
// (sequence, key split).  Keys of a sequence: compressed entries 0..ne-1 then raw positions
// s_lo..t.  LDS: K stages [0, 64K), V stages [64K, 128K), exchange [128K, 144K).
constexpr size_t DEC_SMEM = 4 * TILEB + 4 * 4 * 64 * 16;

__global__ __launch_bounds__(256, 1) void hca_decode2_kernel(HcaParams p, int n_split, int chunk,
                                                             float* part_o, float* part_ml) {
  char* smem = hca2_smem;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps derived values scalar
  const int l16 = lane & 15, g = lane >> 4;
  const int pair = wave >> 1, hf = wave & 1;
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
  const int n_tiles = tiles_c + tiles_w;
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
    return tl;
  };
  Src src;
  src.kc = (const char*)p.kc + (size_t)b * p.n_cap * ROWB;
  src.vc = (const char*)p.vc + (size_t)b * p.n_cap * ROWB;
  src.kw = (const char*)p.k_win + (size_t)b * p.win_len * ROWB;
  src.vw = (const char*)p.v_win + (size_t)b * p.win_len * ROWB;
  src.win_len = p.win_len;

  const int h0 = hg * 64 + 32 * pair;
  const RowVis rv0 = row_vis(t, p.window, p.block);
  const RowVis rv[2] = {rv0, rv0};
  Frag8 qf[2][8];
  const uint16_t* qb = (const uint16_t*)p.q + (size_t)b * p.H * D;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const uint16_t* qr = qb + (size_t)(h0 + 16 * nb + l16) * D + hf * HALF;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[nb][kk].u = *(const uint4*)(qr + 32 * kk + 8 * g);
  }
  HalfState st;
  init_state(st);
  const float scale_log2 = p.scale * LOG2E;
  char* xs = smem + 4 * TILEB;

  if (n_tiles > 0) dma_tile(src, tile_of(0), smem, smem + 2 * TILEB, wave, 4, lane);
  wait_all();
  __syncthreads();
  for (int ti = 0; ti < n_tiles; ++ti) {
    const int buf = ti & 1;
    if (ti + 1 < n_tiles)
      dma_tile(src, tile_of(ti + 1), smem + (buf ^ 1) * TILEB, smem + (2 + (buf ^ 1)) * TILEB,
               wave, 4, lane);
    const Tile tl = tile_of(ti);
    f32x4_t s[2][2];
    partial_scores(s, qf, smem + buf * TILEB, hf, lane);
    xs_write(xs, wave, lane, s);
    __syncthreads();
    xs_add(xs, wave ^ 1, lane, s);
    softmax_pv(st, s, smem + (2 + buf) * TILEB, tl, rv, scale_log2, hf, lane);
    wait_all();
    __syncthreads();
  }
  float lt[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) lt[nb] = wave_sum16(st.l[nb]);
  if (n_split == 1) {
    uint16_t* out = (uint16_t*)p.out + (size_t)b * p.H * D;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float inv = final_scale(st.m[nb], lt[nb]);
      uint16_t* orow = out + (size_t)(h0 + 16 * nb + l16) * D + hf * HALF;
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) store4(orow + 16 * cb + 4 * g, st.o[cb][nb] * inv);
    }
    return;
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int hh = h0 + 16 * nb + l16;
    const size_t pr = ((size_t)b * n_split + sp) * p.H + hh;
    float* po = part_o + pr * D + hf * HALF;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) *(f32x4_t*)(po + 16 * cb + 4 * g) = st.o[cb][nb];
    if (g == 0 && hf == 0) {
      part_ml[pr * 2 + 0] = st.m[nb];
      part_ml[pr * 2 + 1] = lt[nb];
    }
  }
}

__global__ __launch_bounds__(128) void hca_combine2_kernel(const float* __restrict__ part_o,
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
    const float ms = part_ml[pr * 2];
    const float a = fast_exp2(ms - mt);  // an empty split carries the sentinel max: a = 0
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

bool use_decode(const HcaParams& p) { return p.Tq == 1 && p.H % 64 == 0; }

// token groups per prefill workgroup: 4 (128 rows of one head) or 2 (64 rows x 2 heads)
int prefill_tg(const HcaParams& p) {
  const char* e = getenv("LGSA_HCA_TG");  // tuning knob; both values are correct
  if (e && e[0] == '2' && p.H % 2 == 0) return 2;
  return 4;
}

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
  static bool attr_set = false;  // idempotent: racing threads set the same values
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)hca_prefill2_kernel<4>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)PF_SMEM);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)hca_prefill2_kernel<2>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)PF_SMEM);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)hca_decode2_kernel,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)DEC_SMEM);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  if (use_decode(p)) {
    int n_split, chunk;
    decode_plan(p, n_split, chunk);
    float* part_o = (float*)p.ws;
    float* part_ml = part_o ? part_o + (size_t)p.B * n_split * p.H * D : nullptr;
    const long long grid = (long long)p.B * (p.H / 64) * n_split;
    hipLaunchKernelGGL(hca_decode2_kernel, dim3((unsigned)grid), dim3(256), DEC_SMEM, stream, p,
                       n_split, chunk, part_o, part_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (n_split > 1) {
      hipLaunchKernelGGL(hca_combine2_kernel, dim3(p.B * p.H), dim3(128), 0, stream, part_o,
                         part_ml, (uint16_t*)p.out, p.H, n_split);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (p.q_lat != nullptr)
      return launch_gate(p.q_lat, p.w_gate, p.out, p.out, p.B, p.d_lat, p.H * D, DT_BF16,
                         stream);
    return hipSuccess;
  }
  const int tg = prefill_tg(p);
  const int nh = 4 / tg;
  if (p.H % nh != 0) return hipErrorInvalidValue;
  const long long n_qt = (p.Tq + 32 * tg - 1) / (32 * tg);
  const long long grid = (long long)p.B * n_qt * (p.H / nh);
  if (tg == 4)
    hipLaunchKernelGGL(hca_prefill2_kernel<4>, dim3((unsigned)grid), dim3(512), PF_SMEM, stream,
                       p);
  else
    hipLaunchKernelGGL(hca_prefill2_kernel<2>, dim3((unsigned)grid), dim3(512), PF_SMEM, stream,
                       p);
  return hipGetLastError();
}

}  // namespace lgsa
