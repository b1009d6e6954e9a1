// Heavily Compressed Attention forward, bfloat16, 512-wide heads, for gfx950.
//
// ERNIE 5.5 Flash Base release blog, section 2.1 "Latent-Gated Sparse Attention": each HCA
// layer keeps one cache entry per 128 tokens and attends densely to all completed entries
// plus a short window of recent raw tokens (128 tokens per the xenospectrum.com article on
// ERNIE 5.5 Flash Base, long-context section); HCA heads are 512 wide; all layers multiply
// the attention output by a gate computed from the low-rank query latent.
//
// Visibility is closed-form, so no mask tensor exists: query position t sees compressed
// entry e iff e < (t + 1) / block, and raw position s iff t - window + 1 <= s <= t.
//
// Formulation.  All H query heads share one key/value head.  Every product is computed
// transposed, S^T = K Q^T and O^T = V^T P^T, on v_mfma_f32_16x16x32_bf16: the key (or V^T)
// tile staged in LDS is the A operand, the query rows held in registers are the B operand.
// A lane then owns one query row (lane % 16) for all of its accumulators, so row max / sum
// need only two cross-lane shuffles, and the P fragment of the second product is exactly the
// S^T accumulator of the first (keys are relabelled so that no data moves between lanes).
//
// Prefill kernel: one workgroup per (sequence, 128 query rows, head); four waves of 32 rows.
// Keys stream in tiles of 32 (compressed entries first, then the raw window), double
// buffered in LDS; a wave skips tiles that none of its rows can see.  After the key loop the
// gate logits q_lat . W for the 128 rows x 512 channels of the head are computed with the
// same MFMA scheme and multiplied into O before the only store (the logits never reach HBM).
//
// Decode kernel (one query row per sequence): one workgroup per (sequence, key split); the
// 64 heads are the MFMA rows (two waves of 32), two more waves take every other key tile,
// the halves merge through LDS, and partial (max, sum, O) go to the workspace when a
// sequence is split.  A combine kernel merges splits; the gate GEMM then runs in place.
#include "common.h"
#include "kernels.h"

namespace lgsa {

namespace {

constexpr int D = 512;            // head dim
constexpr int KT = 32;            // keys per tile
constexpr int KS_LD = D + 8;      // LDS row of a key tile (bf16): 1040 bytes
constexpr int VT_LD = KT + 8;     // LDS row of a transposed value tile (bf16): 80 bytes
constexpr int KS_ELEMS = KT * KS_LD;
constexpr int VT_ELEMS = D * VT_LD;
constexpr float LOG2E = 1.4426950408889634f;

// Key relabelling.  The S^T accumulator of a 32-key tile gives lane group g (= lane / 16)
// keys 4g..4g+3 (first 16-key block) and 16+4g..16+4g+3 (second block).  For the PV product
// those eight keys must be the lane's eight contraction slots 8g..8g+7, so slot p of a
// transposed value row holds key kappa(p):
__device__ __forceinline__ int slot_key(int p) {
  const int g = p >> 3, j = p & 7;
  return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
}

// One tile of keys: `count` (<= 32) rows starting at compressed entry `start` (kind 0) or
// at raw position `start` (kind 1, row = position % win_len).
struct Tile {
  int kind, start, count;
};

struct KeySrc {
  const uint16_t* kc;  // compressed rows of this sequence
  const uint16_t* vc;
  const uint16_t* kw;  // raw window rows of this sequence
  const uint16_t* vw;
  int win_len;
  __device__ __forceinline__ size_t row(const Tile& t, int j) const {
    return t.kind == 0 ? (size_t)(t.start + j) : (size_t)((t.start + j) % win_len);
  }
  __device__ __forceinline__ const uint16_t* krow(const Tile& t, int j) const {
    return (t.kind == 0 ? kc : kw) + row(t, j) * D;
  }
  __device__ __forceinline__ const uint16_t* vrow(const Tile& t, int j) const {
    return (t.kind == 0 ? vc : vw) + row(t, j) * D;
  }
};

// Register staging of one tile by 256 threads: 8 chunks of K (rows wave + 4p, one 16-byte
// column chunk per lane) and an 8x8 block of V (keys of slot group tid % 4, columns
// 8 * (tid / 4) ..).  Rows past `count` load as zeros.
struct TileRegs {
  uint4 k[8];
  uint4 v[8];
};

__device__ __forceinline__ void load_tile(const KeySrc& src, const Tile& t, int tid,
                                          TileRegs& r) {
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int j = wave + 4 * p;
    r.k[p] = j < t.count ? *(const uint4*)(src.krow(t, j) + 8 * lane) : make_uint4(0, 0, 0, 0);
  }
  const int kg = tid & 3, cg = tid >> 2;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int key = slot_key(8 * kg + j);
    r.v[j] = key < t.count ? *(const uint4*)(src.vrow(t, key) + 8 * cg) : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void store_tile(uint16_t* ks, uint16_t* vt, int tid,
                                           const TileRegs& r) {
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int p = 0; p < 8; ++p) *(uint4*)(ks + (wave + 4 * p) * KS_LD + 8 * lane) = r.k[p];
  const int kg = tid & 3, cg = tid >> 2;
  uint4 col[8];
  transpose8x8(r.v, col);
#pragma unroll
  for (int i = 0; i < 8; ++i) *(uint4*)(vt + (8 * cg + i) * VT_LD + 8 * kg) = col[i];
}

// Per-wave attention state for 32 query rows (two MFMA column blocks nb = 0, 1).
struct RowState {
  f32x4_t o[32][2];  // O^T accumulators: o[cb][nb][r] = O[row 16nb + l16][16cb + 4g + r]
  float m[2];        // running max (log2 domain, scaled)
  float l[2];        // running partial sum of this lane's keys
};

// Visibility of key j of tile t for a query at position tq (tq < 0: nothing visible).
__device__ __forceinline__ bool visible(const Tile& t, int j, int tq, int window, int block) {
  if (j >= t.count || tq < 0) return false;
  if (t.kind == 0) return t.start + j < (tq + 1) / block;
  const int s = t.start + j;
  return s <= tq && s >= tq - window + 1;
}

// One 32-key tile for one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
__device__ __forceinline__ void attend_tile(RowState& st, const Frag8 (&qf)[2][16],
                                            const uint16_t* ks, const uint16_t* vt,
                                            const Tile& t, const int (&trow)[2], int window,
                                            int block, float scale_log2, int lane) {
  const int l16 = lane & 15, g = lane >> 4;
  f32x4_t s[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) s[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks_ = 0; ks_ < D / 32; ++ks_) {
    Frag8 ka[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
      ka[mb].u = *(const uint4*)(ks + (16 * mb + l16) * KS_LD + 32 * ks_ + 8 * g);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) s[mb][nb] = mfma_16x16x32(ka[mb], qf[nb][ks_], s[mb][nb]);
  }
  // mask, scale, running max
  float alpha[2];
  Frag8 pf[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float x[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * mb + 4 * g + r;
        x[mb][r] = visible(t, j, trow[nb], window, block) ? s[mb][nb][r] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, x[mb][r]);
      }
    mx = wave_max16(mx);
    const float m_new = fmaxf(st.m[nb], mx);
    alpha[nb] = st.m[nb] == -INFINITY ? 0.f : fast_exp2(st.m[nb] - m_new);
    st.m[nb] = m_new;
    float psum = 0.f;
    float p[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[mb][r] = x[mb][r] == -INFINITY ? 0.f : fast_exp2(x[mb][r] - m_new);
        psum += p[mb][r];
      }
    st.l[nb] = st.l[nb] * alpha[nb] + psum;
    pf[nb].u = make_uint4(pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                          pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3]));
  }
  // rescale only when some row's max moved (the common case after the first tiles is not)
  const bool rescale = __any((alpha[0] != 1.f) | (alpha[1] != 1.f));
  if (rescale) {
#pragma unroll
    for (int cb = 0; cb < 32; ++cb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) st.o[cb][nb] *= alpha[nb];
  }
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) {
    Frag8 va;
    va.u = *(const uint4*)(vt + (16 * cb + l16) * VT_LD + 8 * g);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) st.o[cb][nb] = mfma_16x16x32(va, pf[nb], st.o[cb][nb]);
  }
}

// Gate epilogue for 128 query rows x the 512 channels of head h, computed 128 channels at a
// time: G^T = W^T q_lat^T with W^T staged (transposed) and q_lat rows staged in LDS, K = d_lat
// in steps of 64; then out = O * sigmoid(G).  `rows` are the 128 flat query rows of the
// workgroup (row index into q_lat / out), `nrows_valid` of them exist.
constexpr int GK = 64, G_LD = GK + 8;

__device__ __forceinline__ void gate_stage_load(const uint16_t* w, const uint16_t* ql,
                                                int d_lat, int N, int ncol0, size_t row0,
                                                int nrows_valid, int k0, int tid,
                                                uint4 (&stage)[8]) {
  if (tid < 128) {
    const int kg = tid & 7, ng = tid >> 3;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      stage[j] = *(const uint4*)(w + (size_t)(k0 + 8 * kg + j) * N + ncol0 + 8 * ng);
  } else {
    const int t = tid - 128;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = t + 128 * j;
      const int r = c >> 3;
      stage[j] = r < nrows_valid ? *(const uint4*)(ql + (row0 + r) * d_lat + k0 + 8 * (c & 7))
                                 : make_uint4(0, 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void gate_stage_store(uint16_t* sw, uint16_t* sq, int tid,
                                                 const uint4 (&stage)[8]) {
  if (tid < 128) {
    const int kg = tid & 7, ng = tid >> 3;
    uint4 col[8];
    transpose8x8(stage, col);
#pragma unroll
    for (int i = 0; i < 8; ++i) *(uint4*)(sw + (8 * ng + i) * G_LD + 8 * kg) = col[i];
  } else {
    const int t = tid - 128;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = t + 128 * j;
      *(uint4*)(sq + (c >> 3) * G_LD + 8 * (c & 7)) = stage[j];
    }
  }
}

__device__ __forceinline__ void store_out4(uint16_t* dst, const f32x4_t& v) {
  uint2 r;
  r.x = pack_bf16x2(v[0], v[1]);
  r.y = pack_bf16x2(v[2], v[3]);
  *(uint2*)dst = r;
}

extern __shared__ __attribute__((aligned(16))) uint16_t hca_smem[];

__global__ __launch_bounds__(256, 1) void hca_prefill_kernel(HcaParams p) {
  auto ks_buf = [&](int i) { return hca_smem + i * KS_ELEMS; };
  auto vt_buf = [&](int i) { return hca_smem + 2 * KS_ELEMS + i * VT_ELEMS; };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int n_qt = (p.Tq + 127) / 128;
  // workgroup -> (sequence, query tile, head), heads fastest
  const int h = blockIdx.x % p.H;
  const int qt = (blockIdx.x / p.H) % n_qt;
  const int b = blockIdx.x / (p.H * n_qt);
  const int pos = p.pos0[b];
  const int i_first = qt * 128;
  const int i_end = min(p.Tq, i_first + 128);
  const int t_first = pos + i_first, t_last = pos + i_end - 1;

  // key stream of the workgroup
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
    } else {
      t.kind = 1;
      t.start = s_lo + KT * (ti - tiles_c);
      t.count = min(KT, t_last - t.start + 1);
    }
    return t;
  };
  KeySrc src;
  src.kc = (const uint16_t*)p.kc + (size_t)b * p.n_cap * D;
  src.vc = (const uint16_t*)p.vc + (size_t)b * p.n_cap * D;
  src.kw = (const uint16_t*)p.k_win + (size_t)b * p.win_len * D;
  src.vw = (const uint16_t*)p.v_win + (size_t)b * p.win_len * D;
  src.win_len = p.win_len;

  // this wave's rows and their positions
  const int wi0 = i_first + 32 * wave;
  int trow[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int i = wi0 + 16 * nb + l16;
    trow[nb] = i < i_end ? pos + i : -1;
  }
  const int wa = pos + wi0, wb = pos + min(i_end, wi0 + 32) - 1;  // wave's position range
  const bool wave_live = wi0 < i_end && wb >= 0;
  const int wave_ne = wave_live ? (wb + 1) / p.block : 0;

  // Q fragments: qf[nb][ks] = q[row 16nb + l16][32ks + 8g .. +7]
  Frag8 qf[2][16];
  const uint16_t* qbase = (const uint16_t*)p.q;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int i = wi0 + 16 * nb + l16;
    const uint16_t* qr = qbase + (((size_t)b * p.Tq + i) * p.H + h) * D;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      qf[nb][k].u = i < i_end ? *(const uint4*)(qr + 32 * k + 8 * g) : make_uint4(0, 0, 0, 0);
  }

  RowState st;
#pragma unroll
  for (int cb = 0; cb < 32; ++cb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) st.o[cb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  st.m[0] = st.m[1] = -INFINITY;
  st.l[0] = st.l[1] = 0.f;
  const float scale_log2 = p.scale * LOG2E;

  TileRegs regs;
  if (n_tiles > 0) {
    load_tile(src, tile_of(0), tid, regs);
    store_tile(ks_buf(0), vt_buf(0), tid, regs);
  }
  __syncthreads();
  for (int ti = 0; ti < n_tiles; ++ti) {
    const int buf = ti & 1;
    if (ti + 1 < n_tiles) load_tile(src, tile_of(ti + 1), tid, regs);
    const Tile t = tile_of(ti);
    bool relevant = wave_live;
    if (t.kind == 0)
      relevant = relevant && t.start < wave_ne;
    else
      relevant = relevant && t.start <= wb && t.start + t.count - 1 >= wa - p.window + 1;
    if (relevant)
      attend_tile(st, qf, ks_buf(buf), vt_buf(buf), t, trow, p.window, p.block, scale_log2,
                  lane);
    if (ti + 1 < n_tiles) store_tile(ks_buf(buf ^ 1), vt_buf(buf ^ 1), tid, regs);
    __syncthreads();
  }

  // normalise
  float inv[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float lt = wave_sum16(st.l[nb]);
    inv[nb] = lt > 0.f ? 1.f / lt : 0.f;
  }
#pragma unroll
  for (int cb = 0; cb < 32; ++cb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) st.o[cb][nb] *= inv[nb];

  uint16_t* out = (uint16_t*)p.out;
  const int HD = p.H * D;
  if (p.q_lat == nullptr) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int i = wi0 + 16 * nb + l16;
      if (i >= i_end) continue;
      uint16_t* orow = out + (((size_t)b * p.Tq + i) * p.H + h) * D;
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) store_out4(orow + 16 * cb + 4 * g, st.o[cb][nb]);
    }
    return;
  }

  // fused gate
  const uint16_t* w = (const uint16_t*)p.w_gate;
  const uint16_t* ql = (const uint16_t*)p.q_lat;
  const size_t row0 = (size_t)b * p.Tq + i_first;
  const int nvalid = i_end - i_first;
  auto sw = [&](int i) { return hca_smem + i * 128 * G_LD; };
  auto sq = [&](int i) { return hca_smem + (2 + i) * 128 * G_LD; };
  const int nk = p.d_lat / GK;
#pragma unroll 1
  for (int cc = 0; cc < 4; ++cc) {
    const int ncol0 = h * D + cc * 128;
    f32x4_t ga[8][2];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) ga[c][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint4 stage[8];
    gate_stage_load(w, ql, p.d_lat, HD, ncol0, row0, nvalid, 0, tid, stage);
    gate_stage_store(sw(0), sq(0), tid, stage);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk)
        gate_stage_load(w, ql, p.d_lat, HD, ncol0, row0, nvalid, (kt + 1) * GK, tid, stage);
#pragma unroll
      for (int ks_ = 0; ks_ < GK / 32; ++ks_) {
        Frag8 qa[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          qa[nb].u = *(const uint4*)(sq(buf) + (32 * wave + 16 * nb + l16) * G_LD + 32 * ks_ +
                                     8 * g);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          Frag8 wa_;
          wa_.u = *(const uint4*)(sw(buf) + (16 * c + l16) * G_LD + 32 * ks_ + 8 * g);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) ga[c][nb] = mfma_16x16x32(wa_, qa[nb], ga[c][nb]);
        }
      }
      if (kt + 1 < nk) gate_stage_store(sw(buf ^ 1), sq(buf ^ 1), tid, stage);
      __syncthreads();
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int i = wi0 + 16 * nb + l16;
      if (i >= i_end) continue;
      uint16_t* orow = out + (((size_t)b * p.Tq + i) * p.H + h) * D + cc * 128;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        f32x4_t v = st.o[cc * 8 + c][nb];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] *= sigmoidf_fast(ga[c][nb][r]);
        store_out4(orow + 16 * c + 4 * g, v);
      }
    }
  }
}

// ------------------------------------------------------------------------------- decode
// Workgroup (sequence b, key split sp): waves 0,1 take heads 0..31 / 32..63 of even tiles,
// waves 2,3 the same heads of odd tiles (each pair of tiles is staged together), then the
// two halves merge through LDS.  The key index space of a sequence is: compressed entries
// 0..ne-1, then raw positions s_lo..t.
constexpr int DEC_HEADS = 64;

__global__ __launch_bounds__(256, 1) void hca_decode_kernel(HcaParams p, int n_split,
                                                            int chunk, float* part_o,
                                                            float* part_ml) {
  auto ks_buf = [&](int i) { return hca_smem + i * KS_ELEMS; };
  auto vt_buf = [&](int i) { return hca_smem + 2 * KS_ELEMS + i * VT_ELEMS; };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int hg = blockIdx.x % (p.H / DEC_HEADS);
  const int sp = (blockIdx.x / (p.H / DEC_HEADS)) % n_split;
  const int b = blockIdx.x / ((p.H / DEC_HEADS) * n_split);
  const int t = p.pos0[b];  // Tq == 1
  const int ne = t >= 0 ? min(p.n_cap, (t + 1) / p.block) : 0;
  const int s_lo = max(0, t - p.window + 1);
  const int nw = t >= 0 ? t - s_lo + 1 : 0;
  const int nkeys = ne + nw;
  const int k_begin = sp * chunk, k_end = min(nkeys, k_begin + chunk);

  KeySrc src;
  src.kc = (const uint16_t*)p.kc + (size_t)b * p.n_cap * D;
  src.vc = (const uint16_t*)p.vc + (size_t)b * p.n_cap * D;
  src.kw = (const uint16_t*)p.k_win + (size_t)b * p.win_len * D;
  src.vw = (const uint16_t*)p.v_win + (size_t)b * p.win_len * D;
  src.win_len = p.win_len;

  // tiles never straddle the compressed/raw boundary: split [k_begin, k_end) at ne
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
    } else {
      tl.kind = 1;
      const int k0 = w_begin + KT * (ti - tiles_c);
      tl.start = s_lo + (k0 - ne);
      tl.count = min(KT, k_end - k0);
    }
    return tl;
  };

  const int half = wave >> 1;                      // which tile of a pair
  const int h0 = hg * DEC_HEADS + 32 * (wave & 1);  // first head of this wave
  int trow[2] = {t, t};
  Frag8 qf[2][16];
  const uint16_t* qbase = (const uint16_t*)p.q + (size_t)b * p.H * D;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const uint16_t* qr = qbase + (size_t)(h0 + 16 * nb + l16) * D;
#pragma unroll
    for (int k = 0; k < 16; ++k) qf[nb][k].u = *(const uint4*)(qr + 32 * k + 8 * g);
  }
  RowState st;
#pragma unroll
  for (int cb = 0; cb < 32; ++cb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) st.o[cb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  st.m[0] = st.m[1] = -INFINITY;
  st.l[0] = st.l[1] = 0.f;
  const float scale_log2 = p.scale * LOG2E;

  TileRegs regs;
  for (int tp = 0; tp < n_tiles; tp += 2) {
    // stage the pair (tp, tp+1) into buffers 0 and 1
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (tp + u < n_tiles) {
        load_tile(src, tile_of(tp + u), tid, regs);
        store_tile(ks_buf(u), vt_buf(u), tid, regs);
      }
    }
    __syncthreads();
    if (tp + half < n_tiles)
      attend_tile(st, qf, ks_buf(half), vt_buf(half), tile_of(tp + half), trow, p.window,
                  p.block, scale_log2, lane);
    __syncthreads();
  }

  // merge the two halves: waves 2,3 publish (m, l, O) and waves 0,1 fold them in
  float* xo = (float*)hca_smem;                       // [2 waves][32 cb][2 nb][64 lanes][4]
  float* xml = (float*)hca_smem + 2 * 32 * 2 * 64 * 4;  // [2 waves][2][2][64]
  float lsum[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) lsum[nb] = wave_sum16(st.l[nb]);
  if (half == 1) {
    const int wv = wave & 1;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        *(f32x4_t*)(xo + (((wv * 32 + cb) * 2 + nb) * 64 + lane) * 4) = st.o[cb][nb];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      xml[((wv * 2 + nb) * 2 + 0) * 64 + lane] = st.m[nb];
      xml[((wv * 2 + nb) * 2 + 1) * 64 + lane] = lsum[nb];
    }
  }
  __syncthreads();
  if (half == 1) return;
  const int wv = wave & 1;
  float a_self[2], a_other[2], m_tot[2], l_tot[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float mo = xml[((wv * 2 + nb) * 2 + 0) * 64 + lane];
    const float lo = xml[((wv * 2 + nb) * 2 + 1) * 64 + lane];
    const float mt = fmaxf(st.m[nb], mo);
    a_self[nb] = st.m[nb] == -INFINITY ? 0.f : fast_exp2(st.m[nb] - mt);
    a_other[nb] = mo == -INFINITY ? 0.f : fast_exp2(mo - mt);
    m_tot[nb] = mt;
    l_tot[nb] = lsum[nb] * a_self[nb] + lo * a_other[nb];
  }
#pragma unroll
  for (int cb = 0; cb < 32; ++cb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const f32x4_t other = *(const f32x4_t*)(xo + (((wv * 32 + cb) * 2 + nb) * 64 + lane) * 4);
      st.o[cb][nb] = st.o[cb][nb] * a_self[nb] + other * a_other[nb];
    }

  if (n_split == 1) {
    // final: normalise and store O (the gate, if any, runs afterwards in place)
    uint16_t* out = (uint16_t*)p.out + (size_t)b * p.H * D;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float inv = l_tot[nb] > 0.f ? 1.f / l_tot[nb] : 0.f;
      uint16_t* orow = out + (size_t)(h0 + 16 * nb + l16) * D;
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) store_out4(orow + 16 * cb + 4 * g, st.o[cb][nb] * inv);
    }
    return;
  }
  // partial: unnormalised O, running max (log2 domain) and sum, per (b, split, head)
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int hh = h0 + 16 * nb + l16;
    const size_t pr = ((size_t)b * n_split + sp) * p.H + hh;
    float* po = part_o + pr * D;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) *(f32x4_t*)(po + 16 * cb + 4 * g) = st.o[cb][nb];
    if (g == 0) {
      part_ml[pr * 2 + 0] = m_tot[nb];
      part_ml[pr * 2 + 1] = l_tot[nb];
    }
  }
}

// Merge of the key splits of one (sequence, head): O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
__global__ __launch_bounds__(128) void hca_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          uint16_t* __restrict__ out, int H,
                                                          int n_split) {
  const int bh = blockIdx.x;  // b * H + h
  const int b = bh / H, h = bh % H;
  float mt = -INFINITY;
  for (int s = 0; s < n_split; ++s)
    mt = fmaxf(mt, part_ml[(((size_t)b * n_split + s) * H + h) * 2]);
  float lt = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < n_split; ++s) {
    const size_t pr = ((size_t)b * n_split + s) * H + h;
    const float ms = part_ml[pr * 2];
    const float a = ms == -INFINITY ? 0.f : fast_exp2(ms - mt);
    lt += a * part_ml[pr * 2 + 1];
    const float4 v = *(const float4*)(part_o + pr * D + 4 * threadIdx.x);
    acc[0] += a * v.x;
    acc[1] += a * v.y;
    acc[2] += a * v.z;
    acc[3] += a * v.w;
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  uint2 r;
  r.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  r.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *(uint2*)(out + (size_t)bh * D + 4 * threadIdx.x) = r;
}

constexpr size_t SMEM_BYTES = (size_t)(2 * KS_ELEMS + 2 * VT_ELEMS) * 2;

// decode split plan: enough workgroups to cover the chip, chunks a multiple of two tiles
void decode_plan(const HcaParams& p, int& n_split, int& chunk) {
  const long long mp = p.max_pos;
  const long long ne = std::min<long long>(p.n_cap, (mp + 1) / p.block);
  const long long nk = ne + std::min<long long>(p.window, mp + 1);
  const long long groups = (long long)p.B * (p.H / DEC_HEADS);
  long long want = (512 + groups - 1) / groups;  // target >= 512 workgroups
  const long long max_split = (nk + 2 * KT - 1) / (2 * KT);
  n_split = (int)std::max<long long>(1, std::min(want, max_split));
  long long c = (nk + n_split - 1) / n_split;
  c = (c + 2 * KT - 1) / (2 * KT) * (2 * KT);
  chunk = (int)std::max<long long>(c, 2 * KT);
  n_split = (int)std::max<long long>(1, (nk + chunk - 1) / chunk);
}

}  // namespace

// one query row per sequence and whole groups of 64 heads: the decode kernel; otherwise the
// prefill kernel (correct for any shape)
bool use_decode(const HcaParams& p) { return p.Tq == 1 && p.H % DEC_HEADS == 0; }

size_t hca_bf16_workspace(const HcaParams& p) {
  if (!use_decode(p)) return 0;
  int n_split, chunk;
  decode_plan(p, n_split, chunk);
  if (n_split == 1) return 0;
  const size_t rows = (size_t)p.B * n_split * p.H;
  return rows * D * sizeof(float) + rows * 2 * sizeof(float);
}

hipError_t launch_hca_bf16(const HcaParams& p, hipStream_t stream) {
  static bool attr_set = false;  // idempotent; racing threads set the same value
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)hca_prefill_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)SMEM_BYTES);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)hca_decode_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)SMEM_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  if (use_decode(p)) {
    int n_split, chunk;
    decode_plan(p, n_split, chunk);
    float* part_o = (float*)p.ws;
    float* part_ml = part_o + (size_t)p.B * n_split * p.H * D;
    const int grid = p.B * (p.H / DEC_HEADS) * n_split;
    hipLaunchKernelGGL(hca_decode_kernel, dim3(grid), dim3(256), SMEM_BYTES, stream, p,
                       n_split, chunk, part_o, part_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (n_split > 1) {
      hipLaunchKernelGGL(hca_combine_kernel, dim3(p.B * p.H), dim3(128), 0, stream, part_o,
                         part_ml, (uint16_t*)p.out, p.H, n_split);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (p.q_lat != nullptr)
      return launch_gate(p.q_lat, p.w_gate, p.out, p.out, p.B, p.d_lat, p.H * D, DT_BF16,
                         stream);
    return hipSuccess;
  }
  const int n_qt = (p.Tq + 127) / 128;
  const long long grid = (long long)p.B * n_qt * p.H;
  hipLaunchKernelGGL(hca_prefill_kernel, dim3((unsigned)grid), dim3(256), SMEM_BYTES, stream, p);
  return hipGetLastError();
}

}  // namespace lgsa
