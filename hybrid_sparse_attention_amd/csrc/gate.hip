// Low-rank output gate (ERNIE 5.5 Flash Base release blog, section 2.1, low-rank gated
// attention): out[m, n] = o[m, n] * sigmoid(q_lat[m, :] . w[:, n]), the gate logits computed
// from the 1024-wide query latent and never written to memory.
//
// bfloat16 paths: MFMA GEMMs computing the transposed product G^T = W^T q_lat^T, so that a
// lane's accumulator holds four consecutive output channels of one row.
//   - gate_bf16_big_kernel (M and N >= 256, the prefill shapes): 256 x 256 tiles fed by LDS
//     DMA, W read through the transposing LDS read, tiles ordered so that the workgroups
//     resident on one XCD share their q_lat and W tiles in that XCD's L2; the epilogue stages
//     the fp32 gate factors in LDS and streams o and out with 16-byte non-temporal accesses,
//     which pass through L2 without displacing those shared tiles.
//   - gate_bf16_kernel (small M or N, e.g. decode): 128 x 128 tiles, the W tile transposed
//     while it is staged in LDS through registers, four waves of 64 x 64, K staged 64 at a
//     time in double-buffered LDS; the lane multiplies its four channels into o and stores
//     8 bytes.
//   - gate_bf16_skinny_kernel (M <= 64 rows, d_lat = 1024: decode): the stream over W of
//     gate_skinny.h, one workgroup per 64 channels.
//
// float32 path: a plain tiled FMA GEMM (used for the small fp32 configuration).
//
// With o == NULL the bfloat16 kernels write the gate factors sigmoid(q_lat W) themselves (the
// attention kernels that apply the gate in their own epilogue read them from there).
#include "common.h"
#include "gate_skinny.h"
#include "kernels.h"

namespace lgsa {

namespace {

constexpr int GT_N = 128, GT_M = 128, GT_K = 64, GT_LD = GT_K + 8;  // LDS row: 72 bf16
// two bfloat16 ones: the factor o takes when the gate alone is asked for (o == NULL)
constexpr uint32_t BF16_ONES = 0x3F803F80u;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte global accesses with the non-temporal cache policy: a stream touched once (o and
// out, 4 bytes per output element) then goes through L2 without evicting the operand tiles
// that the workgroups of an XCD share.
__device__ __forceinline__ uint4 load16_nt(const void* p) {
  const u32x4_t t = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void store16_nt(void* p, uint4 v) {
  const u32x4_t t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, (u32x4_t*)p);
}

// BWD: the backward's first step on the same recomputed G: with s = sigmoid(G), out receives
// dout * s (the gradient of o) and dg receives dout * o * s * (1 - s) (the gradient of G).
template <bool BWD>
__global__ __launch_bounds__(256) void gate_bf16_kernel(const uint16_t* __restrict__ ql,
                                                        const uint16_t* __restrict__ w,
                                                        const uint16_t* o, uint16_t* out,
                                                        int M, int d_lat, int N,
                                                        const uint16_t* dout, uint16_t* dg) {
  __shared__ __attribute__((aligned(16))) uint16_t sW[2][GT_N * GT_LD];
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2][GT_M * GT_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_tiles_n = (N + GT_N - 1) / GT_N;
  const int n0 = (blockIdx.x % n_tiles_n) * GT_N;
  const int m0 = (blockIdx.x / n_tiles_n) * GT_M;
  const int wn = (wave & 1) * 64, wm = (wave >> 1) * 64;
  const int l16 = lane & 15, g = lane >> 4;

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // staging: threads 0..127 transpose one 8x8 block of W each, threads 128..255 copy 8
  // 16-byte chunks of q_lat each.
  uint4 stage[8];
  auto load_stage = [&](int k0) {
    if (tid < 128) {
      const int kg = tid & 7, ng = tid >> 3;  // k rows 8kg.., channels 8ng..
      const int n = n0 + 8 * ng;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        stage[j] = (n < N) ? *(const uint4*)(w + (size_t)(k0 + 8 * kg + j) * N + n)
                           : make_uint4(0, 0, 0, 0);
    } else {
      const int t = tid - 128;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = t + 128 * j;  // 1024 chunks: row c/8, k chunk c%8
        const int m = m0 + (c >> 3);
        stage[j] = (m < M) ? *(const uint4*)(ql + (size_t)m * d_lat + k0 + 8 * (c & 7))
                           : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_stage = [&](int buf) {
    if (tid < 128) {
      const int kg = tid & 7, ng = tid >> 3;
      uint4 col[8];
      transpose8x8(stage, col);
#pragma unroll
      for (int i = 0; i < 8; ++i) *(uint4*)(&sW[buf][(8 * ng + i) * GT_LD + 8 * kg]) = col[i];
    } else {
      const int t = tid - 128;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = t + 128 * j;
        *(uint4*)(&sQ[buf][(c >> 3) * GT_LD + 8 * (c & 7)]) = stage[j];
      }
    }
  };

  const int nk = d_lat / GT_K;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_stage((kt + 1) * GT_K);
#pragma unroll
    for (int ks = 0; ks < GT_K / 32; ++ks) {
      Frag8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i].u = *(const uint4*)(&sW[buf][(wn + 16 * i + l16) * GT_LD + 32 * ks + 8 * g]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j].u = *(const uint4*)(&sQ[buf][(wm + 16 * j + l16) * GT_LD + 32 * ks + 8 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) store_stage(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds G[m = m0+wm+16j+l16][n = n0+wn+16i+4g .. +3]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wm + 16 * j + l16;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + wn + 16 * i + 4 * g;
      if (n >= N) continue;
      const size_t off = (size_t)m * N + n;
      const uint2 ov = o != nullptr ? *(const uint2*)(o + off) : make_uint2(BF16_ONES, BF16_ONES);
      const float o0 = __uint_as_float(ov.x << 16), o1 = __uint_as_float(ov.x & 0xFFFF0000u);
      const float o2 = __uint_as_float(ov.y << 16), o3 = __uint_as_float(ov.y & 0xFFFF0000u);
      if constexpr (BWD) {
        const uint2 dv = *(const uint2*)(dout + off);
        const float d[4] = {__uint_as_float(dv.x << 16), __uint_as_float(dv.x & 0xFFFF0000u),
                            __uint_as_float(dv.y << 16), __uint_as_float(dv.y & 0xFFFF0000u)};
        const float ox[4] = {o0, o1, o2, o3};
        float s4[4], g4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s4[r] = sigmoidf_fast(acc[i][j][r]);
          g4[r] = d[r] * ox[r] * s4[r] * (1.f - s4[r]);
          s4[r] *= d[r];
        }
        *(uint2*)(out + off) = make_uint2(pack_bf16x2(s4[0], s4[1]), pack_bf16x2(s4[2], s4[3]));
        *(uint2*)(dg + off) = make_uint2(pack_bf16x2(g4[0], g4[1]), pack_bf16x2(g4[2], g4[3]));
        continue;
      }
      uint2 r;
      r.x = pack_bf16x2(o0 * sigmoidf_fast(acc[i][j][0]), o1 * sigmoidf_fast(acc[i][j][1]));
      r.y = pack_bf16x2(o2 * sigmoidf_fast(acc[i][j][2]), o3 * sigmoidf_fast(acc[i][j][3]));
      *(uint2*)(out + off) = r;
    }
  }
}

// Large-M bfloat16 path: 256 channels x 256 rows per workgroup, 8 waves of 128 x 64, K in
// steps of 64.  Both operand tiles reach LDS by LDS DMA (no register staging), two stages
// deep.  W rows (256 channels = 512 bytes) keep W row-major in LDS and the MFMA operand W^T
// is read with the transposing LDS read; q_lat rows (64 k = 128 bytes) are read as 16-byte
// fragments.  Bank conflicts are removed by XOR swizzles of 16-byte chunks, applied by
// permuting which chunk each lane fetches; the swizzle bits a lane needs are constant per lane,
// so fragment addresses are lane constants plus immediates.
constexpr int G2_BN = 256, G2_BM = 256, G2_BK = 64;
constexpr int G2_WROW = G2_BN * 2;              // bytes per staged W row
constexpr int G2_QROW = G2_BK * 2;              // bytes per staged q_lat row
constexpr int G2_WSTAGE = G2_BK * G2_WROW;      // 32 KiB
constexpr int G2_QSTAGE = G2_BM * G2_QROW;      // 32 KiB
constexpr int G2_STAGE = G2_WSTAGE + G2_QSTAGE;

__device__ __forceinline__ int g2_wswz(int k) { return 2 * (k & 3) + 8 * ((k >> 3) & 1); }
__device__ __forceinline__ int g2_qswz(int r) { return (r >> 1) & 7; }

// The two stages are separate LDS objects, each named directly wherever it is read or filled
// (the K loop is unrolled by two).  The compiler then sees that the fragment reads of one stage
// cannot touch the LDS DMA writes into the other and does not wait for that DMA before reading;
// with one shared array it would, and the prefetch would not overlap the products at all.
__shared__ __attribute__((aligned(1024))) char g2_stage0[G2_STAGE];
__shared__ __attribute__((aligned(1024))) char g2_stage1[G2_STAGE];

// BWD: the backward's elementwise part instead of the gate: out = dout * s and
// dg = dout * o * s * (1 - s), s = sigmoid(G).
template <bool BWD>
__global__ __launch_bounds__(512, 1) void gate_bf16_big_kernel(const uint16_t* __restrict__ ql,
                                                               const uint16_t* __restrict__ w,
                                                               const uint16_t* o, uint16_t* out,
                                                               int M, int d_lat, int N,
                                                               const uint16_t* dout,
                                                               uint16_t* dg) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int wn = wave & 1, wm = wave >> 1;
  // XCD-aware tile order: XCD x (= id % 8) takes a contiguous run of tiles.  Within the run,
  // tiles are visited in groups of 4 channel tiles x 8 row tiles, so the ~32 workgroups an
  // XCD runs at once share 4 W slices and 8 q_lat slices, which stay in its L2.
  const int n_nt = (N + G2_BN - 1) / G2_BN, n_mt = (M + G2_BM - 1) / G2_BM;
  const int tiles = n_nt * n_mt;
  int lin = blockIdx.x;
  if (tiles % 8 == 0) lin = (blockIdx.x % 8) * (tiles / 8) + blockIdx.x / 8;
  int nt, mt;
  if (n_nt % 4 == 0 && n_mt % 8 == 0) {
    const int grp = lin / 32, in = lin % 32;
    const int groups_m = n_mt / 8;
    nt = (grp / groups_m) * 4 + in / 8;
    mt = (grp % groups_m) * 8 + in % 8;
  } else {
    nt = lin / n_mt;
    mt = lin % n_mt;
  }
  const int n0 = nt * G2_BN, m0 = mt * G2_BM;

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // DMA of one K step into stage s: 32 W instructions (2 k-rows each) and 32 q_lat
  // instructions (8 rows each); 8 per wave.
  auto dma = [&](int k0, char* sw) {
    char* sq = sw + G2_WSTAGE;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ins = wave + 8 * u;                  // 0..31
      const int kr = 2 * ins + (lane >> 5);          // k-row of this lane
      const int chunk = (lane & 31) ^ g2_wswz(kr);   // 16-byte chunk it fetches
      const int n = min(n0 + 8 * chunk, N - 8);      // columns past N repeat the last chunk
      lds_dma16(w + (size_t)(k0 + kr) * N + n, sw + 2 * ins * G2_WROW);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ins = wave + 8 * u;                  // 0..31
      const int r = 8 * ins + (lane >> 3);           // row of this lane
      const int chunk = (lane & 7) ^ g2_qswz(r);
      const int m = min(m0 + r, M - 1);              // rows past M repeat the last row
      lds_dma16(ql + (size_t)m * d_lat + k0 + 8 * chunk, sq + 8 * ins * G2_QROW);
    }
  };

  // lane-constant fragment offsets
  const int a = l16 >> 2, c4 = l16 & 3;
  const int wf = g2_wswz(8 * g + a);                 // same for k-rows 32ks + 8g + 4h + a
  int wcol[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    wcol[i] = 16 * ((16 * wn + 2 * i + (c4 >> 1)) ^ wf) + 8 * (c4 & 1);
  const int qf = g2_qswz(l16);
  const int qrow = (64 * wm + l16) * G2_QROW;
  const int qc0 = 16 * ((g) ^ qf), qc1 = 16 * ((4 + g) ^ qf);

  const int nk = d_lat / G2_BK;
  // one K step on stage `cur` while the next step's tiles stream into `nxt`
  auto step = [&](int kt, const char* cur, char* nxt) {
    if (kt + 1 < nk) dma((kt + 1) * G2_BK, nxt);
    const char* sw = cur;
    const char* sq = cur + G2_WSTAGE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      Frag8 bq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bq[j].u = *(const uint4*)(sq + qrow + 16 * j * G2_QROW + (ks ? qc1 : qc0));
      const char* wr = sw + (32 * ks + 8 * g + a) * G2_WROW;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        Frag8 aw;
        const uint2 lo = lds_read_tr16(wr + wcol[i]);
        const uint2 hi = lds_read_tr16(wr + wcol[i] + 4 * G2_WROW);
        aw.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32(aw, bq[j], acc[i][j]);
      }
    }
    wait_all();
    __syncthreads();
  };
  dma(0, g2_stage0);
  wait_all();
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, g2_stage0, g2_stage1);
    if (kt + 1 < nk) step(kt + 1, g2_stage1, g2_stage0);
  }
  // epilogue: lane holds G[m = m0 + 64wm + 16j + l16][n = n0 + 128wn + 16i + 4g .. +3].
  // In two halves (waves 0-3, then 4-7), the owners write their gate factors sigmoid(G) as
  // fp32 rows [m][n] to LDS (16-byte chunk c of row r at chunk c ^ (r & 15), conflict free),
  // then all 8 waves stream that half of the tile: 16 bytes of o per lane along the rows and
  // 16-byte stores of whole rows.
  // [4 blocks][64 rows][128] fp32 = 128 KiB: blocks 0, 1 in stage 0, blocks 2, 3 in stage 1
  auto fblk = [&](int blk) {
    return (float*)(blk < 2 ? g2_stage0 : g2_stage1) + (blk & 1) * 64 * 128;
  };
  // chunk u of half hl for this thread: 4 blocks x 64 rows x 16 chunks of 8 channels per half
  auto chunk_mn = [&](int hl, int u, int& blk, int& rr, int& m, int& n) {
    const int c = tid + 512 * u;
    blk = c >> 10;
    rr = (c >> 4) & 63;
    m = m0 + 64 * (2 * hl + (blk >> 1)) + rr;
    n = n0 + 128 * (blk & 1) + (c & 15) * 8;
  };
  if constexpr (BWD) {
    // o and dout of one half at a time (the accumulators are still live in the first half);
    // the second half's loads go out once the first half's values are consumed
    uint4 ov[8], dv[8];
    auto load_half = [&](int hl) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        int blk, rr, m, n;
        chunk_mn(hl, u, blk, rr, m, n);
        const size_t off = (size_t)min(m, M - 1) * N + min(n, N - 8);
        ov[u] = load16_nt(o + off);
        dv[u] = load16_nt(dout + off);
      }
    };
    load_half(0);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if ((wave >> 2) == half) {
        float* fw = fblk(wave & 3);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            f32x4_t f;
#pragma unroll
            for (int r = 0; r < 4; ++r) f[r] = sigmoidf_fast(acc[i][j][r]);
            *(f32x4_t*)(fw + (16 * j + l16) * 128 + 4 * ((4 * i + g) ^ l16)) = f;
          }
      }
      lds_barrier();
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        int blk, rr, m, n;
        chunk_mn(half, u, blk, rr, m, n);
        const int c0 = (tid & 15) * 2;
        const float* fw = fblk(blk) + rr * 128;
        const f32x4_t f0 = *(const f32x4_t*)(fw + 4 * (c0 ^ (rr & 15)));
        const f32x4_t f1 = *(const f32x4_t*)(fw + 4 * ((c0 + 1) ^ (rr & 15)));
        const float sg[8] = {f0[0], f0[1], f0[2], f0[3], f1[0], f1[1], f1[2], f1[3]};
        const uint32_t xo[4] = {ov[u].x, ov[u].y, ov[u].z, ov[u].w};
        const uint32_t xd[4] = {dv[u].x, dv[u].y, dv[u].z, dv[u].w};
        uint32_t ro[4], rg[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float o0 = __uint_as_float(xo[c] << 16), o1 = __uint_as_float(xo[c] & 0xFFFF0000u);
          const float d0 = __uint_as_float(xd[c] << 16), d1 = __uint_as_float(xd[c] & 0xFFFF0000u);
          const float s0 = sg[2 * c], s1 = sg[2 * c + 1];
          ro[c] = pack_bf16x2(d0 * s0, d1 * s1);
          rg[c] = pack_bf16x2(d0 * o0 * s0 * (1.f - s0), d1 * o1 * s1 * (1.f - s1));
        }
        if (m < M && n < N) {
          store16_nt(out + (size_t)m * N + n, make_uint4(ro[0], ro[1], ro[2], ro[3]));
          store16_nt(dg + (size_t)m * N + n, make_uint4(rg[0], rg[1], rg[2], rg[3]));
        }
      }
      if (half == 0) load_half(1);
      lds_barrier();
    }
    return;
  }
  // the o loads of both halves are issued before any gate factor is staged, so the second
  // half's loads are in flight while the first half is processed
  uint4 ov[2][8];
#pragma unroll
  for (int hl = 0; hl < 2; ++hl)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      int blk, rr, m, n;
      chunk_mn(hl, u, blk, rr, m, n);
      ov[hl][u] = o != nullptr ? load16_nt(o + (size_t)min(m, M - 1) * N + min(n, N - 8))
                               : make_uint4(BF16_ONES, BF16_ONES, BF16_ONES, BF16_ONES);
    }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if ((wave >> 2) == half) {
      float* fw = fblk(wave & 3);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          f32x4_t f;
#pragma unroll
          for (int r = 0; r < 4; ++r) f[r] = sigmoidf_fast(acc[i][j][r]);
          *(f32x4_t*)(fw + (16 * j + l16) * 128 + 4 * ((4 * i + g) ^ l16)) = f;
        }
    }
    lds_barrier();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      int blk, rr, m, n;
      chunk_mn(half, u, blk, rr, m, n);
      const int c0 = (tid & 15) * 2;
      const float* fw = fblk(blk) + rr * 128;
      const f32x4_t f0 = *(const f32x4_t*)(fw + 4 * (c0 ^ (rr & 15)));
      const f32x4_t f1 = *(const f32x4_t*)(fw + 4 * ((c0 + 1) ^ (rr & 15)));
      const uint4 x = ov[half][u];
      uint4 r;
      r.x = pack_bf16x2(__uint_as_float(x.x << 16) * f0[0],
                        __uint_as_float(x.x & 0xFFFF0000u) * f0[1]);
      r.y = pack_bf16x2(__uint_as_float(x.y << 16) * f0[2],
                        __uint_as_float(x.y & 0xFFFF0000u) * f0[3]);
      r.z = pack_bf16x2(__uint_as_float(x.z << 16) * f1[0],
                        __uint_as_float(x.z & 0xFFFF0000u) * f1[1]);
      r.w = pack_bf16x2(__uint_as_float(x.w << 16) * f1[2],
                        __uint_as_float(x.w & 0xFFFF0000u) * f1[3]);
      if (m < M && n < N) store16_nt(out + (size_t)m * N + n, r);
    }
    lds_barrier();
  }
}

// Few-row bfloat16 path (M <= 64 and d_lat = 1024, decode): the tile of gate_skinny.h, one
// workgroup per 64 channels, its four stages in four LDS objects of its own.
__shared__ __attribute__((aligned(1024))) char sk_st0[gate_skinny::STAGE];
__shared__ __attribute__((aligned(1024))) char sk_st1[gate_skinny::STAGE];
__shared__ __attribute__((aligned(1024))) char sk_st2[gate_skinny::STAGE];
__shared__ __attribute__((aligned(1024))) char sk_st3[gate_skinny::STAGE];

// o of the lane's four 4-channel groups, loaded before the K loop (ones when o is NULL)
struct OLoad {
  const uint16_t* o;
  int N;
  uint2 x[4];
  __device__ __forceinline__ void fetch(int m, int n) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
      x[cb] = o != nullptr ? *(const uint2*)(o + (size_t)m * N + min(n + 16 * cb, N - 4))
                           : make_uint2(BF16_ONES, BF16_ONES);
  }
  __device__ __forceinline__ float4 value(int cb) const {
    return make_float4(__uint_as_float(x[cb].x << 16), __uint_as_float(x[cb].x & 0xFFFF0000u),
                       __uint_as_float(x[cb].y << 16), __uint_as_float(x[cb].y & 0xFFFF0000u));
  }
};

template <int NK>
__global__ __launch_bounds__(256) void gate_bf16_skinny_kernel(const uint16_t* __restrict__ ql,
                                                               const uint16_t* __restrict__ w,
                                                               const uint16_t* o, uint16_t* out,
                                                               int M, int N) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto stage = [](int i) -> char* {
    return i == 0 ? sk_st0 : i == 1 ? sk_st1 : i == 2 ? sk_st2 : sk_st3;
  };
  OLoad ov{o, N};
  gate_skinny::tile<NK>(ql, w, ov, out, M, N, blockIdx.x * gate_skinny::N_TILE, stage, wave,
                        lane);
}

// fp32: 64x64 output tile, each of 256 threads computes a 4x4 block.
template <bool BWD>  // as gate_bf16_kernel
__global__ __launch_bounds__(256) void gate_f32_kernel(const float* __restrict__ ql,
                                                       const float* __restrict__ w,
                                                       const float* o, float* out, int M,
                                                       int d_lat, int N, const float* dout,
                                                       float* dg) {
  __shared__ float sQ[16][64 + 1];
  __shared__ float sW[16][64];
  const int tid = threadIdx.x;
  const int n_tiles_n = (N + 63) / 64;
  const int n0 = (blockIdx.x % n_tiles_n) * 64, m0 = (blockIdx.x / n_tiles_n) * 64;
  const int tm = (tid >> 4) * 4, tn = (tid & 15) * 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < d_lat; k0 += 16) {
    for (int e = tid; e < 16 * 64; e += 256) {
      const int kk = e & 15, mm = e >> 4;  // q_lat[m0+mm][k0+kk]
      sQ[kk][mm] = (m0 + mm < M && k0 + kk < d_lat) ? ql[(size_t)(m0 + mm) * d_lat + k0 + kk]
                                                    : 0.f;
      const int nn = e & 63, kr = e >> 6;  // w[k0+kr][n0+nn]
      sW[kr][nn] = (n0 + nn < N && k0 + kr < d_lat) ? w[(size_t)(k0 + kr) * N + n0 + nn] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sQ[kk][tm + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sW[kk][tn + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + tm + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tn + j;
      if (n >= N) continue;
      const size_t off = (size_t)m * N + n;
      if constexpr (BWD) {
        const float sg = 1.0f / (1.0f + expf(-acc[i][j]));
        dg[off] = dout[off] * o[off] * sg * (1.0f - sg);
        out[off] = dout[off] * sg;
      } else {
        out[off] = o[off] / (1.0f + expf(-acc[i][j]));
      }
    }
  }
}

}  // namespace

hipError_t launch_gate(const void* q_lat, const void* w, const void* o, void* out, int M,
                       int d_lat, int N, int dt, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (dt == DT_BF16 && M >= G2_BM && N >= G2_BN) {
    const int grid = ((N + G2_BN - 1) / G2_BN) * ((M + G2_BM - 1) / G2_BM);
    hipLaunchKernelGGL(gate_bf16_big_kernel<false>, dim3(grid), dim3(512), 0, stream,
                       (const uint16_t*)q_lat, (const uint16_t*)w, (const uint16_t*)o,
                       (uint16_t*)out, M, d_lat, N, nullptr, nullptr);
  } else if (dt == DT_BF16 && M <= 64 && d_lat == 16 * gate_skinny::K_STEP) {
    hipLaunchKernelGGL(gate_bf16_skinny_kernel<16>,
                       dim3((N + gate_skinny::N_TILE - 1) / gate_skinny::N_TILE), dim3(256), 0,
                       stream, (const uint16_t*)q_lat, (const uint16_t*)w, (const uint16_t*)o,
                       (uint16_t*)out, M, N);
  } else if (dt == DT_BF16) {
    const int grid = ((N + GT_N - 1) / GT_N) * ((M + GT_M - 1) / GT_M);
    hipLaunchKernelGGL(gate_bf16_kernel<false>, dim3(grid), dim3(256), 0, stream,
                       (const uint16_t*)q_lat, (const uint16_t*)w, (const uint16_t*)o,
                       (uint16_t*)out, M, d_lat, N, nullptr, nullptr);
  } else {
    const int grid = ((N + 63) / 64) * ((M + 63) / 64);
    hipLaunchKernelGGL(gate_f32_kernel<false>, dim3(grid), dim3(256), 0, stream,
                       (const float*)q_lat, (const float*)w, (const float*)o, (float*)out, M,
                       d_lat, N, nullptr, nullptr);
  }
  return hipGetLastError();
}

// Backward, first step: G recomputed as in the forward, then do = dout * s into d_o and
// dG = dout * o * s * (1 - s) into dg (same dtype as the operands).
hipError_t launch_gate_bwd_elem(const void* q_lat, const void* w, const void* o,
                                const void* dout, void* d_o, void* dg, int M, int d_lat, int N,
                                int dt, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (dt == DT_BF16 && M >= G2_BM && N >= G2_BN) {
    const int grid = ((N + G2_BN - 1) / G2_BN) * ((M + G2_BM - 1) / G2_BM);
    hipLaunchKernelGGL(gate_bf16_big_kernel<true>, dim3(grid), dim3(512), 0, stream,
                       (const uint16_t*)q_lat, (const uint16_t*)w, (const uint16_t*)o,
                       (uint16_t*)d_o, M, d_lat, N, (const uint16_t*)dout, (uint16_t*)dg);
  } else if (dt == DT_BF16) {
    const int grid = ((N + GT_N - 1) / GT_N) * ((M + GT_M - 1) / GT_M);
    hipLaunchKernelGGL(gate_bf16_kernel<true>, dim3(grid), dim3(256), 0, stream,
                       (const uint16_t*)q_lat, (const uint16_t*)w, (const uint16_t*)o,
                       (uint16_t*)d_o, M, d_lat, N, (const uint16_t*)dout, (uint16_t*)dg);
  } else {
    const int grid = ((N + 63) / 64) * ((M + 63) / 64);
    hipLaunchKernelGGL(gate_f32_kernel<true>, dim3(grid), dim3(256), 0, stream,
                       (const float*)q_lat, (const float*)w, (const float*)o, (float*)d_o, M,
                       d_lat, N, (const float*)dout, (float*)dg);
  }
  return hipGetLastError();
}

}  // namespace lgsa
