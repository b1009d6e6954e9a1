// Plain GEMMs of the backward pass (the gate's dq_lat = dG W^T and dW = q_lat^T dG):
//   C[m][n] = sum_k A(m, k) B(k, n), fp32 accumulation, C stored in the operands' dtype.
// An operand is either k-contiguous (A(m, k) at a[m * lda + k], B(k, n) at b[n * ldb + k]) or
// k-major (A(m, k) at a[k * lda + m], B(k, n) at b[k * ldb + n]).
//
// bfloat16: 128 x 128 tiles, four waves of 64 x 64 on v_mfma_f32_16x16x32_bf16, K staged 64
// at a time in double-buffered LDS rows of [row][k] (72 elements: padded against bank
// conflicts).  Threads 0..127 stage A and 128..255 stage B: a k-contiguous operand as eight
// 16-byte chunks per thread, a k-major one as one 8 x 8 block per thread transposed in
// registers.  The next K step is loaded into registers while the current one is used.
// float32: 64 x 64 tiles of plain FMA (the small fp32 configurations).
// Large bfloat16 products (M, N multiples of 256, K of 64) take a 256 x 256 LDS-DMA kernel
// instead (below).
#include "common.h"
#include "kernels.h"

namespace lgsa {

namespace {

constexpr int GM_T = 128, GM_K = 64, GM_LD = GM_K + 8;

template <bool KMAJOR>
__device__ __forceinline__ void gemm_load(const uint16_t* x, long long ld, int r0, int R, int k0,
                                          int K, int t, uint4 (&st)[8]) {
  if (KMAJOR) {
    const int kg = t & 7, rg = t >> 3;  // k rows k0 + 8kg .., tile rows 8rg ..
    const int r = r0 + 8 * rg;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = k0 + 8 * kg + j;
      st[j] = (r < R && k < K) ? *(const uint4*)(x + (size_t)k * ld + r) : make_uint4(0, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = t + 128 * j;  // 1024 chunks: tile row c / 8, k chunk c % 8
      const int r = r0 + (c >> 3), k = k0 + 8 * (c & 7);
      st[j] = (r < R && k < K) ? *(const uint4*)(x + (size_t)r * ld + k) : make_uint4(0, 0, 0, 0);
    }
  }
}

template <bool KMAJOR>
__device__ __forceinline__ void gemm_store(uint16_t* s, int t, const uint4 (&st)[8]) {
  if (KMAJOR) {
    const int kg = t & 7, rg = t >> 3;
    uint4 col[8];
    transpose8x8(st, col);
#pragma unroll
    for (int i = 0; i < 8; ++i) *(uint4*)(&s[(8 * rg + i) * GM_LD + 8 * kg]) = col[i];
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = t + 128 * j;
      *(uint4*)(&s[(c >> 3) * GM_LD + 8 * (c & 7)]) = st[j];
    }
  }
}

// Large bfloat16 products (M, N multiples of 256, K of 64): 256 x 256 tiles, 8 waves of
// 128 (n) x 64 (m), the transposed product C^T = B^T A^T on v_mfma_f32_16x16x32_bf16 so that a
// lane's accumulator holds four consecutive columns of one C row.  Both operand tiles reach LDS
// by LDS DMA (no register staging), two stages deep, as in the forward gate kernel: a k-major
// operand as 64 k-rows of 256 values, read through the transposing LDS read; a k-contiguous one
// as 256 rows of 64 k, read as 16-byte fragments.  16-byte chunks are XOR-swizzled against
// bank conflicts by choosing which chunk each lane fetches.
constexpr int GB_T = 256, GB_K = 64;
constexpr int GB_KROW = GB_T * 2;  // bytes per staged k-major row
constexpr int GB_CROW = GB_K * 2;  // bytes per staged k-contiguous row
constexpr int GB_OP = 32768;       // bytes of one staged operand tile (either layout)

__device__ __forceinline__ int gb_kswz(int k) { return 2 * (k & 3) + 8 * ((k >> 3) & 1); }
__device__ __forceinline__ int gb_cswz(int r) { return (r >> 1) & 7; }

// two stages, each [N-side operand][M-side operand]; separate LDS objects named where used
__shared__ __attribute__((aligned(1024))) char gb_st0[2 * GB_OP];
__shared__ __attribute__((aligned(1024))) char gb_st1[2 * GB_OP];

// DMA of one operand tile (tile rows r0 .. r0 + 255, contraction k0 .. k0 + 63): 32
// instructions, 4 per wave
template <bool KM>
__device__ __forceinline__ void gb_dma(const uint16_t* x, long long ld, int r0, int k0, char* dst,
                                       int wave, int lane) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int ins = wave + 8 * u;
    if (KM) {
      const int kr = 2 * ins + (lane >> 5);  // k-row of this lane
      const int chunk = (lane & 31) ^ gb_kswz(kr);
      lds_dma16(x + (size_t)(k0 + kr) * ld + r0 + 8 * chunk, dst + 2 * ins * GB_KROW);
    } else {
      const int r = 8 * ins + (lane >> 3);  // tile row of this lane
      const int chunk = (lane & 7) ^ gb_cswz(r);
      lds_dma16(x + (size_t)(r0 + r) * ld + k0 + 8 * chunk, dst + 8 * ins * GB_CROW);
    }
  }
}

// MFMA operand of tile rows 16 blk + l16, contraction 32 ks + 8g .. +7
template <bool KM>
__device__ __forceinline__ Frag8 gb_frag(const char* st, int blk, int ks, int lane) {
  const int l16 = lane & 15, g = lane >> 4;
  Frag8 f;
  if (KM) {
    const int a = l16 >> 2, c4 = l16 & 3;
    const int kf = gb_kswz(8 * g + a);  // the same for k-rows 32 ks + 8g + 4h + a
    const char* row = st + (32 * ks + 8 * g + a) * GB_KROW + 16 * ((2 * blk + (c4 >> 1)) ^ kf) +
                      8 * (c4 & 1);
    const uint2 lo = lds_read_tr16(row);
    const uint2 hi = lds_read_tr16(row + 4 * GB_KROW);
    f.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
  } else {
    f.u = *(const uint4*)(st + (16 * blk + l16) * GB_CROW + 16 * ((4 * ks + g) ^ gb_cswz(l16)));
  }
  return f;
}

// F32: C is fp32 and blockIdx.y selects the contraction range y * kchunk .. (split K; the
// partials at C + y * M * ldc are summed afterwards).
template <bool AK, bool BK, bool F32>
__global__ __launch_bounds__(512, 1) void gemm_big_kernel(const uint16_t* __restrict__ a,
                                                          long long lda,
                                                          const uint16_t* __restrict__ b,
                                                          long long ldb, void* __restrict__ c,
                                                          long long ldc, int M, int N, int K,
                                                          int kchunk) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int wn = wave & 1, wm = wave >> 1;
  // XCD-aware order (XCD x = id % 8 takes a contiguous run of tiles), then groups of 4 n-tiles
  // x 8 m-tiles so that the workgroups an XCD runs together share operand tiles in its L2
  const int n_nt = N / GB_T, n_mt = M / GB_T;
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
  const int n0 = nt * GB_T, m0 = mt * GB_T;

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto dma = [&](int k0, char* st) {
    gb_dma<BK>(b, ldb, n0, k0, st, wave, lane);
    gb_dma<AK>(a, lda, m0, k0, st + GB_OP, wave, lane);
  };
  const int kbeg = F32 ? blockIdx.y * kchunk : 0;
  const int nk = ((F32 ? min(K, kbeg + kchunk) : K) - kbeg) / GB_K;
  auto step = [&](int kt, const char* cur, char* nxt) {
    if (kt + 1 < nk) dma(kbeg + (kt + 1) * GB_K, nxt);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      Frag8 bm[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bm[j] = gb_frag<AK>(cur + GB_OP, 4 * wm + j, ks, lane);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const Frag8 an = gb_frag<BK>(cur, 8 * wn + i, ks, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32(an, bm[j], acc[i][j]);
      }
    }
    wait_all();
    __syncthreads();
  };
  if (nk > 0) dma(kbeg, gb_st0);
  wait_all();
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, gb_st0, gb_st1);
    if (kt + 1 < nk) step(kt + 1, gb_st1, gb_st0);
  }
  // lane holds C[m0 + 64 wm + 16 j + l16][n0 + 128 wn + 16 i + 4g .. +3]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const size_t crow = (size_t)(m0 + 64 * wm + 16 * j + l16) * ldc + n0 + 128 * wn + 4 * g;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (F32) {
        float* cp = (float*)c + (size_t)blockIdx.y * M * ldc + crow + 16 * i;
        *(f32x4_t*)cp = acc[i][j];
      } else {
        uint2 r;
        r.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        r.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        *(uint2*)((uint16_t*)c + crow + 16 * i) = r;
      }
    }
  }
}

// whether a bfloat16 product suits the 256 x 256 kernel
bool gemm_big_ok(const void* a, long long lda, const void* b, long long ldb, long long ldc, int M,
                 int N, int K, long long min_tiles) {
  return M % GB_T == 0 && N % GB_T == 0 && K % GB_K == 0 && K > 0 &&
         (long long)(M / GB_T) * (N / GB_T) >= min_tiles && lda % 8 == 0 && ldb % 8 == 0 &&
         ldc % 4 == 0 && ((uintptr_t)a & 15) == 0 && ((uintptr_t)b & 15) == 0;
}

// OUT_F32: C is fp32 and blockIdx.y selects a range of `kchunk` contraction indices whose
// partial product goes to C + blockIdx.y * M * ldc (split K; the partials are summed after).
template <bool AK, bool BK, bool OUT_F32>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const uint16_t* __restrict__ a,
                                                        long long lda,
                                                        const uint16_t* __restrict__ b,
                                                        long long ldb, void* __restrict__ cv,
                                                        long long ldc, int M, int N, int K,
                                                        int kchunk) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][GM_T * GM_LD];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][GM_T * GM_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_tn = (N + GM_T - 1) / GM_T;
  const int n0 = (blockIdx.x % n_tn) * GM_T, m0 = (blockIdx.x / n_tn) * GM_T;
  const int wn = (wave & 1) * 64, wm = (wave >> 1) * 64;
  const int l16 = lane & 15, g = lane >> 4;
  const bool is_a = tid < 128;
  const int t = tid & 127;

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 st[8];
  auto store = [&](int buf) {
    if (is_a)
      gemm_store<AK>(sA[buf], t, st);
    else
      gemm_store<BK>(sB[buf], t, st);
  };
  // contraction range of this workgroup (all of K unless split)
  const int kb = OUT_F32 ? (int)blockIdx.y * kchunk : 0;
  const int ke = OUT_F32 ? min(K, kb + kchunk) : K;
  const int nk = ke > kb ? (ke - kb + GM_K - 1) / GM_K : 0;
  auto load_k = [&](int k0) {
    if (is_a)
      gemm_load<AK>(a, lda, m0, M, k0, ke, t, st);
    else
      gemm_load<BK>(b, ldb, n0, N, k0, ke, t, st);
  };
  load_k(kb);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_k(kb + (kt + 1) * GM_K);
#pragma unroll
    for (int ks = 0; ks < GM_K / 32; ++ks) {
      Frag8 fa[4], fb[4];
      // MFMA A operand = rows of B (n), B operand = rows of A (m): lane gets C[m][n .. n+3]
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i].u = *(const uint4*)(&sB[buf][(wn + 16 * i + l16) * GM_LD + 32 * ks + 8 * g]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[j].u = *(const uint4*)(&sA[buf][(wm + 16 * j + l16) * GM_LD + 32 * ks + 8 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }
  // lane holds C[m0 + wm + 16j + l16][n0 + wn + 16i + 4g .. +3]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wm + 16 * j + l16;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + wn + 16 * i + 4 * g;
      if (n >= N) continue;
      if constexpr (OUT_F32) {
        float* c = (float*)cv + (size_t)blockIdx.y * M * ldc;
        *(f32x4_t*)(c + (size_t)m * ldc + n) = acc[i][j];
      } else {
        uint16_t* c = (uint16_t*)cv;
        *(uint2*)(c + (size_t)m * ldc + n) =
            make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]),
                       pack_bf16x2(acc[i][j][2], acc[i][j][3]));
      }
    }
  }
}

template <bool AK, bool BK>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ a, long long lda,
                                                       const float* __restrict__ b,
                                                       long long ldb, float* __restrict__ c,
                                                       long long ldc, int M, int N, int K) {
  __shared__ float sA[16][64 + 1];
  __shared__ float sB[16][64];
  const int tid = threadIdx.x;
  const int n_tn = (N + 63) / 64;
  const int n0 = (blockIdx.x % n_tn) * 64, m0 = (blockIdx.x / n_tn) * 64;
  const int tm = (tid / 16) * 4, tn = (tid % 16) * 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 256 * u;  // 1024 elements of each 16 x 64 slice
      const int kk = e >> 6, rr = e & 63;
      const int k = k0 + kk, m = m0 + rr, n = n0 + rr;
      sA[kk][rr] = (k < K && m < M) ? (AK ? a[(size_t)k * lda + m] : a[(size_t)m * lda + k]) : 0.f;
      sB[kk][rr] = (k < K && n < N) ? (BK ? b[(size_t)k * ldb + n] : b[(size_t)n * ldb + k]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(sA[kk][tm + i], sB[kk][tn + j], acc[i][j]);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (m0 + tm + i < M && n0 + tn + j < N) c[(size_t)(m0 + tm + i) * ldc + n0 + tn + j] = acc[i][j];
}

template <bool AK, bool BK>
hipError_t gemm_launch(const void* a, long long lda, const void* b, long long ldb, void* c,
                       long long ldc, int M, int N, int K, int dt, hipStream_t stream) {
  if (dt == DT_BF16 && gemm_big_ok(a, lda, b, ldb, ldc, M, N, K, 64) && ((uintptr_t)c & 7) == 0) {
    const int grid = (N / GB_T) * (M / GB_T);
    hipLaunchKernelGGL((gemm_big_kernel<AK, BK, false>), dim3(grid), dim3(512), 0, stream,
                       (const uint16_t*)a, lda, (const uint16_t*)b, ldb, c, ldc, M, N, K, K);
  } else if (dt == DT_BF16) {
    const int grid = ((N + GM_T - 1) / GM_T) * ((M + GM_T - 1) / GM_T);
    hipLaunchKernelGGL((gemm_bf16_kernel<AK, BK, false>), dim3(grid), dim3(256), 0, stream,
                       (const uint16_t*)a, lda, (const uint16_t*)b, ldb, c, ldc, M, N, K, K);
  } else {
    const int grid = ((N + 63) / 64) * ((M + 63) / 64);
    hipLaunchKernelGGL((gemm_f32_kernel<AK, BK>), dim3(grid), dim3(256), 0, stream,
                       (const float*)a, lda, (const float*)b, ldb, (float*)c, ldc, M, N, K);
  }
  return hipGetLastError();
}

// Sum of `splits` fp32 partials of M x N (row stride ldc) into out (fp32, row stride ldc).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            float* __restrict__ out, int splits,
                                                            long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int k = 0; k < splits; ++k) s += part[(size_t)k * n + i];
  out[i] = s;
}

}  // namespace

hipError_t launch_gemm_splitk_f32(const void* a, long long lda, bool a_kmajor, const void* b,
                                  long long ldb, bool b_kmajor, float* c, int M, int N, int K,
                                  int splits, float* part, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int kchunk = ((K + splits - 1) / splits + GM_K - 1) / GM_K * GM_K;
  splits = K > 0 ? (K + kchunk - 1) / kchunk : 1;
  const dim3 grid(((N + GM_T - 1) / GM_T) * ((M + GM_T - 1) / GM_T), splits);
  const uint16_t* pa = (const uint16_t*)a;
  const uint16_t* pb = (const uint16_t*)b;
  if (gemm_big_ok(a, lda, b, ldb, N, M, N, K, 1) && a_kmajor && b_kmajor) {
    // the 256 x 256 kernel with the same split (kchunk is a multiple of 64)
    hipLaunchKernelGGL((gemm_big_kernel<true, true, true>), dim3((N / GB_T) * (M / GB_T), splits),
                       dim3(512), 0, stream, pa, lda, pb, ldb, (void*)part, (long long)N, M, N, K,
                       kchunk);
  } else if (a_kmajor && b_kmajor)
    hipLaunchKernelGGL((gemm_bf16_kernel<true, true, true>), grid, dim3(256), 0, stream, pa, lda,
                       pb, ldb, (void*)part, (long long)N, M, N, K, kchunk);
  else if (a_kmajor)
    hipLaunchKernelGGL((gemm_bf16_kernel<true, false, true>), grid, dim3(256), 0, stream, pa, lda,
                       pb, ldb, (void*)part, (long long)N, M, N, K, kchunk);
  else if (b_kmajor)
    hipLaunchKernelGGL((gemm_bf16_kernel<false, true, true>), grid, dim3(256), 0, stream, pa, lda,
                       pb, ldb, (void*)part, (long long)N, M, N, K, kchunk);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<false, false, true>), grid, dim3(256), 0, stream, pa,
                       lda, pb, ldb, (void*)part, (long long)N, M, N, K, kchunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n = (long long)M * N;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     stream, part, c, splits, n);
  return hipGetLastError();
}

hipError_t launch_gemm(const void* a, long long lda, bool a_kmajor, const void* b,
                       long long ldb, bool b_kmajor, void* c, long long ldc, int M, int N, int K,
                       int dt, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (a_kmajor)
    return b_kmajor ? gemm_launch<true, true>(a, lda, b, ldb, c, ldc, M, N, K, dt, stream)
                    : gemm_launch<true, false>(a, lda, b, ldb, c, ldc, M, N, K, dt, stream);
  return b_kmajor ? gemm_launch<false, true>(a, lda, b, ldb, c, ldc, M, N, K, dt, stream)
                  : gemm_launch<false, false>(a, lda, b, ldb, c, ldc, M, N, K, dt, stream);
}

}  // namespace lgsa
