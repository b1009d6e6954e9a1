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
  if (dt == DT_BF16) {
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
  if (a_kmajor && b_kmajor)
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
