// Low-rank output gate (ERNIE 5.5 Flash Base release blog, section 2.1, low-rank gated
// attention): out[m, n] = o[m, n] * sigmoid(q_lat[m, :] . w[:, n]), the gate logits computed
// from the 1024-wide query latent and never written to memory.
//
// bfloat16 path: an MFMA GEMM computing the transposed product G^T = W^T q_lat^T so that
// every lane ends with four consecutive output channels of one row, which it multiplies into
// o and stores as 8 bytes.  The W tile is transposed while it is staged in LDS (the MFMA
// wants the contraction index contiguous per lane, W has it strided).
// Workgroup tile: 128 channels x 128 rows, four waves of 64 x 64, K staged 64 at a time in
// double-buffered LDS.
//
// float32 path: a plain tiled FMA GEMM (used for the small fp32 configuration).
#include "common.h"
#include "kernels.h"

namespace lgsa {

namespace {

constexpr int GT_N = 128, GT_M = 128, GT_K = 64, GT_LD = GT_K + 8;  // LDS row: 72 bf16

__global__ __launch_bounds__(256) void gate_bf16_kernel(const uint16_t* __restrict__ ql,
                                                        const uint16_t* __restrict__ w,
                                                        const uint16_t* o, uint16_t* out,
                                                        int M, int d_lat, int N) {
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
      const uint2 ov = *(const uint2*)(o + off);
      const float o0 = __uint_as_float(ov.x << 16), o1 = __uint_as_float(ov.x & 0xFFFF0000u);
      const float o2 = __uint_as_float(ov.y << 16), o3 = __uint_as_float(ov.y & 0xFFFF0000u);
      uint2 r;
      r.x = pack_bf16x2(o0 * sigmoidf_fast(acc[i][j][0]), o1 * sigmoidf_fast(acc[i][j][1]));
      r.y = pack_bf16x2(o2 * sigmoidf_fast(acc[i][j][2]), o3 * sigmoidf_fast(acc[i][j][3]));
      *(uint2*)(out + off) = r;
    }
  }
}

// fp32: 64x64 output tile, each of 256 threads computes a 4x4 block.
__global__ __launch_bounds__(256) void gate_f32_kernel(const float* __restrict__ ql,
                                                       const float* __restrict__ w,
                                                       const float* o, float* out, int M,
                                                       int d_lat, int N) {
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
      out[off] = o[off] / (1.0f + expf(-acc[i][j]));
    }
  }
}

}  // namespace

hipError_t launch_gate(const void* q_lat, const void* w, const void* o, void* out, int M,
                       int d_lat, int N, int dt, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (dt == DT_BF16) {
    const int grid = ((N + GT_N - 1) / GT_N) * ((M + GT_M - 1) / GT_M);
    hipLaunchKernelGGL(gate_bf16_kernel, dim3(grid), dim3(256), 0, stream,
                       (const uint16_t*)q_lat, (const uint16_t*)w, (const uint16_t*)o,
                       (uint16_t*)out, M, d_lat, N);
  } else {
    const int grid = ((N + 63) / 64) * ((M + 63) / 64);
    hipLaunchKernelGGL(gate_f32_kernel, dim3(grid), dim3(256), 0, stream, (const float*)q_lat,
                       (const float*)w, (const float*)o, (float*)out, M, d_lat, N);
  }
  return hipGetLastError();
}

}  // namespace lgsa
