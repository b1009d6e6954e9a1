// Virtual Head Attention mixing step (ERNIE 5.5 Flash Base release blog, section 2.1: after
// attention, a light low-rank mix across heads with an identity skip connection):
//   out[m, h, :] = o[m, h, :] + sum_h' (U V^T)[h, h'] o[m, h', :]
// computed per token m as z = V^T o[m] (rank r <= 16) and out = o[m] + U z.
//
// bfloat16, 64 heads: one workgroup of 4 waves per (token, 256 channels of the head dimension).
// The 64 x 256 tile reaches LDS through registers (rows padded by 32 bytes); wave w mixes
// channels 64w .. 64w + 63 in four blocks of 16 (vha_tile.h: z = V^T o and out^T = z^T U^T + o^T
// on MFMA, in place), and the tile leaves in 16-byte rows.
// A workgroup uses 34 KiB of LDS, so four share a CU and cover each other's memory latency:
// the kernel is bound by reading o and writing out once.
// float32 (any head count): a plain loop per (token, channel).
#include "common.h"
#include "kernels.h"
#include "vha_tile.h"

namespace lgsa {

namespace {

constexpr int VH = 64;               // heads of the bfloat16 path
constexpr int VJ = 256;              // channels per workgroup
constexpr int VROW = VJ * 2 + 32;    // LDS bytes per head row (32-byte pad)

__global__ __launch_bounds__(256) void vha_bf16_kernel(const uint16_t* __restrict__ o,
                                                       const uint16_t* __restrict__ u,
                                                       const uint16_t* __restrict__ v,
                                                       uint16_t* out, int d, int r) {
  __shared__ __attribute__((aligned(16))) char tile[VH * VROW];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_jt = d / VJ;
  const int m = blockIdx.x / n_jt, jt = blockIdx.x % n_jt;
  const size_t base = (size_t)m * VH * d + (size_t)jt * VJ;  // element (m, head 0, channel 0)

  // the tile: 64 rows of 512 bytes = 2048 chunks of 16 bytes; thread tid takes tid + 256 i
  uint4 x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + 256 * i;
    x[i] = *(const uint4*)(o + base + (size_t)(c >> 5) * d + (c & 31) * 8);
  }
  vha_tile::Factors f;
  vha_tile::load_factors(f, u, v, r, lane);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + 256 * i;
    *(uint4*)(tile + (c >> 5) * VROW + (c & 31) * 16) = x[i];
  }
  __syncthreads();
  // wave w takes channels 64w .. 64w + 63 (four blocks of 16)
  vha_tile::mix_blocks([&](int h) { return tile + h * VROW; }, f, 4 * wave, 4, lane);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + 256 * i;
    *(uint4*)(out + base + (size_t)(c >> 5) * d + (c & 31) * 8) =
        *(const uint4*)(tile + (c >> 5) * VROW + (c & 31) * 16);
  }
}

__global__ __launch_bounds__(256) void vha_f32_kernel(const float* o, const float* __restrict__ u,
                                                      const float* __restrict__ v, float* out,
                                                      int M, int H, int d, int r) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)M * d) return;
  const int m = (int)(idx / d), j = (int)(idx % d);
  const size_t b = (size_t)m * H * d + j;
  float z[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) z[k] = 0.f;
  for (int h = 0; h < H; ++h) {
    const float x = o[b + (size_t)h * d];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (k < r) z[k] += v[h * r + k] * x;
  }
  for (int h = 0; h < H; ++h) {
    float acc = o[b + (size_t)h * d];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (k < r) acc += u[h * r + k] * z[k];
    out[b + (size_t)h * d] = acc;
  }
}

}  // namespace

hipError_t launch_vha(const void* o, const void* u, const void* v, void* out, int M, int H,
                      int d, int r, int dt, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (dt == DT_BF16) {
    const long long grid = (long long)M * (d / VJ);
    hipLaunchKernelGGL(vha_bf16_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint16_t*)o, (const uint16_t*)u, (const uint16_t*)v,
                       (uint16_t*)out, d, r);
  } else {
    const long long n = (long long)M * d;
    hipLaunchKernelGGL(vha_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       (const float*)o, (const float*)u, (const float*)v, (float*)out, M, H, d,
                       r);
  }
  return hipGetLastError();
}

}  // namespace lgsa
