// HCA block compressor: one cache entry per complete block of `block` tokens, read as the
// mean of the block's keys (and, separately, values).  ERNIE 5.5 Flash Base release blog,
// section 2.1 "Latent-Gated Sparse Attention" (every 128 tokens become one cache entry).
//
// HBM-bound: each input row is read once with 16-byte loads and each entry written once.
// One workgroup per (entry, 64 column vectors, K or V); its four waves sum interleaved rows
// in fp32 and combine their partial sums through LDS in a fixed order (deterministic).
#include "common.h"
#include "kernels.h"

namespace lgsa {

template <bool BF16>
__global__ __launch_bounds__(256) void compress_kernel(const void* __restrict__ k,
                                                       const void* __restrict__ v,
                                                       void* __restrict__ kc,
                                                       void* __restrict__ vc, int T, int d,
                                                       int block, int n_ent) {
  constexpr int V = BF16 ? 8 : 4;  // elements per 16-byte vector
  __shared__ float part[4][64][V];
  const int ent = blockIdx.x;      // b * n_ent + e
  const int b = ent / n_ent, e = ent % n_ent;
  const int cv = blockIdx.y * 64 + (threadIdx.x & 63);
  const int rg = threadIdx.x >> 6;
  const int n_cv = d / V;
  const char* src = (const char*)(blockIdx.z == 0 ? k : v);
  char* dst = (char*)(blockIdx.z == 0 ? kc : vc);
  const size_t esz = BF16 ? 2 : 4;
  float acc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) acc[j] = 0.f;
  if (cv < n_cv) {
    const size_t row0 = (size_t)b * T + (size_t)e * block;
    for (int i = rg; i < block; i += 4) {
      const uint4 x = *(const uint4*)(src + ((row0 + i) * d + (size_t)cv * V) * esz);
      if (BF16) {
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] += __uint_as_float(w[j] << 16);
          acc[2 * j + 1] += __uint_as_float(w[j] & 0xFFFF0000u);
        }
      } else {
        acc[0] += __uint_as_float(x.x);
        acc[1] += __uint_as_float(x.y);
        acc[2] += __uint_as_float(x.z);
        acc[3] += __uint_as_float(x.w);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < V; ++j) part[rg][threadIdx.x & 63][j] = acc[j];
  __syncthreads();
  if (rg == 0 && cv < n_cv) {
    const float inv = 1.0f / (float)block;
    float s[V];
#pragma unroll
    for (int j = 0; j < V; ++j)
      s[j] = (((part[0][threadIdx.x][j] + part[1][threadIdx.x][j]) + part[2][threadIdx.x][j]) +
              part[3][threadIdx.x][j]) *
             inv;
    const size_t off = ((size_t)ent * d + (size_t)cv * V) * esz;
    if (BF16) {
      uint4 o;
      o.x = pack_bf16x2(s[0], s[1]);
      o.y = pack_bf16x2(s[2], s[3]);
      o.z = pack_bf16x2(s[4], s[5]);
      o.w = pack_bf16x2(s[6], s[7]);
      *(uint4*)(dst + off) = o;
    } else {
      *(uint4*)(dst + off) = make_uint4(__float_as_uint(s[0]), __float_as_uint(s[1]),
                                        __float_as_uint(s[2]), __float_as_uint(s[3]));
    }
  }
}

hipError_t launch_compress(const void* k, const void* v, void* kc, void* vc, int B, int T,
                           int d, int block, int dt, hipStream_t stream) {
  const int n_ent = T / block;
  if (B == 0 || n_ent == 0) return hipSuccess;
  const int V = dt == DT_BF16 ? 8 : 4;
  dim3 grid(B * n_ent, (d / V + 63) / 64, 2);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(compress_kernel<true>, grid, dim3(256), 0, stream, k, v, kc, vc, T, d,
                       block, n_ent);
  else
    hipLaunchKernelGGL(compress_kernel<false>, grid, dim3(256), 0, stream, k, v, kc, vc, T, d,
                       block, n_ent);
  return hipGetLastError();
}

}  // namespace lgsa
