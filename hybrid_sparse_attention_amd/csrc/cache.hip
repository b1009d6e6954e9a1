// Decode-time cache maintenance (ERNIE 5.5 Flash Base release blog, section 2.1: HCA layers
// keep one entry per completed block of 128 tokens plus a window of recent raw tokens, DSA
// layers keep an indexer key and a latent row per position; the 128-token window is from the
// xenospectrum.com article, long-context section).  A decode step appends its new token to
// these caches before its attention runs.
//
// HCA: one workgroup of four waves per (sequence, 64 column vectors of 16 bytes, K or V).
// Wave 0 writes the new row into the ring; when the token completes a block, the four waves
// sum the block's rows in the order the block compressor uses (wave g adds rows g, g + 4, ...
// in fp32; the four sums are combined as ((g0 + g1) + g2) + g3 and scaled by 1/block), so the
// entry is bit-identical to the one the compressor makes from the same rows.  The block's last
// row is taken from the new token itself: no lane reads a row written by this launch.
#include "common.h"
#include "kernels.h"

namespace lgsa {

namespace {

template <bool BF16>
__global__ __launch_bounds__(256) void hca_append_kernel(const int32_t* __restrict__ pos,
                                                         const void* __restrict__ k_new,
                                                         const void* __restrict__ v_new,
                                                         void* k_win, void* v_win, void* kc,
                                                         void* vc, int d, int win_len,
                                                         int n_cap, int block) {
  constexpr int V = BF16 ? 8 : 4;  // elements per 16-byte vector
  constexpr size_t ESZ = BF16 ? 2 : 4;
  __shared__ float part[4][64][V];
  const int b = blockIdx.x;
  const bool is_v = blockIdx.z != 0;
  const int cv = blockIdx.y * 64 + (threadIdx.x & 63);
  const int rg = threadIdx.x >> 6;  // row group of the block sum
  const int t = pos[b];
  if (t < 0) return;  // uniform over the workgroup
  const bool col = cv < d / V;
  const size_t row_bytes = (size_t)d * ESZ;
  const char* nw = (const char*)(is_v ? v_new : k_new) + b * row_bytes + (size_t)cv * 16;
  char* ring = (char*)(is_v ? v_win : k_win) + (size_t)b * win_len * row_bytes + (size_t)cv * 16;
  uint4 x = make_uint4(0, 0, 0, 0);
  if (col) x = *(const uint4*)nw;
  if (col && rg == 0) *(uint4*)(ring + (size_t)(t % win_len) * row_bytes) = x;
  if (t % block != block - 1 || t / block >= n_cap) return;  // uniform

  // the block sum: wave rg adds rows i = rg, rg + 4, ... in increasing order, as the block
  // compressor does; row block - 1 is the new token
  float acc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) acc[j] = 0.f;
  auto add = [&](const uint4& y) {
    if (BF16) {
      const uint32_t w[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += __uint_as_float(w[j] << 16);
        acc[2 * j + 1] += __uint_as_float(w[j] & 0xFFFF0000u);
      }
    } else {
      acc[0] += __uint_as_float(y.x);
      acc[1] += __uint_as_float(y.y);
      acc[2] += __uint_as_float(y.z);
      acc[3] += __uint_as_float(y.w);
    }
  };
  if (col) {
    const int p0 = t - block + 1;  // first position of the block (>= 0: it is complete)
    int i = rg;
    for (; i + 28 < block - 1; i += 32) {  // eight rows of the group per round, loads first
      uint4 y[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        y[u] = *(const uint4*)(ring + (size_t)((p0 + i + 4 * u) % win_len) * row_bytes);
#pragma unroll
      for (int u = 0; u < 8; ++u) add(y[u]);
    }
    for (; i < block; i += 4)
      add(i == block - 1 ? x : *(const uint4*)(ring + (size_t)((p0 + i) % win_len) * row_bytes));
  }
#pragma unroll
  for (int j = 0; j < V; ++j) part[rg][threadIdx.x & 63][j] = acc[j];
  __syncthreads();
  if (rg != 0 || !col) return;
  const float inv = 1.0f / (float)block;
  float s[V];
#pragma unroll
  for (int j = 0; j < V; ++j)
    s[j] = (((part[0][threadIdx.x][j] + part[1][threadIdx.x][j]) + part[2][threadIdx.x][j]) +
            part[3][threadIdx.x][j]) *
           inv;
  char* dst = (char*)(is_v ? vc : kc) + ((size_t)b * n_cap + t / block) * row_bytes +
              (size_t)cv * 16;
  if (BF16) {
    uint4 o;
    o.x = pack_bf16x2(s[0], s[1]);
    o.y = pack_bf16x2(s[2], s[3]);
    o.z = pack_bf16x2(s[4], s[5]);
    o.w = pack_bf16x2(s[6], s[7]);
    *(uint4*)dst = o;
  } else {
    *(uint4*)dst = make_uint4(__float_as_uint(s[0]), __float_as_uint(s[1]),
                              __float_as_uint(s[2]), __float_as_uint(s[3]));
  }
}

// DSA: one workgroup per sequence copies the new indexer key and latent row, 16 bytes a lane.
__global__ __launch_bounds__(64) void dsa_append_kernel(const int32_t* __restrict__ pos, int S,
                                                        const float* __restrict__ k_idx_new,
                                                        float* k_idx, int di,
                                                        const char* __restrict__ kv_new,
                                                        char* kv_lat, int row_bytes,
                                                        long long stride_bytes) {
  const int b = blockIdx.x;
  const int t = pos[b];
  if (t < 0 || t >= S) return;
  const uint4* ks = (const uint4*)(k_idx_new + (size_t)b * di);
  uint4* kd = (uint4*)(k_idx + ((size_t)b * S + t) * di);
  for (int c = threadIdx.x; c < di / 4; c += 64) kd[c] = ks[c];
  const uint4* vs = (const uint4*)(kv_new + (size_t)b * row_bytes);
  uint4* vd = (uint4*)(kv_lat + ((long long)b * S + t) * stride_bytes);
  for (int c = threadIdx.x; c < row_bytes / 16; c += 64) vd[c] = vs[c];
}

}  // namespace

hipError_t launch_hca_append(const int32_t* pos, const void* k_new, const void* v_new,
                             void* k_win, void* v_win, void* kc, void* vc, int B, int d,
                             int win_len, int n_cap, int block, int dt, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const int n_cv = d / (dt == DT_BF16 ? 8 : 4);
  const dim3 grid(B, (n_cv + 63) / 64, 2);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(hca_append_kernel<true>, grid, dim3(256), 0, stream, pos, k_new, v_new,
                       k_win, v_win, kc, vc, d, win_len, n_cap, block);
  else
    hipLaunchKernelGGL(hca_append_kernel<false>, grid, dim3(256), 0, stream, pos, k_new, v_new,
                       k_win, v_win, kc, vc, d, win_len, n_cap, block);
  return hipGetLastError();
}

hipError_t launch_dsa_append(const int32_t* pos, int B, int S, const float* k_idx_new,
                             float* k_idx, int di, const void* kv_new, void* kv_lat, int row,
                             long long stride, int dt, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const int esz = dt == DT_BF16 ? 2 : 4;
  hipLaunchKernelGGL(dsa_append_kernel, dim3(B), dim3(64), 0, stream, pos, S, k_idx_new, k_idx,
                     di, (const char*)kv_new, (char*)kv_lat, row * esz, stride * esz);
  return hipGetLastError();
}

}  // namespace lgsa
