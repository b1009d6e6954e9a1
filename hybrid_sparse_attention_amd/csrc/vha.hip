// Virtual Head Attention mixing step (ERNIE 5.5 Flash Base release blog, section 2.1: after
// attention, a light low-rank mix across heads with an identity skip connection):
//   out[m, h, :] = o[m, h, :] + sum_h' (U V^T)[h, h'] o[m, h', :]
// computed per token m as z = V^T o[m] (rank r <= 16) and out = o[m] + U z.
//
// bfloat16, 64 heads: one workgroup of 4 waves per (token, 256 channels of the head dimension).
// The 64 x 256 tile reaches LDS through registers (rows padded by 32 bytes); wave w takes
// channels 64w .. 64w + 63 in four blocks of 16:
//   - z (16 x 16 per block, fp32) = V^T (16 x 64) o (64 x 16): two v_mfma_f32_16x16x32_bf16.
//     The B operand (8 heads of one channel per lane) comes from the transposing LDS read.
//     The contraction over heads does not depend on their order, so lane group g's eight
//     k-slots take heads g, g + 4, ..., g + 28 (of each half): the 16 rows one transposing
//     read touches then fall on distinct bank groups.
//   - out^T (16 channels x 16 heads per head block) = z^T U^T + o^T: v_mfma_f32_16x16x16_bf16
//     whose A operand is the lane's four z values rounded to bf16 (z's accumulator layout is
//     already that operand's layout) and whose accumulator starts as o^T, which is four
//     consecutive channels of one head per lane (one 8-byte LDS read).  The result is written
//     back in place, and the tile leaves in 16-byte rows.
// A workgroup uses 34 KiB of LDS, so four share a CU and cover each other's memory latency:
// the kernel is bound by reading o and writing out once.
// float32 (any head count): a plain loop per (token, channel).
#include "common.h"
#include "kernels.h"

namespace lgsa {

namespace {

typedef short v4i16_mx __attribute__((ext_vector_type(4)));

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
  const int l16 = lane & 15, g = lane >> 4;
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
  // factors (zero beyond rank r): V^T as the A operand of the first product (row = rank
  // index l16, k-slot 8g + e = head 32 kh + g + 4e), U^T as the B operand of the second
  // (column = head 16 hb + l16, k-slot 4g + e = rank index 4g + e)
  Frag8 vt[2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    uint16_t e8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) e8[e] = l16 < r ? v[(32 * kh + g + 4 * e) * r + l16] : 0;
    __builtin_memcpy(&vt[kh].u, e8, sizeof e8);
  }
  v4i16_mx ut[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      ut[hb][e] = (short)(4 * g + e < r ? u[(16 * hb + l16) * r + 4 * g + e] : 0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + 256 * i;
    *(uint4*)(tile + (c >> 5) * VROW + (c & 31) * 16) = x[i];
  }
  __syncthreads();

#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    const int j = 64 * wave + 16 * jb;  // first channel of the block within the tile
    f32x4_t z = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      // lanes 4a .. 4a + 3 of group g point at head 32 kh + g + 4a (lo) / + 16 (hi), channels
      // j + 4 (l16 % 4) ..: lane l16 receives channel j + l16 of those four heads
      const char* p = tile + (32 * kh + g + 4 * (l16 >> 2)) * VROW + (j + 4 * (l16 & 3)) * 2;
      const uint2 lo = lds_read_tr16(p);
      const uint2 hi = lds_read_tr16(p + 16 * VROW);
      Frag8 ob;
      ob.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
      z = mfma_16x16x32(vt[kh], ob, z);
    }
    // z[i] = Z[rank 4g + i][channel j + l16]: the A operand of z^T U^T as it stands
    v4i16_mx za;
    const uint32_t z01 = pack_bf16x2(z[0], z[1]), z23 = pack_bf16x2(z[2], z[3]);
    za[0] = (short)(z01 & 0xFFFF);
    za[1] = (short)(z01 >> 16);
    za[2] = (short)(z23 & 0xFFFF);
    za[3] = (short)(z23 >> 16);
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      // accumulator: out^T[channel j + 4g + i][head 16 hb + l16] starting from o
      uint2* q = (uint2*)(tile + (16 * hb + l16) * VROW + (j + 4 * g) * 2);
      const uint2 ov = *q;
      f32x4_t acc;
      acc[0] = __uint_as_float(ov.x << 16);
      acc[1] = __uint_as_float(ov.x & 0xFFFF0000u);
      acc[2] = __uint_as_float(ov.y << 16);
      acc[3] = __uint_as_float(ov.y & 0xFFFF0000u);
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(za, ut[hb], acc, 0, 0, 0);
      uint2 res;
      res.x = pack_bf16x2(acc[0], acc[1]);
      res.y = pack_bf16x2(acc[2], acc[3]);
      *q = res;  // only this wave touches these channels
    }
  }
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
