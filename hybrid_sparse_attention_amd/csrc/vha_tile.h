// Virtual Head Attention on a token's 64 heads held in LDS (ERNIE 5.5 Flash Base release blog,
// section 2.1: after attention, a light low-rank mix across heads with an identity skip):
//   out[h, :] = o[h, :] + sum_h' (U V^T)[h, h'] o[h', :],  z = V^T o (rank r <= 16), out = o + U z
// shared by the stand-alone mixing kernel and the epilogue of the sparse attention kernel.
// Each head's row is 256 bfloat16 channels; row(h) gives its LDS address (any pitch whose
// transposing reads of heads g, g + 4, .. fall on distinct banks: 544 bytes).  Per block of 16
// channels:
//   - z (16 x 16, fp32) = V^T (16 x 64) o (64 x 16): two v_mfma_f32_16x16x32_bf16 whose B
//     operand (8 heads of one channel per lane) comes from the transposing LDS read; the
//     contraction over heads is order-free, so lane group g's eight k-slots take heads g, g + 4,
//     .., g + 28 of each half;
//   - out^T (16 channels x 16 heads per head block) = z^T U^T + o^T on v_mfma_f32_16x16x16_bf16,
//     whose A operand is the lane's four z values rounded to bf16 (z's accumulator layout as it
//     stands) and whose accumulator starts as o^T: four consecutive channels of one head per
//     lane, one 8-byte LDS read.  The result replaces o in place.
#pragma once

#include "common.h"

namespace lgsa {
namespace vha_tile {

typedef short v4i16_t2 __attribute__((ext_vector_type(4)));

struct Factors {
  Frag8 vt[2];        // V^T as the A operand of z: row = rank l16, k-slot 8g + e = head 32kh + g + 4e
  v4i16_t2 ut[4];     // U^T as the B operand of out^T: column = head 16hb + l16, k-slot 4g + e = rank
};

// u, v [64, r] bfloat16; ranks r .. 15 read as zero
__device__ __forceinline__ void load_factors(Factors& f, const uint16_t* u, const uint16_t* v,
                                             int r, int lane) {
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    uint16_t e8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) e8[e] = l16 < r ? v[(32 * kh + g + 4 * e) * r + l16] : 0;
    __builtin_memcpy(&f.vt[kh].u, e8, sizeof e8);
  }
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      f.ut[hb][e] = (short)(4 * g + e < r ? u[(16 * hb + l16) * r + 4 * g + e] : 0);
}

// Mixes channel blocks jb0 .. jb0 + nb - 1 (16 channels each) of the 64 rows in place; a
// block is touched by the calling wave only.
template <class RowOf>
__device__ __forceinline__ void mix_blocks(const RowOf& row, const Factors& f, int jb0, int nb,
                                           int lane) {
  const int l16 = lane & 15, g = lane >> 4;
  for (int jb = jb0; jb < jb0 + nb; ++jb) {
    const int j = 16 * jb;  // first channel of the block
    f32x4_t z = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      // lanes 4a .. 4a + 3 of group g point at head 32 kh + g + 4a (lo) / + 16 (hi), channels
      // j + 4 (l16 % 4) ..: lane l16 receives channel j + l16 of those four heads
      const int hd = 32 * kh + g + 4 * (l16 >> 2);
      const int cb = (j + 4 * (l16 & 3)) * 2;
      const uint2 lo = lds_read_tr16(row(hd) + cb);
      const uint2 hi = lds_read_tr16(row(hd + 16) + cb);
      Frag8 ob;
      ob.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
      z = mfma_16x16x32(f.vt[kh], ob, z);
    }
    // z[i] = Z[rank 4g + i][channel j + l16]: the A operand of z^T U^T as it stands
    v4i16_t2 za;
    const uint32_t z01 = pack_bf16x2(z[0], z[1]), z23 = pack_bf16x2(z[2], z[3]);
    za[0] = (short)(z01 & 0xFFFF);
    za[1] = (short)(z01 >> 16);
    za[2] = (short)(z23 & 0xFFFF);
    za[3] = (short)(z23 >> 16);
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      // accumulator: out^T[channel j + 4g + i][head 16 hb + l16] starting from o
      uint2* q = (uint2*)(row(16 * hb + l16) + (j + 4 * g) * 2);
      const uint2 ov = *q;
      f32x4_t acc;
      acc[0] = __uint_as_float(ov.x << 16);
      acc[1] = __uint_as_float(ov.x & 0xFFFF0000u);
      acc[2] = __uint_as_float(ov.y << 16);
      acc[3] = __uint_as_float(ov.y & 0xFFFF0000u);
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(za, f.ut[hb], acc, 0, 0, 0);
      uint2 res;
      res.x = pack_bf16x2(acc[0], acc[1]);
      res.y = pack_bf16x2(acc[2], acc[3]);
      *q = res;
    }
  }
}

}  // namespace vha_tile
}  // namespace lgsa
