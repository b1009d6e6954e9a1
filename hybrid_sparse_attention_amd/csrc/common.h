// Device-side helpers shared by the gfx950 kernels of the Latent-Gated Sparse Attention
// library: bfloat16 conversion, MFMA wrappers and fragment types, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lgsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// A 16-byte fragment of eight bfloat16 values, viewed either as raw words or as the vector
// type the MFMA builtins take.
union Frag8 {
  uint4 u;
  bf16x8_t v;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Round-to-nearest-even float -> bfloat16 (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats to a packed bfloat16 pair, round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// D = A(16x32) * B(32x16) + C in fp32.  Lane l supplies A row (l % 16) and B column (l % 16),
// each with the eight contraction indices 8*(l/16) .. 8*(l/16)+7 (any fixed relabelling of
// the contraction index used for both operands gives the same product).  Lane l receives
// D rows 4*(l/16) .. 4*(l/16)+3 of column (l % 16).
__device__ __forceinline__ f32x4_t mfma_16x16x32(const Frag8& a, const Frag8& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

// Reductions over the four lanes l, l^16, l^32, l^48 that hold the same MFMA column, with the
// VALU lane swaps of gfx950 instead of LDS permutes.  v_permlane16_swap(x, x) leaves in each
// lane of rows 2i and 2i + 1 (16 lanes each) the pair (row 2i's x, row 2i + 1's x) of its
// position; v_permlane32_swap(x, x) leaves the pair (lower half's x, upper half's x).  Every
// lane thus combines the same two values in the same order, so all four lanes of a column
// end with the same bits.
__device__ __forceinline__ void pair16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

__device__ __forceinline__ void pair32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max16(float v) {
  float a, b;
  pair16(v, a, b);
  pair32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float wave_sum16(float v) {
  float a, b;
  pair16(v, a, b);
  pair32(a + b, a, b);
  return a + b;
}

// Transposes an 8x8 block of bfloat16 held as eight 16-byte rows r[0..7] (row j holds
// columns 0..7) into eight 16-byte columns c[0..7] (column i holds rows 0..7).
__device__ __forceinline__ void transpose8x8(const uint4 r[8], uint4 c[8]) {
  const uint32_t* w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = reinterpret_cast<const uint32_t*>(&r[j]);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    // columns 2m (low halves) and 2m+1 (high halves) of every row
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const uint32_t x = w[2 * n][m], y = w[2 * n + 1][m];
      lo[n] = (x & 0xFFFFu) | (y << 16);
      hi[n] = (x >> 16) | (y & 0xFFFF0000u);
    }
    c[2 * m] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    c[2 * m + 1] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float sigmoidf_fast(float g) {
  // 1 / (1 + e^-g) with e^-g = 2^(-g * log2 e); the hardware reciprocal (about 1 ulp) instead
  // of a correctly rounded division: the factor multiplies a bfloat16 value.  1 + e^-g = inf
  // gives 0, as it should.
  return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-g * 1.4426950408889634f));
}

}  // namespace lgsa

namespace lgsa {

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// LDS DMA: every lane fetches 16 bytes from its global address `src`; lane l's bytes land at
// lds + 16 * l, where `lds` must be the same for all lanes of the wave (it is passed through
// M0).  The data is in LDS once the wave's vector-memory counter has drained.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds, 16, 0, 0);
}

// Transposed LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane i reads the
// four 16-bit values R_i[0..3] at its own address; lane j = 4a + c then receives
// { R_a[c], R_{a+4}[c], R_{a+8}[c], R_{a+12}[c] }.  With lane i pointing at row K_{i/4},
// columns 4(i%4) .. 4(i%4)+3 of a row-major tile, lane j receives column j of rows K_0..K_3:
// the strided operand an MFMA needs when the contraction runs over rows.
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
  const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t*)p);
  uint2 u;
  __builtin_memcpy(&u, &r, sizeof u);
  return u;
}

__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

// Waits until at most N of this wave's vector-memory operations are outstanding (they complete
// in issue order), leaving the LDS and export counters alone.  s_waitcnt fields: vmcnt in bits
// 3:0 and 15:14, expcnt in 6:4, lgkmcnt in 11:8.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS reads and writes
// (lgkmcnt 0), not for its vector-memory loads, so LDS DMA transfers in flight stay in flight
// (__syncthreads waits for those too).  Use it only where no wave reads LDS that a DMA still in
// flight may write.  The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt and expcnt at their maxima, lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Hides a value from the optimiser so that addresses derived from it are recomputed where
// they are used instead of being hoisted (and kept live) across a loop.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

}  // namespace lgsa
