// Few-row bfloat16 gate tile (ERNIE 5.5 Flash Base release blog, section 2.1, low-rank gated
// attention): out[m, n] = o[m, n] * sigmoid(q_lat[m, :] . w[:, n]) for 64 channels
// n0 .. n0 + 63 and every row m < M <= 64, d_lat = 64 NK.  At decode shapes the gate is a
// stream over W, read once: each of these tiles reads its 64 columns of W (128 bytes of each
// of the d_lat rows) and all M rows of q_lat.
//
// Four waves; wave w takes rows 16w .. 16w + 15 and all four 16-channel blocks.  Each K step of
// 64 brings an 8 KiB W chunk and an 8 KiB q_lat chunk to LDS by LDS DMA, four steps in flight
// in four stages (separate LDS objects chosen by the caller, at least STAGE bytes each); W^T
// fragments come from the transposing LDS read.  Rows of 128 bytes are XOR-swizzled by
// 16-byte chunk: W row r at chunk c ^ (2 ((r >> 1) & 1) + 4 ((r >> 3) & 1)), q_lat row r at
// c ^ ((r >> 1) & 7), which keeps both fragment reads free of bank conflicts.  The K loop is
// fully unrolled: with straight-line code the compiler can tell that the transfers into the
// stage being read have completed (the explicit waits guarantee it).
//
// The factor each output takes is given by the caller's object ov: ov.fetch(m, n0 + 4g) runs
// before the K loop (its loads then arrive while W streams), and ov.value(cb) returns
// o[m, n0 + 16cb + 4g .. + 3] as floats in the epilogue.  The gate kernel reads o there (or
// gives ones when the gate factors alone are asked for); the decode attention merges its key
// splits there.  m is the lane's row, clamped to M - 1.
#pragma once

#include "common.h"

namespace lgsa {
namespace gate_skinny {

constexpr int N_TILE = 64, K_STEP = 64, ROWB = 128;
constexpr int CHUNK = K_STEP * ROWB;  // 8 KiB: 64 rows of 128 bytes
constexpr int STAGE = 2 * CHUNK;      // W chunk then q_lat chunk

__device__ __forceinline__ int wsw(int r) { return 2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1); }
__device__ __forceinline__ int qsw(int r) { return (r >> 1) & 7; }

// stage(i) returns the LDS stage i (0..3).  The caller's four waves all call this; it starts
// and ends with every stage free (the last step ends with a barrier).
template <int NK, class Stage, class OVal>
__device__ __forceinline__ void tile(const uint16_t* __restrict__ ql,
                                     const uint16_t* __restrict__ w, OVal& ov, uint16_t* out,
                                     int M, int N, int n0, const Stage& stage, int wave,
                                     int lane) {
  const int l16 = lane & 15, g = lane >> 4;
  constexpr int nk = NK;
  const int d_lat = NK * K_STEP;
  // DMA of K step kt into stage st: 8 W instructions (8 k-rows each) and 8 q_lat instructions
  // (8 rows each), 4 per wave
  auto dma = [&](int kt, char* st) {
    const int ln = opaque(lane);
    const int k0 = kt * K_STEP;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ins = wave + 4 * u;                 // 0..7
      const int r = 8 * ins + (ln >> 3);            // k-row
      const int chunk = (ln & 7) ^ wsw(r);
      const int n = min(n0 + 8 * chunk, N - 8);     // columns past N repeat the last chunk
      const uint16_t* rowp = w + (size_t)(k0 + 8 * ins) * N;
      lds_dma16(rowp + (uint32_t)((ln >> 3) * N + n), st + ins * 8 * ROWB);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ins = wave + 4 * u;                 // 0..7
      const int r = 8 * ins + (ln >> 3);            // q_lat row
      const int chunk = (ln & 7) ^ qsw(r);
      const int m_first = min(8 * ins, M - 1);      // rows past M repeat the last row
      const int rel = min(r, M - 1) - m_first;
      const uint16_t* rowp = ql + (size_t)m_first * d_lat + k0;
      lds_dma16(rowp + (uint32_t)(rel * d_lat + 8 * chunk), st + CHUNK + ins * 8 * ROWB);
    }
  };
  // lane-constant fragment offsets.  B = q_lat^T: row 16 wave + l16, k 32ks + 8g .. +7.
  const int qr = 16 * wave + l16;
  ov.fetch(min(qr, M - 1), n0 + 4 * g);
  int qoff[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) qoff[ks] = CHUNK + qr * ROWB + 16 * ((4 * ks + g) ^ qsw(qr));
  // A = W^T: channel 16cb + l16, k 32ks + 8g + 4h + 0..3 from the transposed read of rows
  // 32ks + 8g + 4h + l16/4, columns 16cb + 4(l16 % 4) .. +3
  const int a = l16 >> 2;
  auto woff = [&](int ks, int h, int cb) {
    const int r = 32 * ks + 8 * g + 4 * h + a;
    const int c = 2 * cb + ((l16 & 3) >> 1);
    return r * ROWB + 16 * (c ^ wsw(r)) + 8 * (l16 & 1);
  };
  f32x4_t acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const char* st) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      Frag8 bq;
      bq.u = *(const uint4*)(st + qoff[ks]);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const uint2 lo = lds_read_tr16(st + woff(ks, 0, cb));
        const uint2 hi = lds_read_tr16(st + woff(ks, 1, cb));
        Frag8 aw;
        aw.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
        acc[cb] = mfma_16x16x32(aw, bq, acc[cb]);
      }
    }
  };
  // four K steps in flight; stage of step kt = kt % 4.  At step kt the wave waits until its
  // own transfers of step kt have landed (those of kt + 1 .. kt + 2 may still fly: 4 each),
  // then a barrier makes every wave's share visible.
#pragma unroll
  for (int kt = 0; kt < 3 && kt < nk; ++kt) dma(kt, stage(kt & 3));
#pragma unroll
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 3 < nk) dma(kt + 3, stage((kt + 3) & 3));
    // transfers issued after step kt's: min(3, nk - 1 - kt) steps of 4 instructions each
    const int later = (nk - 1 - kt) < 3 ? (nk - 1 - kt) : 3;
    if (later == 3) wait_vm<12>();
    else if (later == 2) wait_vm<8>();
    else if (later == 1) wait_vm<4>();
    else wait_vm<0>();
    lds_barrier();  // every wave's share of step kt has landed (each waited for its own)
    compute(stage(kt & 3));
    lds_barrier();  // every wave is done with this stage before it is refilled
  }
  // epilogue: lane holds G[row 16 wave + l16][channels n0 + 16cb + 4g .. +3]
  if (qr >= M) return;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int n = n0 + 16 * cb + 4 * g;
    if (n >= N) continue;
    const float4 x = ov.value(cb);
    uint2 r;
    r.x = pack_bf16x2(x.x * sigmoidf_fast(acc[cb][0]), x.y * sigmoidf_fast(acc[cb][1]));
    r.y = pack_bf16x2(x.z * sigmoidf_fast(acc[cb][2]), x.w * sigmoidf_fast(acc[cb][3]));
    *(uint2*)(out + (size_t)qr * N + n) = r;
  }
}

}  // namespace gate_skinny
}  // namespace lgsa
