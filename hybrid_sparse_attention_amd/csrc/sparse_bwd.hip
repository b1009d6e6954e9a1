// Backward of the DSA sparse core attention (ERNIE 5.5 Flash Base release blog, section 2.1:
// core attention over the top-k positions the indexer picks, 256-wide MLA heads), by the chain
// rule of the forward: with P rebuilt from the forward's log-sum-exp, dP = dO V^T and
// D = rowsum(dO * O),
//     dS = P (dP - D),  dq = scale dS K,  (row s of dk) += scale dS^T q,  (row s of dv) += P^T dO
// over every (query row, entry) that lists s.
//
// Each query row lists its own keys, so the key-side gradients of one row are 32 rows of 256
// columns per tile, scattered over the latent rows.  They are made deterministic without
// atomics on floating point: a counting pass gives every (row, entry) a slot in an order sorted
// by key and then by query row, the main kernel writes each contribution (bfloat16) to its
// slot, and a reduction sums each key's slots in that order in fp32.  Rows are processed in
// chunks that bound the slot buffer; a chunk's sums are carried in an fp32 accumulator.
//
//   rank    one workgroup per range of query rows: for each row in turn, each valid entry takes
//           the next count of (key, range) with an integer atomic.  A row lists a key once
//           (twice only as a duplicate, whose contributions are equal), and the rows of a range
//           are ranked one after another, so the counts it returns follow the row order.
//   scan    exclusive prefix sum over the (key, range) counts in key-major order (stored
//           range-major, as counted): each key's slots are contiguous and ordered by range (per
//           block of counters, plus the blocks' prefix, which the readers add).
//   slot    slot = offset(key, range) + rank.
//   main    one workgroup (8 waves) per query row and group of 64 heads.  Wave w takes heads
//           16(w % 4) .. +15 and keys 16(w / 4) .. +15 of each 32-key tile for S^T = K Q^T and
//           dP^T = V dO^T (K rows read row-wise, Q and dO in registers); P and scale*dS go to
//           LDS as [key][head] bfloat16; then dq^T = K^T dS^T over the tile's 32 keys for dims
//           128(w / 4) .. +127 (K through the transposing read) and the key-side contributions
//           C^T = Q^T dS^T + dO^T P^T for dims 32w .. +31 (Q^T, dO^T in registers, staged
//           through LDS once per row).  Tiles are pipelined (the scores of tile t + 1 are
//           computed between the same two barriers as the products of tile t), K tiles are
//           gathered by LDS DMA two tiles ahead, and the contributions are stored without
//           waiting for them.
//   reduce  one wave per key: its slots in order, plus the accumulator of earlier chunks.
#include <algorithm>
#include <cstdint>

#include "common.h"
#include "kernels.h"
#include "sparse_tile.h"

namespace lgsa {

namespace {

using namespace sparse_tile;

constexpr float LOG2E = 1.4426950408889634f;
constexpr int NW = 8;                          // waves of the main kernel
constexpr int PROW = 144;                      // bytes per key row of the P, dS tiles (64 heads + pad)
constexpr int QROW = 544;                      // bytes per head row of the staged Q, dO (256 + pad)
constexpr size_t BUF_BUDGET = 8ull << 30;      // bytes of contributions held per chunk of rows
constexpr long long SCAN_BLOCK = 4096;         // counters per block of the scan
constexpr long long MAX_COUNTERS = SCAN_BLOCK * 16384;  // what the two-level scan covers
constexpr int MAX_RANGES = 256;
constexpr int RANK_LDS_KEYS = 65536;                   // keys the LDS counters of a range hold

__device__ __forceinline__ void store4(uint16_t* dst, const f32x4_t& v) {
  uint2 r;
  r.x = pack_bf16x2(v[0], v[1]);
  r.y = pack_bf16x2(v[2], v[3]);
  *(uint2*)dst = r;
}

__device__ __forceinline__ float dot8(const uint4& a, const uint4& b) {
  const uint32_t x[4] = {a.x, a.y, a.z, a.w}, y[4] = {b.x, b.y, b.z, b.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s += __uint_as_float(x[i] << 16) * __uint_as_float(y[i] << 16);
    s += __uint_as_float(x[i] & 0xFFFF0000u) * __uint_as_float(y[i] & 0xFFFF0000u);
  }
  return s;
}

// slot row of tile key `lane` (lane < 32): a real slot, or this workgroup's scratch row for a
// skipped entry (stores stay unconditional, so every tile issues the same number of them)
__device__ __forceinline__ int load_slot(const int32_t* sl, int j0, int k, int lane) {
  const int j = j0 + lane;
  return (lane < KT && j < k) ? sl[j] : -1;
}

typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef int v4i_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lds_addr(const char* a) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)a;
}

// The P and dS tiles are read in asm blocks that wait for their own reads.  Read through the
// builtins, the compiler made each tile wait for the gathers in flight before these reads (it
// could not tell that the LDS DMA does not write them), which took away the overlap of the
// gathers with compute.  Four 16-byte rows: key rows l16 and 16 + l16, heads 8g .. 8g+7 and
// 32 + 8g .. 32 + 8g + 7, from `a` = row l16, column 8g.
__device__ __forceinline__ void read_rows4(Frag8 (&f)[2][2], const char* a) {
  v4i_t x0, x1, x2, x3;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:64\n\t"
      "ds_read_b128 %2, %4 offset:%5\n\t"
      "ds_read_b128 %3, %4 offset:%6\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(x0), "=v"(x1), "=v"(x2), "=v"(x3)
      : "v"(lds_addr(a)), "i"(16 * PROW), "i"(16 * PROW + 64));
  f[0][0].u = make_uint4(x0[0], x0[1], x0[2], x0[3]);
  f[0][1].u = make_uint4(x1[0], x1[1], x1[2], x1[3]);
  f[1][0].u = make_uint4(x2[0], x2[1], x2[2], x2[3]);
  f[1][1].u = make_uint4(x3[0], x3[1], x3[2], x3[3]);
}

// two transposing reads, of rows K_0..K_3 at `a` and of the rows 16 further down
__device__ __forceinline__ Frag8 read_tr_pair(const char* a) {
  v2i_t lo, hi;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %2\n\t"
      "ds_read_b64_tr_b16 %1, %2 offset:%3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(lo), "=v"(hi)
      : "v"(lds_addr(a)), "i"(16 * PROW));
  Frag8 f;
  f.u = make_uint4(lo[0], lo[1], hi[0], hi[1]);
  return f;
}

// grid: chunk row q (of n_rows) x head group; rows 0 .. n_wg - 1 of buf are the scratch rows.
// Tiles are pipelined: between two barriers a wave computes S^T, dP^T and writes P, dS of tile
// t + 1 (stage A) and the products of tile t (stage B), so one barrier per tile suffices and
// the VALU work of A overlaps the matrix work of B.  K tiles are triple buffered (t, t + 1, and
// t + 2 in flight), P / dS double buffered.
template <bool ALIAS>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sparse_bwd_kernel(SparseBwdParams p, long long row0, const int32_t* __restrict__ slot,
                       uint16_t* __restrict__ buf) {
  constexpr int RW = ALIAS ? D : 2 * D;  // columns of one contribution row
  constexpr int PD_P = KT * PROW;        // P after scale*dS in one P / dS buffer
  constexpr int PD = 2 * PD_P;
  __shared__ __attribute__((aligned(1024))) char kt0[TILE];
  __shared__ __attribute__((aligned(1024))) char kt1[TILE];
  __shared__ __attribute__((aligned(1024))) char kt2[TILE];
  __shared__ __attribute__((aligned(1024))) char vt0[ALIAS ? 16 : TILE];
  __shared__ __attribute__((aligned(1024))) char vt1[ALIAS ? 16 : TILE];
  __shared__ __attribute__((aligned(1024))) char vt2[ALIAS ? 16 : TILE];
  __shared__ __attribute__((aligned(16))) char pd[2 * PD];     // [key][head] bf16, two tiles
  __shared__ __attribute__((aligned(16))) char qs[64 * QROW];  // Q, then dO [head][dim]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int hb = wave & 3, kh = wave >> 2;
  const int hl = 16 * hb + l16;  // this lane's head (S^T and dq^T column)
  const int n_hg = p.H / 64;
  const int hg = blockIdx.x % n_hg;
  const int q = blockIdx.x / n_hg;
  const long long row = row0 + q;  // b * Tq + i
  const int b = (int)(row / p.Tq);
  const long long n_wg = (long long)gridDim.x;
  const size_t hrow = (size_t)row * p.H + 64 * hg;  // first head of the group
  const uint16_t* Q = (const uint16_t*)p.q + hrow * D;
  const uint16_t* dO = (const uint16_t*)p.dout + hrow * D;
  const uint16_t* O = (const uint16_t*)p.out + hrow * D;
  const int32_t* idx = p.idx + (size_t)row * p.k;
  const int32_t* sl = slot + (size_t)q * p.k;
  const uint16_t* kl = (const uint16_t*)p.k_lat + (size_t)b * p.S * p.k_stride;
  const uint16_t* vl = (const uint16_t*)p.v_lat + (size_t)b * p.S * p.v_stride;
  const int n_tiles = (p.k + KT - 1) / KT;

  // tiles 0 and 1 in flight first
  const int ix0 = valid_ix(load_ix(idx, 0, p.k, lane), p.S);
  const uint32_t valid0 = (uint32_t)__ballot(ix0 >= 0);
  gather_tile<NW>(kl, p.k_stride, ix0, kt0, wave, lane);
  if (!ALIAS) gather_tile<NW>(vl, p.v_stride, ix0, vt0, wave, lane);
  uint32_t valid_n1 = 0;
  if (n_tiles > 1) {
    const int ix1 = valid_ix(load_ix(idx, KT, p.k, lane), p.S);
    valid_n1 = (uint32_t)__ballot(ix1 >= 0);
    gather_tile<NW>(kl, p.k_stride, ix1, kt1, wave, lane);
    if (!ALIAS) gather_tile<NW>(vl, p.v_stride, ix1, vt1, wave, lane);
  }
  int ix_n2 = load_ix(idx, 2 * KT, p.k, lane);
  int slot_cur = load_slot(sl, 0, p.k, lane);

  // Q and dO in registers for S^T (and D), and through LDS (one after the other) for the
  // transposed A operand of C^T: rows = dims 32w + 16mb + l16, contraction = heads
  // 32(ks & 1) + 8g .. +7 of Q (ks < 2) or dO (ks >= 2)
  Frag8 qf[8], df[8];
  float dsum = 0.f;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    qf[kk].u = *(const uint4*)(Q + hl * D + 32 * kk + 8 * g);
    df[kk].u = *(const uint4*)(dO + hl * D + 32 * kk + 8 * g);
    dsum += dot8(df[kk].u, *(const uint4*)(O + hl * D + 32 * kk + 8 * g));
  }
  const float Dh = wave_sum16(dsum);
  const float lse2 = p.lse[hrow + hl] * LOG2E;
  const bool live = lse2 > -INFINITY;
  const float scale_log2 = p.scale * LOG2E;
  Frag8 cq[4][2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const uint16_t* src = half ? dO : Q;
    for (int i = tid; i < 64 * 32; i += 64 * NW) {
      const int h = i >> 5, c = i & 31;
      *(uint4*)(qs + h * QROW + 16 * c) = *(const uint4*)(src + h * D + 8 * c);
    }
    __syncthreads();
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      const char* base = qs + (32 * kq + 8 * g + (l16 >> 2)) * QROW;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int col = 32 * wave + 16 * mb + 4 * (l16 & 3);
        const uint2 lo = lds_read_tr16(base + 2 * col);
        const uint2 hi = lds_read_tr16(base + 4 * QROW + 2 * col);
        cq[2 * half + kq][mb].u = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    }
    __syncthreads();
  }

  // lane-constant LDS offsets: key rows 16kh + l16 read row-wise (as the forward's scores) and
  // the transposing reads of K^T (rows 4g + l16/4 and +16, as the forward's V^T)
  // key row 16kh + l16, chunk 4kk + g at position (4kk + kcol) mod 32
  const int kb = l16 * TROW + 16 * TROW * kh, kcol = g + 2 * l16 + 16 * (l16 & 1);
  const int vr = 4 * g + (l16 >> 2);
  const int vrow = vr * TROW + 8 * (l16 & 1);
  // K^T reads: chunk 2j + vh of rows vr, vr + 16 at position (2j + vcol) mod 32
  const int vcol = ((l16 & 3) >> 1) + 2 * vr + 16 * (vr & 1);
  // dS^T operand of dq^T: column = head hl, contraction slots 8g .. 8g+7 = keys 4g .. 4g+3 and
  // 16 + 4g .. 16 + 4g + 3 (the order the K^T read gives)
  const int dsb = (4 * g + (l16 >> 2)) * PROW + 2 * (16 * hb + 4 * (l16 & 3));
  const int rwb = l16 * PROW + 16 * g;  // C^T operand rows l16 (+16), heads 8g (+32)

  f32x4_t dq[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) dq[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // stage A: S^T and dP^T of a tile (keys 16kh + 4g + r, head hl), P and scale*dS to LDS
  auto stage_a = [&](const char* kx, const char* vx, uint32_t valid, char* pw) {
    f32x4_t s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      Frag8 ka;
      const int ko = kb + 16 * ((4 * kk + kcol) & 31);
      ka.u = *(const uint4*)(kx + ko);
      s = mfma_16x16x32(ka, qf[kk], s);
      if (ALIAS) {
        dp = mfma_16x16x32(ka, df[kk], dp);
      } else {
        Frag8 va;
        va.u = *(const uint4*)(vx + ko);
        dp = mfma_16x16x32(va, df[kk], dp);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 16 * kh + 4 * g + r;
      const bool v = live && ((valid >> key) & 1u);
      const float pr = v ? fast_exp2(s[r] * scale_log2 - lse2) : 0.f;
      const float dsv = pr * (dp[r] - Dh) * p.scale;
      const bf16x2_t pp = {(__bf16)pr, (__bf16)dsv};
      const uint32_t u = __builtin_bit_cast(uint32_t, pp);
      *(uint16_t*)(pw + PD_P + key * PROW + 2 * hl) = (uint16_t)(u & 0xFFFFu);
      *(uint16_t*)(pw + key * PROW + 2 * hl) = (uint16_t)(u >> 16);
    }
  };

  // Stages A (of the next tile: S^T, dP^T from kx, then P and scale*dS to pw) and B (of the
  // current tile: dq^T += K^T dS^T from kc, and the contributions C^T = Q^T dS^T (+ dO^T P^T)
  // from pr) written interleaved, one step of each per contraction step, so that the matrix
  // cores have independent work while A's chains and LDS reads wait.
  auto tile_ops = [&](const char* kx, const char* vx, uint32_t valid, char* pw, const char* kc,
                      const char* pr_, int slot_c) {
    const Frag8 bds = read_tr_pair(pr_ + dsb);
    Frag8 bd[2][2], bp[2][2];
    read_rows4(bd, pr_ + rwb);
    read_rows4(bp, pr_ + PD_P + rwb);
    f32x4_t s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
    f32x4_t ck[2][2], cv[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) ck[mb][nb] = cv[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int vc_t = opaque(vcol);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      Frag8 ka;
      const int ko = kb + 16 * ((4 * kk + kcol) & 31);
      ka.u = *(const uint4*)(kx + ko);
      const int pos = (2 * (8 * kh + kk) + vc_t) & 31;
      const char* at = kc + vrow + 16 * pos;
      const uint2 lo = lds_read_tr16(at);
      const uint2 hi = lds_read_tr16(at + 16 * TROW);
      Frag8 kq;
      kq.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
      s = mfma_16x16x32(ka, qf[kk], s);
      if (ALIAS) {
        dp = mfma_16x16x32(ka, df[kk], dp);
      } else {
        Frag8 va;
        va.u = *(const uint4*)(vx + ko);
        dp = mfma_16x16x32(va, df[kk], dp);
      }
      dq[kk] = mfma_16x16x32(kq, bds, dq[kk]);
      // C^T products j = 2kk, 2kk + 1 of 16: nb = j / 8, ks = (j / 4) % 2, mb = (j / 2) % 2,
      // and j % 2 picks the dS (Q) or the P (dO) term
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * kk + jj;
        const int nb = j >> 3, ks = (j >> 2) & 1, mb = (j >> 1) & 1;
        if ((j & 1) == 0)
          ck[mb][nb] = mfma_16x16x32(cq[ks][mb], bd[nb][ks], ck[mb][nb]);
        else if (ALIAS)
          ck[mb][nb] = mfma_16x16x32(cq[2 + ks][mb], bp[nb][ks], ck[mb][nb]);
        else
          cv[mb][nb] = mfma_16x16x32(cq[2 + ks][mb], bp[nb][ks], cv[mb][nb]);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 16 * kh + 4 * g + r;
      const bool v = live && ((valid >> key) & 1u);
      const float pv = v ? fast_exp2(s[r] * scale_log2 - lse2) : 0.f;
      const float dsv = pv * (dp[r] - Dh) * p.scale;
      const bf16x2_t pp = {(__bf16)pv, (__bf16)dsv};
      const uint32_t u = __builtin_bit_cast(uint32_t, pp);
      *(uint16_t*)(pw + PD_P + key * PROW + 2 * hl) = (uint16_t)(u & 0xFFFFu);
      *(uint16_t*)(pw + key * PROW + 2 * hl) = (uint16_t)(u >> 16);
    }
    const int rix = slot_c >= 0 ? (int)(n_wg + (long long)slot_c * n_hg + hg) : (int)blockIdx.x;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int rk = __shfl(rix, 16 * nb + l16);
      uint16_t* dst = buf + (size_t)rk * RW + 32 * wave + 4 * g;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        store4(dst + 16 * mb, ck[mb][nb]);
        if (!ALIAS) store4(dst + D + 16 * mb, cv[mb][nb]);
      }
    }
  };

  wait_all();  // tiles 0 and 1 (this wave's part) and the entries loaded so far
  __syncthreads();
  stage_a(kt0, vt0, valid0, pd);
  lds_barrier();

  auto body = [&](int ti, const char* kc, const char* k1, const char* v1, char* k2, char* v2) {
    uint32_t valid_n2 = 0;
    if (ti + 2 < n_tiles) {
      const int ixv = valid_ix(ix_n2, p.S);
      valid_n2 = (uint32_t)__ballot(ixv >= 0);
      gather_tile<NW>(kl, p.k_stride, ixv, k2, wave, lane);
      if (!ALIAS) gather_tile<NW>(vl, p.v_stride, ixv, v2, wave, lane);
    }
    const int ix_after = load_ix(idx, KT * (ti + 3), p.k, lane);
    const int slot_after = load_slot(sl, KT * (ti + 1), p.k, lane);
    // past the last tile, stage A works on a stale buffer with no valid key and writes zeros
    // that nobody reads
    tile_ops(k1, v1, valid_n1, pd + ((ti + 1) & 1) * PD, kc, pd + (ti & 1) * PD, slot_cur);
    // this wave's gathers of tile ti + 2 and its entry loads have landed: they were issued
    // before the stores, and on this target vector memory loads and stores leave the counter
    // in issue order (the compiler's own waits rely on the same: after a load and a later
    // store, it uses the load's result behind vmcnt(1)); the stores stay in flight
    wait_vm<ALIAS ? 4 : 8>();
    lds_barrier();
    valid_n1 = valid_n2;
    ix_n2 = ix_after;
    slot_cur = slot_after;
  };
  for (int ti = 0; ti < n_tiles; ti += 3) {
    body(ti, kt0, kt1, vt1, kt2, vt2);
    if (ti + 1 < n_tiles) body(ti + 1, kt1, kt2, vt2, kt0, vt0);
    if (ti + 2 < n_tiles) body(ti + 2, kt2, kt0, vt0, kt1, vt1);
  }

  uint16_t* dqr = (uint16_t*)p.dq + (hrow + hl) * D + 128 * kh + 4 * g;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) store4(dqr + 16 * mb, dq[mb]);
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* __restrict__ p, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (long long)gridDim.x * 256)
    p[i] = 0;
}

// range r = blockIdx.x of rows [r*qr, min(n_rows, (r+1)*qr)): rows one after another
__global__ __launch_bounds__(256) void sparse_bwd_rank_kernel(const int32_t* __restrict__ idx,
                                                              int k, int S, int n_rows, int qr,
                                                              int R, int32_t* __restrict__ cnt,
                                                              int32_t* __restrict__ rank) {
  const int r = blockIdx.x;
  const int q1 = min(n_rows, (r + 1) * qr);
  for (int q = r * qr; q < q1; ++q) {
    const int32_t* ir = idx + (size_t)q * k;
    int32_t* rr = rank + (size_t)q * k;
    for (int j = threadIdx.x; j < k; j += 256) {
      const int s = ir[j];
      int rk = -1;
      if (s >= 0 && s < S) rk = atomicAdd(&cnt[(size_t)r * S + s], 1);
      rr[j] = rk;  // uses the returned count: the atomic has been performed before the barrier
    }
    __syncthreads();
  }
}

// The same ranks with the counters of the range in LDS: two 16-bit counters per word (key s
// in half s & 1 of word s / 2), so up to 65536 keys; a count stays below 2^16 because the range
// holds fewer than 2^16 entries.  The range's counts then go to cnt (every key written).
__global__ __launch_bounds__(1024) void sparse_bwd_rank_lds_kernel(
    const int32_t* __restrict__ idx, int k, int S, int n_rows, int qr, int R,
    int32_t* __restrict__ cnt, int32_t* __restrict__ rank) {
  __shared__ uint32_t c16[RANK_LDS_KEYS / 2];
  const int r = blockIdx.x;
  for (int i = threadIdx.x; i < (S + 1) / 2; i += 1024) c16[i] = 0u;
  __syncthreads();
  const int q1 = min(n_rows, (r + 1) * qr);
  for (int q = r * qr; q < q1; ++q) {
    const int32_t* ir = idx + (size_t)q * k;
    int32_t* rr = rank + (size_t)q * k;
    for (int j = threadIdx.x; j < k; j += 1024) {
      const int s = ir[j];
      int rk = -1;
      if (s >= 0 && s < S) {
        const int sh = 16 * (s & 1);
        rk = (int)((atomicAdd(&c16[s >> 1], 1u << sh) >> sh) & 0xFFFFu);
      }
      rr[j] = rk;
    }
    __syncthreads();
  }
  for (int s = threadIdx.x; s < S; s += 1024)
    cnt[(size_t)r * S + s] = (int32_t)((c16[s >> 1] >> (16 * (s & 1))) & 0xFFFFu);
}

// exclusive scan of 16 * NT values in place (global or LDS); their total to *total
template <int NT>
__device__ __forceinline__ void block_scan16(int32_t* __restrict__ data, long long n,
                                             long long base, int32_t* total) {
  __shared__ int32_t wsum[NT / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long long i0 = base + 16ll * threadIdx.x;
  int v[16];
  if (i0 + 16 <= n) {  // 64 aligned bytes
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int4 x = *(const int4*)(data + i0 + 4 * c);
      v[4 * c] = x.x;
      v[4 * c + 1] = x.y;
      v[4 * c + 2] = x.z;
      v[4 * c + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = i0 + e < n ? data[i0 + e] : 0;
  }
  int sum = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int x = v[e];
    v[e] = sum;
    sum += x;
  }
  int x = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int pre = 0;
  for (int i = 0; i < w; ++i) pre += wsum[i];
  const int ex = pre + x - sum;
  if (i0 + 16 <= n) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *(int4*)(data + i0 + 4 * c) = make_int4(v[4 * c] + ex, v[4 * c + 1] + ex, v[4 * c + 2] + ex,
                                              v[4 * c + 3] + ex);
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (i0 + e < n) data[i0 + e] = v[e] + ex;
  }
  if (threadIdx.x == NT - 1) *total = pre + x;
}

// Counts are stored range-major (data[r * S + s], as counted); the scan runs key-major.  A
// block takes kb whole keys (kb * R <= 4096 counters): it reads them along the keys (coalesced
// runs), scans them key-major in LDS and writes them back; the blocks' totals go to bsum.
__global__ __launch_bounds__(256) void scan_keys_kernel(int32_t* __restrict__ data, int S, int R,
                                                        int kb, int32_t* __restrict__ bsum) {
  __shared__ __attribute__((aligned(16))) int32_t sv[SCAN_BLOCK];
  const int s0 = blockIdx.x * kb, ns = min(kb, S - s0), n = ns * R;
  for (int j = threadIdx.x; j < n; j += 256) {
    const int sl = j % ns, r = j / ns;
    sv[sl * R + r] = data[(size_t)r * S + s0 + sl];
  }
  __syncthreads();
  block_scan16<256>(sv, n, 0, bsum + blockIdx.x);
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += 256) {
    const int sl = j % ns, r = j / ns;
    data[(size_t)r * S + s0 + sl] = sv[sl * R + r];
  }
}

// one workgroup: the block totals (at most 16384) scanned in place, the grand total after them
__global__ __launch_bounds__(1024) void scan_top_kernel(int32_t* __restrict__ bsum, int nblk) {
  block_scan16<1024>(bsum, nblk, 0, bsum + nblk);
}

// offset of the counter of (key s, range r): its exclusive sum within its block of kb keys
// plus the blocks before it
__device__ __forceinline__ int scan_at(const int32_t* off, const int32_t* bsum, int S, int kb,
                                       int s, int r) {
  return off[(size_t)r * S + s] + bsum[s / kb];
}

__global__ __launch_bounds__(256) void sparse_bwd_slot_kernel(const int32_t* __restrict__ idx,
                                                              long long n, int k, int S, int qr,
                                                              int kb, const int32_t* __restrict__ off,
                                                              const int32_t* __restrict__ bsum,
                                                              int32_t* __restrict__ rank) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (long long)gridDim.x * 256) {
    const int rk = rank[i];
    if (rk < 0) continue;
    const int r = (int)(i / k) / qr;
    rank[i] = scan_at(off, bsum, S, kb, idx[i], r) + rk;
  }
}

// One wave per key: its slots [off(s, 0), off(s + 1, 0)) in order, then the accumulator.
// mode 0: acc = sum; 1: acc += sum; 2: out = acc + sum; 3: out = sum.
template <bool ALIAS>
__global__ __launch_bounds__(256) void sparse_bwd_reduce_kernel(
    const uint16_t* __restrict__ buf, long long row_base, const int32_t* __restrict__ off,
    const int32_t* __restrict__ bsum, const int32_t* __restrict__ total, int kb, int S, int n_hg,
    float* __restrict__ acc, int mode,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
  constexpr int RW = ALIAS ? D : 2 * D;
  constexpr int PER = RW / 64;  // columns per lane
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= S) return;
  const int lane = threadIdx.x & 63;
  const long long a = row_base + (long long)scan_at(off, bsum, S, kb, s, 0) * n_hg;
  const long long e =
      row_base + (long long)(s + 1 < S ? scan_at(off, bsum, S, kb, s + 1, 0) : *total) * n_hg;
  float sum[PER];
#pragma unroll
  for (int c = 0; c < PER; ++c) sum[c] = 0.f;
  const uint16_t* src = buf + PER * lane;
  auto add = [&](const uint4& u) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int c = 0; c < PER / 2; ++c) {
      sum[2 * c] += __uint_as_float(w[c] << 16);
      sum[2 * c + 1] += __uint_as_float(w[c] & 0xFFFF0000u);
    }
  };
  auto load = [&](long long i) {
    if constexpr (ALIAS) {
      const uint2 x = *(const uint2*)(src + (size_t)i * RW);
      return make_uint4(x.x, x.y, 0u, 0u);
    }
    return *(const uint4*)(src + (size_t)i * RW);
  };
  long long i = a;
  for (; i + 8 <= e; i += 8) {
    uint4 u[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) u[t] = load(i + t);
#pragma unroll
    for (int t = 0; t < 8; ++t) add(u[t]);
  }
  for (; i < e; ++i) add(load(i));
  float* ac = acc + (size_t)s * RW + PER * lane;
  if (mode == 1 || mode == 2) {
#pragma unroll
    for (int c = 0; c < PER; ++c) sum[c] = ac[c] + sum[c];
  }
  if (mode <= 1) {
#pragma unroll
    for (int c = 0; c < PER; ++c) ac[c] = sum[c];
    return;
  }
  uint32_t o[PER / 2];
#pragma unroll
  for (int c = 0; c < PER / 2; ++c) o[c] = pack_bf16x2(sum[2 * c], sum[2 * c + 1]);
  if constexpr (ALIAS) {
    *(uint2*)(dk + (size_t)s * D + PER * lane) = make_uint2(o[0], o[1]);
  } else {
    uint16_t* dst =
        lane < 32 ? dk + (size_t)s * D + PER * lane : dv + (size_t)s * D + PER * (lane - 32);
    *(uint4*)dst = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct SbwdPlan {
  bool alias;
  int rw, n_hg, qc, qr, rmax;
  int chunks;  // per sequence
  size_t o_cnt, o_bsum, o_rank, o_buf, o_acc, bytes;
};

// layout for chunks of qc query rows
size_t sbwd_layout(const SparseBwdParams& p, long long qc, SbwdPlan& pl) {
  pl.alias = p.dv == nullptr;
  pl.rw = pl.alias ? D : 2 * D;
  pl.n_hg = p.H / 64;
  // a scan block holds SCAN_BLOCK / R whole keys, and the top level at most 16384 blocks
  const long long kmin = (p.S + 16383) / 16384;
  const long long rcap = std::max(1ll, SCAN_BLOCK / kmin);
  long long rmax =
      std::max(1ll, std::min(std::min((long long)MAX_RANGES, MAX_COUNTERS / p.S), rcap));
  rmax = std::min(rmax, qc);
  pl.qr = (int)((qc + rmax - 1) / rmax);
  // ranges short enough for the 16-bit LDS counters when the keys fit (a few more ranges)
  if (p.S <= RANK_LDS_KEYS && (long long)pl.qr * p.k >= 65536 && p.k < 65536) {
    const int q2 = std::max(1, 65535 / p.k);
    if ((qc + q2 - 1) / q2 <= rcap) pl.qr = q2;
  }
  pl.rmax = (int)((qc + pl.qr - 1) / pl.qr);
  pl.qc = (int)qc;
  pl.chunks = (int)((p.Tq + qc - 1) / qc);
  const long long counters = (long long)p.S * pl.rmax;
  const long long nblk = (p.S + std::max(1ll, SCAN_BLOCK / pl.rmax) - 1) /
                         std::max(1ll, SCAN_BLOCK / pl.rmax);
  size_t o = 0;
  pl.o_cnt = o;
  o = align256(o + (size_t)counters * 4);
  pl.o_bsum = o;
  o = align256(o + (size_t)(nblk + 1) * 4);
  pl.o_rank = o;
  o = align256(o + (size_t)qc * p.k * 4);
  pl.o_buf = o;
  o = align256(o + ((size_t)qc * pl.n_hg + (size_t)qc * p.k * pl.n_hg) * pl.rw * 2);
  pl.o_acc = o;
  if (pl.chunks > 1) o = align256(o + (size_t)p.S * pl.rw * 4);
  pl.bytes = o;
  return o;
}

// The largest chunk that fits `avail` bytes, at most the one whose contributions fill the
// default budget (and at most one sequence).
SbwdPlan sbwd_plan(const SparseBwdParams& p, size_t avail) {
  SbwdPlan pl;
  const size_t row_bytes = (size_t)p.k * (p.H / 64) * (p.dv == nullptr ? D : 2 * D) * 2;
  long long qc = (long long)(BUF_BUDGET / std::max<size_t>(row_bytes, 1));
  qc = std::max(1ll, std::min(qc, (long long)p.Tq));
  if (sbwd_layout(p, qc, pl) <= avail) return pl;
  long long lo = 1, hi = qc - 1;  // below qc every size includes the accumulator: monotone
  while (lo < hi) {
    const long long mid = (lo + hi + 1) / 2;
    if (sbwd_layout(p, mid, pl) <= avail)
      lo = mid;
    else
      hi = mid - 1;
  }
  sbwd_layout(p, lo, pl);
  return pl;
}

}  // namespace

size_t sparse_bwd_workspace(const SparseBwdParams& p) { return sbwd_plan(p, SIZE_MAX).bytes; }

// one row at a time, unless the default (a single chunk needs no accumulator) is smaller
size_t sparse_bwd_min_workspace(const SparseBwdParams& p) {
  SbwdPlan pl;
  return std::min(sbwd_layout(p, 1, pl), sparse_bwd_workspace(p));
}

hipError_t launch_sparse_bwd(const SparseBwdParams& p, hipStream_t stream) {
  const SbwdPlan pl = sbwd_plan(p, p.ws_bytes);
  char* ws = (char*)p.ws;
  int32_t* cnt = (int32_t*)(ws + pl.o_cnt);
  int32_t* bsum = (int32_t*)(ws + pl.o_bsum);
  int32_t* rank = (int32_t*)(ws + pl.o_rank);
  uint16_t* buf = (uint16_t*)(ws + pl.o_buf);
  float* acc = (float*)(ws + pl.o_acc);
  for (int b = 0; b < p.B; ++b) {
    uint16_t* dk = (uint16_t*)p.dk + (size_t)b * p.S * D;
    uint16_t* dv = pl.alias ? nullptr : (uint16_t*)p.dv + (size_t)b * p.S * D;
    for (int c = 0; c < pl.chunks; ++c) {
      const int t0 = c * pl.qc, n_rows = std::min(pl.qc, p.Tq - t0);
      const long long row0 = (long long)b * p.Tq + t0;
      const int R = (n_rows + pl.qr - 1) / pl.qr;
      const long long counters = (long long)p.S * R;
      const int kb = (int)std::max(1ll, SCAN_BLOCK / R);  // keys per scan block
      const long long nblk = (p.S + kb - 1) / kb;
      const int32_t* idx = p.idx + (size_t)row0 * p.k;
      const long long n_pairs = (long long)n_rows * p.k;
      if (p.S <= RANK_LDS_KEYS && (long long)pl.qr * p.k < 65536) {
        hipLaunchKernelGGL(sparse_bwd_rank_lds_kernel, dim3(R), dim3(1024), 0, stream, idx, p.k,
                           p.S, n_rows, pl.qr, R, cnt, rank);
      } else {
        hipLaunchKernelGGL(fill_i32_kernel,
                           dim3((unsigned)std::min(4096ll, (counters + 255) / 256)), dim3(256), 0,
                           stream, cnt, counters);
        hipLaunchKernelGGL(sparse_bwd_rank_kernel, dim3(R), dim3(256), 0, stream, idx, p.k, p.S,
                           n_rows, pl.qr, R, cnt, rank);
      }
      hipLaunchKernelGGL(scan_keys_kernel, dim3((unsigned)nblk), dim3(256), 0, stream, cnt, p.S,
                         R, kb, bsum);
      hipLaunchKernelGGL(scan_top_kernel, dim3(1), dim3(1024), 0, stream, bsum, (int)nblk);
      hipLaunchKernelGGL(sparse_bwd_slot_kernel,
                         dim3((unsigned)std::min(8192ll, (n_pairs + 255) / 256)), dim3(256), 0,
                         stream, idx, n_pairs, p.k, p.S, pl.qr, kb, cnt, bsum, rank);
      const unsigned grid = (unsigned)n_rows * pl.n_hg;
      if (pl.alias)
        hipLaunchKernelGGL(sparse_bwd_kernel<true>, dim3(grid), dim3(64 * NW), 0, stream, p,
                           row0, rank, buf);
      else
        hipLaunchKernelGGL(sparse_bwd_kernel<false>, dim3(grid), dim3(64 * NW), 0, stream, p,
                           row0, rank, buf);
      const int mode = pl.chunks == 1 ? 3 : c == 0 ? 0 : c + 1 < pl.chunks ? 1 : 2;
      const dim3 rgrid((unsigned)((p.S + 3) / 4));
      if (pl.alias)
        hipLaunchKernelGGL(sparse_bwd_reduce_kernel<true>, rgrid, dim3(256), 0, stream, buf,
                           (long long)grid, cnt, bsum, bsum + nblk, kb, p.S, pl.n_hg, acc, mode, dk,
                           dv);
      else
        hipLaunchKernelGGL(sparse_bwd_reduce_kernel<false>, rgrid, dim3(256), 0, stream, buf,
                           (long long)grid, cnt, bsum, bsum + nblk, kb, p.S, pl.n_hg, acc, mode, dk,
                           dv);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace lgsa
