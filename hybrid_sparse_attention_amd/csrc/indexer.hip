// DSA lightweight indexer and per-query top-k (ERNIE 5.5 Flash Base release blog, section
// 2.1: an indexer scores the past positions of each query; core attention then runs only on
// the k highest-scoring positions).  Score form taken here:
//   score(t, s) = sum_h w[t, h] * max(0, <q_I[t, h], k_I[s]>),  s <= t, in fp32.
// Selection is exact integer work on an order-preserving 32-bit image of each fp32 score
// (-0.0 mapped to +0.0 first): a most-significant-digit radix select finds the k-th largest
// key K* and how many keys equal to K* are needed, then one ascending pass keeps every key
// above K* and the lowest-positioned keys equal to K*, which writes the kept positions in
// ascending order.  Block-wide ranks come from wavefront ballots.
//
// Prefill (many queries per sequence): scores come from fp32 MFMA (v_mfma_f32_32x32x2f32,
// rows = (query, indexer head), columns = keys, contraction = the 64 indexer dims), so each
// key tile in LDS serves 64 queries; they are written as keys to the workspace, a chunk of up
// to 2048 queries at a time, and a 1024-thread workgroup per query selects.
// Decode (few queries, long context): one workgroup per (query, 16384-position segment)
// streams its key rows once, scores them with fp32 FMA, selects the segment's top-k in LDS and
// writes them as a candidate list in ascending position (the union of the top-k sets of
// disjoint parts contains the top k of the whole).  Each full segment also reports a key that
// bounds the row's k-th largest from below; a filter keeps the candidates at or above the
// bound, which leaves a few thousand, and one workgroup per query selects the top k among
// them.  Position order is kept throughout, so the lower-index rule stays exact.
#include "common.h"
#include "kernels.h"

namespace lgsa {

namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Number of keys visible to the query at position t: keys s < (t + 1) / block, at most
// `bound` (the keys that exist and the rows' promised range); none for t < 0.
__device__ __forceinline__ int visible_keys(int t, int block, int bound) {
  return t >= 0 ? min((t + 1) / block, bound) : 0;
}

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 counts as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sums, in thread order, of two per-thread counts, and their totals.
// `wsum` holds 2 * NT / 64 ints.  Contains two workgroup barriers.
template <int NT>
__device__ __forceinline__ void block_scan2(int a, int b, int& a_ex, int& b_ex, int& a_tot,
                                            int& b_tot, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int ai = a, bi = b;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int ya = __shfl_up(ai, off), yb = __shfl_up(bi, off);
    if (lane >= off) {
      ai += ya;
      bi += yb;
    }
  }
  if (lane == 63) {
    wsum[2 * wave] = ai;
    wsum[2 * wave + 1] = bi;
  }
  __syncthreads();
  int pa = 0, pb = 0, ta = 0, tb = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int ca = wsum[2 * w], cb = wsum[2 * w + 1];
    pa += w < wave ? ca : 0;
    pb += w < wave ? cb : 0;
    ta += ca;
    tb += cb;
  }
  a_ex = pa + ai - a;
  b_ex = pb + bi - b;
  a_tot = ta;
  b_tot = tb;
  __syncthreads();
}

// Selection of the digit that holds the kr-th largest key from a digit histogram (one private
// copy per wave, hist: NT / 64 x 256 counters): thread t < 256 takes digit 255 - t, the counts
// are scanned in that (descending) order across the first four waves, and the one thread whose
// inclusive count first reaches kr writes sh[0] = digit, sh[1] = kr - (keys in larger digits)
// and sh[2] = keys in the digit.
template <int NT>
__device__ void pick_digit(int kr, const uint32_t* hist, int* sh, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int c = 0, incl = 0;
  if (tid < 256) {
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) c += (int)hist[w * 256 + 255 - tid];
    incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
  }
  __syncthreads();
  if (tid < 256) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    incl += before;
    const int excl = incl - c;
    if (incl >= kr && excl < kr) {
      sh[0] = 255 - tid;
      sh[1] = kr - excl;
      sh[2] = c;
    }
  }
  __syncthreads();
}

// Histogram of one radix digit (bits shift .. shift + 7) over the keys whose bits above the
// digit equal `prefix`, then pick_digit.
template <int NT, class Get>
__device__ void radix_digit(const Get& get, int n, uint32_t prefix, uint32_t hi_mask, int shift,
                            int kr, uint32_t* hist, int* sh, int* wsum) {
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int x = tid; x < (NT / 64) * 256; x += NT) hist[x] = 0u;
  __syncthreads();
  uint32_t* mine = hist + wave * 256;
  constexpr int PER = 8;  // loads in flight per thread; consecutive threads read consecutive keys
  for (int c0 = tid; c0 < n; c0 += NT * PER) {
    uint32_t u[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) u[j] = c0 + j * NT < n ? get(c0 + j * NT) : 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (c0 + j * NT < n && (u[j] & hi_mask) == prefix)
        atomicAdd(&mine[(u[j] >> shift) & 255u], 1u);
  }
  __syncthreads();
  pick_digit<NT>(kr, hist, sh, wsum);
}

// Finds the k-th largest key K* among get(0..n-1) (1 <= k <= n) and the number of keys equal
// to K* that belong to the top k; 8-bit digits, most significant first.
template <int NT, class Get>
__device__ void radix_threshold(const Get& get, int n, int k, uint32_t* hist, int* sh,
                                int* wsum, uint32_t& kstar, int& need_eq) {
  uint32_t prefix = 0u;
  int kr = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    const uint32_t hi_mask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
    radix_digit<NT>(get, n, prefix, hi_mask, shift, kr, hist, sh, wsum);
    prefix |= (uint32_t)sh[0] << shift;
    kr = sh[1];
    __syncthreads();  // sh is rewritten by the next digit
  }
  kstar = prefix;
  need_eq = kr;
}

constexpr int EMIT_PER = 8;

// Ascending pass: emit(slot, i, key) for every i whose key is above K*, and for the first
// need_eq (in index order) whose key equals K*.  Each thread takes EMIT_PER consecutive
// indices of a chunk of NT * EMIT_PER, so one block scan per chunk orders the whole chunk.
// With a `stage` buffer (NT * EMIT_PER keys of LDS) each chunk is first copied there with
// coalesced reads (for keys in global memory); without one, get() is read directly (LDS).
template <int NT, class Get, class Emit>
__device__ void emit_topk(const Get& get, int n, uint32_t kstar, int need_eq, int* wsum,
                          uint32_t* stage, const Emit& emit) {
  constexpr int PER = EMIT_PER;
  int base = 0, eq_seen = 0;
  for (int c0 = 0; c0 < n; c0 += NT * PER) {
    if (stage != nullptr) {
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int x = c0 + j * NT + (int)threadIdx.x;
        stage[j * NT + threadIdx.x] = x < n ? get(x) : 0u;
      }
      __syncthreads();
    }
    const int i0 = c0 + (int)threadIdx.x * PER;
    uint32_t u[PER];
    int n_gt = 0, n_eq = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      u[j] = i0 + j < n ? (stage != nullptr ? stage[threadIdx.x * PER + j] : get(i0 + j)) : 0u;
      n_gt += (i0 + j < n && u[j] > kstar) ? 1 : 0;
      n_eq += (i0 + j < n && u[j] == kstar) ? 1 : 0;
    }
    int gt_ex, eq_ex, gt_tot, eq_tot;
    block_scan2<NT>(n_gt, n_eq, gt_ex, eq_ex, gt_tot, eq_tot, wsum);
    // equal keys of earlier threads in this chunk that are kept
    const int eq_keep_before = min(max(need_eq - eq_seen, 0), eq_ex);
    int slot = base + gt_ex + eq_keep_before;
    int eq_rank = eq_seen + eq_ex;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (i0 + j >= n) continue;
      bool sel = u[j] > kstar;
      if (u[j] == kstar) {
        sel = eq_rank < need_eq;
        ++eq_rank;
      }
      if (sel) emit(slot++, i0 + j, u[j]);
    }
    base += gt_tot + min(max(need_eq - eq_seen, 0), eq_tot);
    eq_seen += eq_tot;
  }
}

// ------------------------------------------------------------------------------ prefill
constexpr int SC_Q = 64;     // queries per workgroup (4 waves x 16)
constexpr int SC_KT = 64;    // keys per LDS tile
constexpr int SC_CH = 512;   // keys per workgroup
constexpr int SK_LD = 64 + 4;

typedef float f32x16v __attribute__((ext_vector_type(16)));

// Scores of queries [i_begin, i_begin + nq) of sequence b against keys, written as ordered
// keys to ws[(i - i_begin) * s_ld + s].  Products on v_mfma_f32_32x32x2f32: a wave's rows are
// (query, indexer head) pairs, 8 queries x 4 heads per 32-row block, two blocks per wave; the
// columns are 32 keys of the tile; the contraction runs over the 64 indexer dims, 2 per step.
// A lane's accumulator then holds the four heads of one (query, key) pair in consecutive
// registers, so the weighted head sum is lane-local.  Key tiles are double buffered through
// registers: the next tile's loads are in flight while the current one is used.
__global__ __launch_bounds__(256) void index_scores_kernel(IndexParams p, int b, int i_begin,
                                                           int nq, uint32_t* ws, int s_ld) {
  __shared__ __attribute__((aligned(16))) float sk[2][SC_KT * SK_LD];
  __shared__ __attribute__((aligned(16))) float sw[SC_Q * 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int i0 = i_begin + blockIdx.x * SC_Q;
  const int i_stop = i_begin + nq;
  const int pos = p.pos0[b];
  const int kbound = min(p.S, (p.max_pos + 1) / p.block);
  // keys visible to the workgroup's last query bound the keys scored (earlier queries' rows
  // get scores past their own visible range, which their selection never reads)
  const int n_hi = visible_keys(pos + min(i_stop, i0 + SC_Q) - 1, p.block, kbound);
  const int s_begin = blockIdx.y * SC_CH;
  if (s_begin >= n_hi) return;
  const int s_end = min(n_hi, s_begin + SC_CH);

  {  // head weights of the workgroup's queries: sw[4q + h]
    const int i = i0 + (tid >> 2), h = tid & 3;
    sw[tid] = (i < i_stop && h < p.Hi) ? p.w_idx[((size_t)b * p.Tq + i) * p.Hi + h] : 0.f;
  }
  // A operands: row l32 of block mb is (query 16 wave + 8 mb + l32 / 4, head l32 % 4); step ks
  // takes dim 2 ks + hi
  float a[2][32];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int i = i0 + 16 * wave + 8 * mb + (l32 >> 2), hq = l32 & 3;
    const bool ok = i < i_stop && hq < p.Hi;
    const float* qr = p.q_idx + (((size_t)b * p.Tq + (ok ? i : 0)) * p.Hi + (ok ? hq : 0)) * 64;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) a[mb][ks] = ok ? qr[2 * ks + hi] : 0.f;
  }
  const float* kb = p.k_idx + (size_t)b * p.S * 64;
  float4 kv[4];
  auto load_tile = [&](int s0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u;  // float4 index in the 64 x 64 tile
      const int key = c >> 4, dim = (c & 15) * 4;
      kv[u] = s0 + key < s_end ? *(const float4*)(kb + (size_t)(s0 + key) * 64 + dim)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store_tile = [&](float* dst) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u;
      *(float4*)(&dst[(c >> 4) * SK_LD + (c & 15) * 4]) = kv[u];
    }
  };
  load_tile(s_begin);
  store_tile(sk[0]);
  __syncthreads();
  int buf = 0;
  for (int s0 = s_begin; s0 < s_end; s0 += SC_KT) {
    const bool more = s0 + SC_KT < s_end;
    if (more) load_tile(s0 + SC_KT);
    const float* skc = sk[buf];
    f32x16v acc[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x16v{};
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) {
      float bv[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) bv[nb] = skc[(32 * nb + l32) * SK_LD + 2 * ks + hi];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[mb][ks], bv[nb], acc[mb][nb],
                                                             0, 0, 0);
    }
    // acc[mb][nb][4j + h]: query 16 wave + 8 mb + 2j + hi, head h, key s0 + 32 nb + l32
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ql = 16 * wave + 8 * mb + 2 * j + hi;
        const int i = i0 + ql;
        const float4 w4 = *(const float4*)(sw + 4 * ql);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int s = s0 + 32 * nb + l32;
          float sc = 0.f;
          sc = fmaf(w4.x, fmaxf(acc[mb][nb][4 * j + 0], 0.f), sc);
          sc = fmaf(w4.y, fmaxf(acc[mb][nb][4 * j + 1], 0.f), sc);
          sc = fmaf(w4.z, fmaxf(acc[mb][nb][4 * j + 2], 0.f), sc);
          sc = fmaf(w4.w, fmaxf(acc[mb][nb][4 * j + 3], 0.f), sc);
          if (i < i_stop && s < s_end) ws[(size_t)(i - i_begin) * s_ld + s] = order_key(sc);
        }
      }
    if (more) store_tile(sk[buf ^ 1]);
    __syncthreads();
    buf ^= 1;
  }
}

constexpr int SEL_NT = 1024;
constexpr int SEL_N16 = 65536;  // rows of up to this many keys keep 16-bit key images in LDS
constexpr int SEL_CAP = 2048;   // keys of the threshold's 16-bit bin held in full

// One workgroup per query row.  Rows of at most SEL_N16 keys: one pass over the row in global
// memory stores the upper 16 bits of every key in LDS and counts its upper 12 bits in one
// shared 4096-bin histogram (scores crowd into a few exponents: 8-bit digits would send most
// of a wave's atomic adds to the same counter); the next 4 bits are counted from LDS; the keys whose upper 16 bits equal the threshold's (the bin the
// k-th largest key falls in) are then read in full, in position order, into LDS, where the
// last two digits are resolved; the selection is emitted from LDS.  The row is read from
// global memory once, plus the threshold bin's keys.  Longer rows, and rows whose threshold
// bin holds more than SEL_CAP keys, take all four digits and the emission over global memory.
__global__ __launch_bounds__(SEL_NT) void index_select_rows_kernel(IndexParams p, int b,
                                                                   int i_begin,
                                                                   const uint32_t* ws,
                                                                   int s_ld) {
  __shared__ __attribute__((aligned(16))) uint16_t k16[SEL_N16];
  __shared__ uint32_t hist[(SEL_NT / 64) * 256];
  __shared__ uint32_t cand[SEL_CAP];
  __shared__ int sh[3];
  __shared__ int wsum[2 * SEL_NT / 64];
  const int tid = threadIdx.x;
  const int i = i_begin + blockIdx.x;
  const int n = visible_keys(p.pos0[b] + i, p.block, min(p.S, (p.max_pos + 1) / p.block));
  int32_t* out = p.idx_out + ((size_t)b * p.Tq + i) * p.k;
  if (n <= p.k) {
    for (int j = tid; j < p.k; j += SEL_NT) out[j] = j < n ? j : -1;
    return;
  }
  const uint32_t* row = ws + (size_t)blockIdx.x * s_ld;
  auto get = [&](int x) { return row[x]; };
  auto emit_global = [&](uint32_t prefix, uint32_t hi_mask, int shift, int kr) {
    // remaining digits and the emission over global memory (k16 serves as the staging buffer)
    for (; shift >= 0; shift -= 8) {
      radix_digit<SEL_NT>(get, n, prefix, hi_mask, shift, kr, hist, sh, wsum);
      prefix |= (uint32_t)sh[0] << shift;
      kr = sh[1];
      hi_mask = 0xFFFFFFFFu << shift;
      __syncthreads();
    }
    emit_topk<SEL_NT>(get, n, prefix, kr, wsum, (uint32_t*)k16,
                      [&](int slot, int x, uint32_t) { out[slot] = x; });
  };
  if (n > SEL_N16) {
    emit_global(0u, 0u, 24, p.k);
    return;
  }

  // bits 31..20 (one shared histogram of 4096 counters in the space of the per-wave ones),
  // with the 16-bit images stored on the way
  constexpr int NB = 4096, BPT = NB / SEL_NT;
  static_assert(NB <= (SEL_NT / 64) * 256, "the 12-bit histogram reuses the digit histograms");
  for (int x = tid; x < NB; x += SEL_NT) hist[x] = 0u;
  __syncthreads();
  {
    constexpr int PER = 8;
    for (int c0 = tid; c0 < n; c0 += SEL_NT * PER) {
      uint32_t u[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) u[j] = c0 + j * SEL_NT < n ? row[c0 + j * SEL_NT] : 0u;
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (c0 + j * SEL_NT < n) {
          k16[c0 + j * SEL_NT] = (uint16_t)(u[j] >> 16);
          atomicAdd(&hist[u[j] >> 20], 1u);
        }
    }
  }
  __syncthreads();
  {
    // thread t covers bins NB - 1 - BPT t - j (j < BPT), the bins in descending order
    int cnt[BPT], tot = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      cnt[j] = (int)hist[NB - 1 - BPT * tid - j];
      tot += cnt[j];
    }
    int ex, z_ex, all, z_tot;
    block_scan2<SEL_NT>(tot, 0, ex, z_ex, all, z_tot, wsum);
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      if (ex < p.k && ex + cnt[j] >= p.k) {
        sh[0] = NB - 1 - BPT * tid - j;
        sh[1] = p.k - ex;
      }
      ex += cnt[j];
    }
  }
  __syncthreads();
  const uint32_t d1 = (uint32_t)sh[0];  // upper 12 bits of the k-th largest key
  const int kr1 = sh[1];
  __syncthreads();
  // bits 19..16 from LDS (an 8-bit digit of the images whose upper 4 bits the prefix fixes)
  auto get16 = [&](int x) { return (uint32_t)k16[x]; };
  radix_digit<SEL_NT>(get16, n, d1 << 4, 0xFFF0u, 0, kr1, hist, sh, wsum);
  const uint32_t p16 = (d1 << 4) | ((uint32_t)sh[0] & 15u);  // upper 16 bits of the k-th key
  const int kr2 = sh[1];                              // keys needed from that bin
  const int c16 = sh[2];                              // keys in that bin
  __syncthreads();
  if (c16 > SEL_CAP) {
    emit_global(p16 << 16, 0xFFFF0000u, 8, kr2);
    return;
  }

  // the bin's keys in full, in position order: thread t of a chunk takes positions
  // c0 + 8t .. c0 + 8t + 7
  constexpr int PER = EMIT_PER;
  static_assert(PER == 8, "one 16-byte LDS read per thread and chunk");
  int cbase = 0;
  for (int c0 = 0; c0 < n; c0 += SEL_NT * PER) {
    const int i0 = c0 + tid * PER;
    const uint4 w4 = *(const uint4*)(k16 + min(i0, SEL_N16 - PER));
    const uint32_t wv[4] = {w4.x, w4.y, w4.z, w4.w};
    int nc = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t h = (wv[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      nc += (i0 + j < n && h == p16) ? 1 : 0;
    }
    int c_ex, z_ex, c_tot, z_tot;
    block_scan2<SEL_NT>(nc, 0, c_ex, z_ex, c_tot, z_tot, wsum);
    int slot = cbase + c_ex;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t h = (wv[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      if (i0 + j < n && h == p16) cand[slot++] = row[i0 + j];
    }
    cbase += c_tot;
  }
  __syncthreads();
  // digits 3 and 4 over the bin's keys
  auto getc = [&](int x) { return cand[x]; };
  uint32_t kstar = p16 << 16;
  int kr = kr2;
  for (int shift = 8; shift >= 0; shift -= 8) {
    radix_digit<SEL_NT>(getc, c16, kstar, 0xFFFFFFFFu << (shift + 8), shift, kr, hist, sh, wsum);
    kstar |= (uint32_t)sh[0] << shift;
    kr = sh[1];
    __syncthreads();
  }
  const int need_eq = kr;

  // emission from LDS: keys above the bin are kept, keys below it dropped; a key of the bin
  // (its full value the next in `cand`) is kept if above K*, or equal to K* and among the
  // first need_eq such
  int base = 0, eq_seen = 0;
  cbase = 0;
  for (int c0 = 0; c0 < n; c0 += SEL_NT * PER) {
    const int i0 = c0 + tid * PER;
    const uint4 w4 = *(const uint4*)(k16 + min(i0, SEL_N16 - PER));
    const uint32_t wv[4] = {w4.x, w4.y, w4.z, w4.w};
    uint32_t h[PER];
    int nc = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      h[j] = i0 + j < n ? (wv[j >> 1] >> (16 * (j & 1))) & 0xFFFFu : 0u;
      nc += (i0 + j < n && h[j] == p16) ? 1 : 0;
    }
    int c_ex, z_ex, c_tot, z_tot;
    block_scan2<SEL_NT>(nc, 0, c_ex, z_ex, c_tot, z_tot, wsum);
    // full keys: above the bin -> above K*, below it -> below K*, in it -> from cand
    uint32_t u[PER];
    int ci = cbase + c_ex, n_gt = 0, n_eq = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      u[j] = h[j] > p16 ? 0xFFFFFFFFu : (h[j] == p16 && i0 + j < n ? cand[ci++] : 0u);
      n_gt += (i0 + j < n && u[j] > kstar) ? 1 : 0;
      n_eq += (i0 + j < n && u[j] == kstar) ? 1 : 0;
    }
    cbase += c_tot;
    int gt_ex, eq_ex, gt_tot, eq_tot;
    block_scan2<SEL_NT>(n_gt, n_eq, gt_ex, eq_ex, gt_tot, eq_tot, wsum);
    const int eq_keep_before = min(max(need_eq - eq_seen, 0), eq_ex);
    int slot = base + gt_ex + eq_keep_before;
    int eq_rank = eq_seen + eq_ex;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (i0 + j >= n) continue;
      bool sel = u[j] > kstar;
      if (u[j] == kstar) {
        sel = eq_rank < need_eq;
        ++eq_rank;
      }
      if (sel) out[slot++] = i0 + j;
    }
    base += gt_tot + min(max(need_eq - eq_seen, 0), eq_tot);
    eq_seen += eq_tot;
  }
}

// ------------------------------------------------------------------------------ decode
constexpr int SEG = 16384;       // positions per segment (>= the largest supported k)
constexpr int DEC_NT = 256;

// One workgroup per (query row, segment of SEG positions): every lane scores one key row per
// batch of 64 (its 256 bytes read straight into registers, the next batch's rows already in
// flight while this one is scored, the query from LDS), the segment's scores stay in LDS as
// ordered keys, and the segment's top k are written as candidates in ascending position,
// with their count.
__global__ __launch_bounds__(DEC_NT) void index_segment_kernel(IndexParams p, int n_seg,
                                                               uint32_t* cand_key,
                                                               int32_t* cand_pos,
                                                               int* cand_cnt,
                                                               uint32_t* lo_key) {
  __shared__ uint32_t skey[SEG];
  __shared__ __attribute__((aligned(16))) float sq[4 * 64 + 4];
  __shared__ uint32_t hist[(DEC_NT / 64) * 256];
  __shared__ int sh[3];
  __shared__ int wsum[2 * DEC_NT / 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = blockIdx.x / n_seg, seg = blockIdx.x % n_seg;  // r = b * Tq + i
  const int b = r / p.Tq;
  const int n = visible_keys(p.pos0[b] + r % p.Tq, p.block, min(p.S, (p.max_pos + 1) / p.block));
  const int seg_start = seg * SEG;
  if (n <= p.k) return;  // short rows are finished by the last reduction
  if (seg_start >= n) {  // a segment past the row's last position contributes nothing
    if (tid == 0) cand_cnt[(size_t)r * n_seg + seg] = 0;
    return;
  }
  const int seg_n = min(SEG, n - seg_start);
  if (tid == 0) cand_cnt[(size_t)r * n_seg + seg] = min(seg_n, p.k);
  for (int x = tid; x < 4 * 64; x += DEC_NT) {
    const int h = x >> 6;
    sq[x] = h < p.Hi ? p.q_idx[((size_t)r * p.Hi + h) * 64 + (x & 63)] : 0.f;
  }
  if (tid < 4) sq[256 + tid] = tid < p.Hi ? p.w_idx[(size_t)r * p.Hi + tid] : 0.f;
  __syncthreads();
  const float* kb = p.k_idx + ((size_t)b * p.S + seg_start) * 64;
  const int n_batch = (seg_n + 63) / 64;
  float4 kn[16];
  auto load = [&](int bi) {
    const int key = min(bi * 64 + lane, seg_n - 1);  // lanes past the end reread the last row
    const float4* src = (const float4*)(kb + (size_t)key * 64);
#pragma unroll
    for (int j = 0; j < 16; ++j) kn[j] = src[j];
  };
  if (wave < n_batch) load(wave);
  for (int bi = wave; bi < n_batch; bi += 4) {
    float4 kv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) kv[j] = kn[j];
    if (bi + 4 < n_batch) load(bi + 4);
    // the query is read from LDS (a broadcast) per batch: an opaque offset keeps the compiler
    // from holding all 256 values in registers
    const float* qp = sq + opaque(0);
    float dot[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float4 qv = *(const float4*)(qp + h * 64 + 4 * j);
        dot[h] = fmaf(qv.x, kv[j].x, dot[h]);
        dot[h] = fmaf(qv.y, kv[j].y, dot[h]);
        dot[h] = fmaf(qv.z, kv[j].z, dot[h]);
        dot[h] = fmaf(qv.w, kv[j].w, dot[h]);
      }
    }
    float sc = 0.f;
#pragma unroll
    for (int h = 0; h < 4; ++h) sc = fmaf(sq[256 + h], fmaxf(dot[h], 0.f), sc);
    if (bi * 64 + lane < seg_n) skey[bi * 64 + lane] = order_key(sc);
  }
  __syncthreads();
  const size_t cbase = ((size_t)r * n_seg + seg) * p.k;
  auto get = [&](int x) { return skey[x]; };
  uint32_t kstar;
  int need_eq;
  if (seg_n <= p.k) {
    for (int x = tid; x < seg_n; x += DEC_NT) {
      cand_key[cbase + x] = skey[x];
      cand_pos[cbase + x] = seg_start + x;
    }
  } else {
    radix_threshold<DEC_NT>(get, seg_n, p.k, hist, sh, wsum, kstar, need_eq);
    emit_topk<DEC_NT>(get, seg_n, kstar, need_eq, wsum, nullptr,
                      [&](int slot, int x, uint32_t u) {
      cand_key[cbase + slot] = u;
      cand_pos[cbase + slot] = seg_start + x;
      // compacted in place: slot <= x, and every key of x's chunk has been read
      skey[slot] = u;
    });
  }
  // the bound of a full segment (every segment of the row but the last): its k_lo-th largest
  // key, k_lo = ceil(k / (full segments)), so that the full segments hold >= k keys at or
  // above the smallest of their bounds.  k_lo <= k, so it is the k_lo-th largest of the
  // segment's top k, now in skey[0 .. k).
  const int n_full = (n + SEG - 1) / SEG - 1;
  if (seg < n_full) {
    const int k_lo = (p.k + n_full - 1) / n_full;  // <= k < SEG = seg_n
    __syncthreads();
    radix_threshold<DEC_NT>(get, p.k, k_lo, hist, sh, wsum, kstar, need_eq);
    if (tid == 0) lo_key[(size_t)r * n_seg + seg] = kstar;
  }
}

// Filter: workgroup (row, group g) concatenates the candidate lists of segments
// g G .. g G + G - 1 (in segment order, so in ascending position) and keeps the candidates
// whose key is at least L, the smallest bound of the row's full segments.  Those segments hold
// at least k keys >= L, so the row's k-th largest key is >= L and every key of the top k (ties
// included) passes.  A row of one segment has no bound (L = 0: everything passes).  Output
// list g has room for G k entries.
constexpr int FLT_NT = 512;
constexpr int FIN_NT = 512;
constexpr int FIN_CAP = 16384;    // candidates the final selection holds in LDS
constexpr int FIN_MAX_GRP = 1024; // filter groups per row (the group size grows past this)

__host__ __device__ inline int filter_g(int n_seg) {
  return n_seg <= 4 * FIN_MAX_GRP ? 4 : (n_seg + FIN_MAX_GRP - 1) / FIN_MAX_GRP;
}

constexpr int FLT_MAX_G = 128;  // filter_g for up to 2^31 keys
constexpr int FLT_R = 16;       // slots a thread holds per round

__global__ __launch_bounds__(FLT_NT) void index_filter_kernel(IndexParams p, int n_seg,
                                                              const uint32_t* in_key,
                                                              const int32_t* in_pos,
                                                              const int* in_cnt,
                                                              const uint32_t* lo_key,
                                                              uint32_t* out_key,
                                                              int32_t* out_pos, int* out_cnt) {
  __shared__ int wsum[2 * FLT_NT / 64];
  __shared__ int s_cnt[FLT_MAX_G];
  __shared__ uint32_t s_lo;
  const int G = filter_g(n_seg);
  const int n_grp = (n_seg + G - 1) / G;
  const int r = blockIdx.x / n_grp, grp = blockIdx.x % n_grp;
  const int b = r / p.Tq;
  const int n = visible_keys(p.pos0[b] + r % p.Tq, p.block, min(p.S, (p.max_pos + 1) / p.block));
  if (n <= p.k) return;  // written directly by the final selection
  const int n_full = (n + SEG - 1) / SEG - 1;
  if (threadIdx.x < 64) {
    uint32_t m = 0xFFFFFFFFu;
    for (int s = threadIdx.x; s < n_full; s += 64) m = min(m, lo_key[(size_t)r * n_seg + s]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = min(m, (uint32_t)__shfl_xor((int)m, off));
    if (threadIdx.x == 0) s_lo = n_full >= 1 ? m : 0u;
  }
  for (int q = threadIdx.x; q < G; q += FLT_NT) {
    const int li = grp * G + q;
    s_cnt[q] = li < n_seg ? in_cnt[(size_t)r * n_seg + li] : 0;
  }
  __syncthreads();
  const uint32_t lo = s_lo;
  const int k = p.k;
  // the group's lists laid end to end at a stride of k (list q's entries j < count are
  // candidates), in rounds of FLT_NT FLT_R consecutive slots: thread t takes FLT_R consecutive
  // slots of the round, loads their keys and positions once, counts the kept ones, and writes
  // them after the block scan, so the output keeps slot (position) order.
  const int n_slots = G * k;
  const size_t gbase = ((size_t)r * n_seg + (size_t)grp * G) * k;  // slot 0 of the group
  auto valid = [&](int x) { return x < G * k && x % k < s_cnt[x / k]; };
  const size_t dst = (size_t)r * n_grp + grp;
  uint32_t* ok = out_key + dst * G * k;
  int32_t* op = out_pos + dst * G * k;
  int base = 0;
  for (int r0 = 0; r0 < n_slots; r0 += FLT_NT * FLT_R) {
    const int x0 = r0 + (int)threadIdx.x * FLT_R;
    uint32_t u[FLT_R];
    int32_t ps[FLT_R];
    bool keep[FLT_R];
    int c = 0;
#pragma unroll
    for (int j = 0; j < FLT_R; ++j) {
      const bool v = valid(x0 + j);
      u[j] = v ? in_key[gbase + x0 + j] : 0u;
      ps[j] = v ? in_pos[gbase + x0 + j] : 0;
      keep[j] = v && u[j] >= lo;
      c += keep[j] ? 1 : 0;
    }
    int ex, ex2, tot, tot2;
    block_scan2<FLT_NT>(c, 0, ex, ex2, tot, tot2, wsum);
    (void)ex2;
    (void)tot2;
    int o = base + ex;
#pragma unroll
    for (int j = 0; j < FLT_R; ++j)
      if (keep[j]) {
        ok[o] = u[j];
        op[o] = ps[j];
        ++o;
      }
    base += tot;
  }
  if (threadIdx.x == 0) out_cnt[dst] = base;
}

// Final selection, one workgroup per row: the filtered lists in group order (ascending
// position), their top k by radix select, emitted in ascending position into idx_out.  Up to
// FIN_CAP candidates are held in LDS; more (only when very many keys tie at the bound) are
// selected over global memory.  Rows with at most k positions get all of them, then -1.
__global__ __launch_bounds__(FIN_NT) void index_final_kernel(IndexParams p, int n_seg,
                                                             const uint32_t* in_key,
                                                             const int32_t* in_pos,
                                                             const int* in_cnt) {
  __shared__ uint32_t rkey[FIN_CAP];
  __shared__ int32_t rpos[FIN_CAP];
  __shared__ uint32_t hist[(FIN_NT / 64) * 256];
  __shared__ int sh[3];
  __shared__ int wsum[2 * FIN_NT / 64];
  __shared__ int goff[FIN_MAX_GRP + 1];
  const int G = filter_g(n_seg);
  const int n_grp = (n_seg + G - 1) / G;
  const int r = blockIdx.x;
  const int b = r / p.Tq, i = r % p.Tq;
  const int n = visible_keys(p.pos0[b] + i, p.block, min(p.S, (p.max_pos + 1) / p.block));
  const int k = p.k;
  int32_t* out = p.idx_out + (size_t)r * k;
  if (n <= k) {
    for (int j = threadIdx.x; j < k; j += FIN_NT) out[j] = j < n ? j : -1;
    return;
  }
  {
    // offsets of the lists: thread t sums lists 2t and 2t + 1 (n_grp <= 2 FIN_NT)
    const int g0 = 2 * (int)threadIdx.x;
    const int c0 = g0 < n_grp ? in_cnt[(size_t)r * n_grp + g0] : 0;
    const int c1 = g0 + 1 < n_grp ? in_cnt[(size_t)r * n_grp + g0 + 1] : 0;
    int ex, ex2, tot, tot2;
    block_scan2<FIN_NT>(c0 + c1, 0, ex, ex2, tot, tot2, wsum);
    if (g0 < n_grp) goff[g0] = ex;
    if (g0 + 1 < n_grp) goff[g0 + 1] = ex + c0;
    if (threadIdx.x == 0) goff[n_grp] = tot;
    __syncthreads();
  }
  const int total = goff[n_grp];  // >= k: the top k passed the filter
  const size_t lbase = (size_t)r * n_grp * G * k;  // list g starts at lbase + g G k
  uint32_t kstar;
  int need_eq;
  // candidate x of the concatenation: list g with goff[g] <= x < goff[g + 1]
  auto at = [&](int x) {
    int lo = 0, hi = n_grp - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (goff[mid] <= x) lo = mid;
      else hi = mid - 1;
    }
    return lbase + (size_t)lo * G * k + (x - goff[lo]);
  };
  if (total <= FIN_CAP) {
    for (int x0 = threadIdx.x; x0 < total; x0 += 4 * FIN_NT) {
      uint32_t u[4];
      int32_t ps[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int x = x0 + j * FIN_NT;
        if (x < total) {
          const size_t a = at(x);
          u[j] = in_key[a];
          ps[j] = in_pos[a];
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int x = x0 + j * FIN_NT;
        if (x < total) {
          rkey[x] = u[j];
          rpos[x] = ps[j];
        }
      }
    }
    __syncthreads();
    auto get = [&](int x) { return rkey[x]; };
    radix_threshold<FIN_NT>(get, total, k, hist, sh, wsum, kstar, need_eq);
    emit_topk<FIN_NT>(get, total, kstar, need_eq, wsum, nullptr,
                      [&](int slot, int x, uint32_t) { out[slot] = rpos[x]; });
    return;
  }
  auto get = [&](int x) { return in_key[at(x)]; };
  radix_threshold<FIN_NT>(get, total, k, hist, sh, wsum, kstar, need_eq);
  emit_topk<FIN_NT>(get, total, kstar, need_eq, wsum, rkey,
                    [&](int slot, int x, uint32_t) { out[slot] = in_pos[at(x)]; });
}

bool use_decode_path(const IndexParams& p) { return p.Tq <= 4; }

long long key_bound(const IndexParams& p) {
  return std::max<long long>(1, std::min<long long>(p.S, ((long long)p.max_pos + 1) / p.block));
}

int n_segments(const IndexParams& p) {
  return (int)std::max<long long>(1, (key_bound(p) + SEG - 1) / SEG);
}

}  // namespace

// Decode workspace: the segments' candidate lists (k keys, k positions and a count each),
// their bounds, and the filtered lists (G k entries and a count each).
struct DecodeWs {
  size_t seg_lists, grp_lists, k;
  int G;
  size_t bytes() const {
    return seg_lists * (k * 8 + 4 + 4) + grp_lists * ((size_t)G * k * 8 + 4);
  }
};

static DecodeWs decode_ws(const IndexParams& p) {
  DecodeWs w;
  const size_t rows = (size_t)p.B * p.Tq;
  const int n_seg = n_segments(p);
  w.G = filter_g(n_seg);
  w.k = (size_t)p.k;
  w.seg_lists = rows * n_seg;
  w.grp_lists = rows * ((n_seg + w.G - 1) / w.G);
  return w;
}

size_t index_workspace(const IndexParams& p) {
  if (use_decode_path(p)) return decode_ws(p).bytes();
  const size_t q_chunk = std::min(p.Tq, 2048);
  return q_chunk * (size_t)key_bound(p) * sizeof(uint32_t);
}

hipError_t launch_index(const IndexParams& p, hipStream_t stream) {
  if ((long long)p.B * p.Tq == 0) return hipSuccess;
  if (use_decode_path(p)) {
    const int n_seg = n_segments(p);
    const size_t rows = (size_t)p.B * p.Tq;
    const DecodeWs w = decode_ws(p);
    char* base = (char*)p.ws;
    uint32_t* seg_key = (uint32_t*)base;
    int32_t* seg_pos = (int32_t*)(seg_key + w.seg_lists * w.k);
    int* seg_cnt = (int*)(seg_pos + w.seg_lists * w.k);
    uint32_t* lo_key = (uint32_t*)(seg_cnt + w.seg_lists);
    uint32_t* grp_key = lo_key + w.seg_lists;
    int32_t* grp_pos = (int32_t*)(grp_key + w.grp_lists * w.G * w.k);
    int* grp_cnt = (int*)(grp_pos + w.grp_lists * w.G * w.k);
    hipLaunchKernelGGL(index_segment_kernel, dim3((unsigned)(rows * n_seg)), dim3(DEC_NT), 0,
                       stream, p, n_seg, seg_key, seg_pos, seg_cnt, lo_key);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(index_filter_kernel, dim3((unsigned)w.grp_lists), dim3(FLT_NT), 0, stream,
                       p, n_seg, seg_key, seg_pos, seg_cnt, lo_key, grp_key, grp_pos, grp_cnt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(index_final_kernel, dim3((unsigned)rows), dim3(FIN_NT), 0, stream, p,
                       n_seg, grp_key, grp_pos, grp_cnt);
    return hipGetLastError();
  }
  const long long s_ld = key_bound(p);
  const long long q_chunk = std::min<long long>(p.Tq, (long long)(p.ws_bytes / (s_ld * 4)));
  uint32_t* ws = (uint32_t*)p.ws;
  const int n_sc = (int)((s_ld + SC_CH - 1) / SC_CH);
  for (int b = 0; b < p.B; ++b) {
    for (int i0 = 0; i0 < p.Tq; i0 += (int)q_chunk) {
      const int nq = (int)std::min<long long>(q_chunk, p.Tq - i0);
      hipLaunchKernelGGL(index_scores_kernel, dim3((nq + SC_Q - 1) / SC_Q, n_sc), dim3(256), 0,
                         stream, p, b, i0, nq, ws, (int)s_ld);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(index_select_rows_kernel, dim3(nq), dim3(SEL_NT), 0, stream, p, b, i0,
                         ws, (int)s_ld);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

size_t index_min_workspace(const IndexParams& p) {
  if (use_decode_path(p)) return index_workspace(p);
  return (size_t)key_bound(p) * sizeof(uint32_t);
}

}  // namespace lgsa
