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
// Prefill (many queries per sequence): scores come from fp32 MFMA (v_mfma_f32_16x16x4f32,
// rows = (query, indexer head), columns = keys, contraction = the 64 indexer dims), so each
// key tile in LDS serves 64 queries; they are written as keys to the workspace, a chunk of
// queries at a time, and a 1024-thread workgroup per query selects.
// Decode (few queries, long context): one workgroup per (query, 16384-position segment)
// streams its key rows through LDS once, scores them with fp32 FMA, selects the segment's
// top-k in LDS and writes them as candidates; a second kernel selects the final top-k among
// the candidates (the union of per-segment top-k sets contains the global top-k).
#include "common.h"
#include "kernels.h"

namespace lgsa {

namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 counts as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive rank of `flag` among the workgroup's threads (thread order), and the total.
template <int NT>
__device__ __forceinline__ int block_rank(bool flag, int& total, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long bal = __ballot(flag);
  const int in_wave = __popcll(bal & ((1ull << lane) - 1ull));
  __syncthreads();
  if (lane == 0) wsum[wave] = __popcll(bal);
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int c = wsum[w];
    before += w < wave ? c : 0;
    tot += c;
  }
  total = tot;
  return before + in_wave;
}

// Finds the k-th largest key K* among get(0..n-1) (k <= n) and the number of keys equal to
// K* that belong to the top k; 8-bit digits, most significant first.
template <int NT, class Get>
__device__ void radix_threshold(const Get& get, int n, int k, uint32_t* hist, int* sh,
                                uint32_t& kstar, int& need_eq) {
  uint32_t prefix = 0u;
  int kr = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int x = threadIdx.x; x < 256; x += NT) hist[x] = 0u;
    __syncthreads();
    const uint32_t hi_mask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int i = threadIdx.x; i < n; i += NT) {
      const uint32_t u = get(i);
      if ((u & hi_mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int cum = 0, dsel = 0;
      for (int dg = 255; dg >= 0; --dg) {
        const int c = (int)hist[dg];
        if (cum + c >= kr) {
          dsel = dg;
          break;
        }
        cum += c;
      }
      sh[0] = dsel;
      sh[1] = kr - cum;
    }
    __syncthreads();
    prefix |= (uint32_t)sh[0] << shift;
    kr = sh[1];
    __syncthreads();
  }
  kstar = prefix;
  need_eq = kr;
}

// Ascending pass: emit(slot, i, key) for every i whose key is above K*, and for the first
// need_eq (in index order) whose key equals K*.
template <int NT, class Get, class Emit>
__device__ void emit_topk(const Get& get, int n, uint32_t kstar, int need_eq, int* wsum,
                          const Emit& emit) {
  int base = 0, eq_seen = 0;
  for (int c0 = 0; c0 < n; c0 += NT) {
    const int i = c0 + (int)threadIdx.x;
    const uint32_t u = i < n ? get(i) : 0u;
    const bool gt = i < n && u > kstar;
    const bool eq = i < n && u == kstar;
    int eq_tot, sel_tot;
    const int eq_rank = block_rank<NT>(eq, eq_tot, wsum);
    const bool sel = gt || (eq && eq_seen + eq_rank < need_eq);
    const int r = block_rank<NT>(sel, sel_tot, wsum);
    if (sel) emit(base + r, i, u);
    base += sel_tot;
    eq_seen += eq_tot;
  }
}

// ------------------------------------------------------------------------------ prefill
constexpr int SC_Q = 64;     // queries per workgroup (4 waves x 16)
constexpr int SC_KT = 64;    // keys per LDS tile
constexpr int SC_CH = 512;   // keys per workgroup
constexpr int SK_LD = 64 + 4;

// Scores of queries [i_begin, i_begin + nq) of sequence b against keys, written as ordered
// keys to ws[(i - i_begin) * s_ld + s].
__global__ __launch_bounds__(256) void index_scores_kernel(IndexParams p, int b, int i_begin,
                                                           int nq, uint32_t* ws, int s_ld) {
  __shared__ __attribute__((aligned(16))) float sk[SC_KT * SK_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int i0 = i_begin + blockIdx.x * SC_Q;
  const int i_stop = i_begin + nq;
  const int pos = p.pos0[b];
  const int t_hi = min(min(p.S, p.max_pos + 1) - 1, pos + min(i_stop, i0 + SC_Q) - 1);
  const int s_begin = blockIdx.y * SC_CH;
  if (s_begin > t_hi) return;
  const int s_end = min(t_hi + 1, s_begin + SC_CH);

  // A fragments: row (query 4mb + l16/4, head l16%4), contraction index 4ks + g
  float a[4][16];
  float wv[4][4];
  const int hq = l16 & 3;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int i = i0 + 16 * wave + 4 * mb + (l16 >> 2);
    const bool ok = i < i_stop && hq < p.Hi;
    const float* qr = p.q_idx + (((size_t)b * p.Tq + i) * p.Hi + hq) * 64;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) a[mb][ks] = ok ? qr[4 * ks + g] : 0.f;
    const int io = i0 + 16 * wave + 4 * mb + g;  // the query of output rows 4g..4g+3
#pragma unroll
    for (int r = 0; r < 4; ++r)
      wv[mb][r] = (io < i_stop && r < p.Hi) ? p.w_idx[((size_t)b * p.Tq + io) * p.Hi + r] : 0.f;
  }
  const float* kb = p.k_idx + (size_t)b * p.S * 64;
  for (int s0 = s_begin; s0 < s_end; s0 += SC_KT) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u;  // float4 index in the 64 x 64 tile
      const int key = c >> 4, dim = (c & 15) * 4;
      const float4 v = s0 + key < s_end ? *(const float4*)(kb + (size_t)(s0 + key) * 64 + dim)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
      *(float4*)(&sk[key * SK_LD + dim]) = v;
    }
    __syncthreads();
    f32x4v acc[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      float bv[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) bv[nb] = sk[(16 * nb + l16) * SK_LD + 4 * ks + g];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mb][ks], bv[nb], acc[mb][nb], 0, 0, 0);
    }
    // lane: query 4mb + g (of this wave), key s0 + 16nb + l16, heads r = 0..3
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int i = i0 + 16 * wave + 4 * mb + g;
      if (i >= i_stop) continue;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int s = s0 + 16 * nb + l16;
        if (s >= s_end) continue;
        float sc = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) sc = fmaf(wv[mb][r], fmaxf(acc[mb][nb][r], 0.f), sc);
        ws[(size_t)(i - i_begin) * s_ld + s] = order_key(sc);
      }
    }
  }
}

constexpr int SEL_NT = 1024;

__global__ __launch_bounds__(SEL_NT) void index_select_rows_kernel(IndexParams p, int b,
                                                                   int i_begin,
                                                                   const uint32_t* ws,
                                                                   int s_ld) {
  __shared__ uint32_t hist[256];
  __shared__ int sh[2];
  __shared__ int wsum[SEL_NT / 64];
  const int i = i_begin + blockIdx.x;
  const int t = min(p.pos0[b] + i, min(p.S, p.max_pos + 1) - 1);
  const int n = t >= 0 ? t + 1 : 0;
  int32_t* out = p.idx_out + ((size_t)b * p.Tq + i) * p.k;
  if (n <= p.k) {
    for (int j = threadIdx.x; j < p.k; j += SEL_NT) out[j] = j < n ? j : -1;
    return;
  }
  const uint32_t* row = ws + (size_t)blockIdx.x * s_ld;
  auto get = [&](int x) { return row[x]; };
  uint32_t kstar;
  int need_eq;
  radix_threshold<SEL_NT>(get, n, p.k, hist, sh, kstar, need_eq);
  emit_topk<SEL_NT>(get, n, kstar, need_eq, wsum,
                    [&](int slot, int x, uint32_t) { out[slot] = x; });
}

// ------------------------------------------------------------------------------ decode
constexpr int SEG = 16384;       // positions per segment (>= the largest supported k)
constexpr int DEC_NT = 256;
constexpr int DK_LD = 64 + 4;

__global__ __launch_bounds__(DEC_NT) void index_segment_kernel(IndexParams p, int n_seg,
                                                               uint32_t* cand_key,
                                                               int32_t* cand_pos) {
  extern __shared__ __attribute__((aligned(16))) uint32_t seg_smem[];
  uint32_t* skey = seg_smem;                                   // [SEG]
  float* stage = (float*)(seg_smem + SEG);                     // [4 waves][64][DK_LD]
  float* sq = stage + 4 * 64 * DK_LD;                          // [4][64] query, [4] weights
  uint32_t* hist = (uint32_t*)(sq + 4 * 64 + 4);               // [256]
  int* sh = (int*)(hist + 256);                                // [2]
  int* wsum = sh + 2;                                          // [4]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x / n_seg, seg = blockIdx.x % n_seg;  // r = b * Tq + i
  const int b = r / p.Tq, i = r % p.Tq;
  const int t = min(p.pos0[b] + i, min(p.S, p.max_pos + 1) - 1);
  const int n = t >= 0 ? t + 1 : 0;
  const int seg_start = seg * SEG;
  if (n <= p.k || seg_start >= n) return;  // short rows are finished by the merge kernel
  const int seg_n = min(SEG, n - seg_start);
  for (int x = tid; x < 4 * 64; x += DEC_NT) {
    const int h = x >> 6;
    sq[x] = h < p.Hi ? p.q_idx[((size_t)r * p.Hi + h) * 64 + (x & 63)] : 0.f;
  }
  if (tid < 4) sq[256 + tid] = tid < p.Hi ? p.w_idx[(size_t)r * p.Hi + tid] : 0.f;
  __syncthreads();
  const float* kb = p.k_idx + ((size_t)b * p.S + seg_start) * 64;
  float* st = stage + wave * 64 * DK_LD;
  const int n_batch = (seg_n + 63) / 64;
  for (int bi = wave; bi < n_batch; bi += 4) {
    const int k0 = bi * 64;
    // 64 consecutive key rows = 16 KB contiguous: coalesced float4 loads into LDS rows
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int f = 64 * j + lane;  // float4 index within the batch
      const int key = f >> 4, dim = (f & 15) * 4;
      const float4 v = k0 + key < seg_n ? *(const float4*)(kb + (size_t)(k0 + key) * 64 + dim)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
      *(float4*)(st + key * DK_LD + dim) = v;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    const float* kr = st + lane * DK_LD;
    float dot[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 64; c += 4) {
      const float4 kv = *(const float4*)(kr + c);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float4 qv = *(const float4*)(sq + h * 64 + c);
        dot[h] = fmaf(qv.x, kv.x, dot[h]);
        dot[h] = fmaf(qv.y, kv.y, dot[h]);
        dot[h] = fmaf(qv.z, kv.z, dot[h]);
        dot[h] = fmaf(qv.w, kv.w, dot[h]);
      }
    }
    float sc = 0.f;
#pragma unroll
    for (int h = 0; h < 4; ++h) sc = fmaf(sq[256 + h], fmaxf(dot[h], 0.f), sc);
    if (k0 + lane < seg_n) skey[k0 + lane] = order_key(sc);
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  const size_t cbase = ((size_t)r * n_seg + seg) * p.k;
  auto get = [&](int x) { return skey[x]; };
  if (seg_n <= p.k) {
    for (int x = tid; x < seg_n; x += DEC_NT) {
      cand_key[cbase + x] = skey[x];
      cand_pos[cbase + x] = seg_start + x;
    }
    return;
  }
  uint32_t kstar;
  int need_eq;
  radix_threshold<DEC_NT>(get, seg_n, p.k, hist, sh, kstar, need_eq);
  emit_topk<DEC_NT>(get, seg_n, kstar, need_eq, wsum, [&](int slot, int x, uint32_t u) {
    cand_key[cbase + slot] = u;
    cand_pos[cbase + slot] = seg_start + x;
  });
}

__global__ __launch_bounds__(SEL_NT) void index_merge_kernel(IndexParams p, int n_seg,
                                                             const uint32_t* cand_key,
                                                             const int32_t* cand_pos) {
  __shared__ uint32_t hist[256];
  __shared__ int sh[2];
  __shared__ int wsum[SEL_NT / 64];
  const int r = blockIdx.x;
  const int b = r / p.Tq, i = r % p.Tq;
  const int t = min(p.pos0[b] + i, min(p.S, p.max_pos + 1) - 1);
  const int n = t >= 0 ? t + 1 : 0;
  int32_t* out = p.idx_out + (size_t)r * p.k;
  if (n <= p.k) {
    for (int j = threadIdx.x; j < p.k; j += SEL_NT) out[j] = j < n ? j : -1;
    return;
  }
  // candidates: every segment but the last contributes exactly k, in ascending position
  const int segs = (n + SEG - 1) / SEG;
  const int last_n = n - (segs - 1) * SEG;
  const int nc = (segs - 1) * p.k + min(p.k, last_n);
  const uint32_t* ck = cand_key + (size_t)r * n_seg * p.k;
  const int32_t* cp = cand_pos + (size_t)r * n_seg * p.k;
  auto get = [&](int x) { return ck[x]; };
  uint32_t kstar;
  int need_eq;
  radix_threshold<SEL_NT>(get, nc, p.k, hist, sh, kstar, need_eq);
  emit_topk<SEL_NT>(get, nc, kstar, need_eq, wsum,
                    [&](int slot, int x, uint32_t) { out[slot] = cp[x]; });
}

constexpr size_t SEG_SMEM = (size_t)SEG * 4 + (size_t)4 * 64 * DK_LD * 4 + (4 * 64 + 4) * 4 +
                            256 * 4 + 2 * 4 + 4 * 4;

bool use_decode_path(const IndexParams& p) { return p.Tq <= 4; }

long long key_bound(const IndexParams& p) {
  return std::min<long long>(p.S, (long long)p.max_pos + 1);
}

int n_segments(const IndexParams& p) {
  return (int)std::max<long long>(1, (key_bound(p) + SEG - 1) / SEG);
}

}  // namespace

size_t index_workspace(const IndexParams& p) {
  if (use_decode_path(p)) {
    const size_t rows = (size_t)p.B * p.Tq;
    return rows * n_segments(p) * p.k * (sizeof(uint32_t) + sizeof(int32_t));
  }
  const size_t q_chunk = std::min(p.Tq, 1024);
  return q_chunk * (size_t)key_bound(p) * sizeof(uint32_t);
}

hipError_t launch_index(const IndexParams& p, hipStream_t stream) {
  if ((long long)p.B * p.Tq == 0) return hipSuccess;
  if (use_decode_path(p)) {
    static bool attr_set = false;
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute((const void*)index_segment_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)SEG_SMEM);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    const int n_seg = n_segments(p);
    const size_t rows = (size_t)p.B * p.Tq;
    uint32_t* ck = (uint32_t*)p.ws;
    int32_t* cp = (int32_t*)(ck + rows * n_seg * p.k);
    hipLaunchKernelGGL(index_segment_kernel, dim3((unsigned)(rows * n_seg)), dim3(DEC_NT),
                       SEG_SMEM, stream, p, n_seg, ck, cp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(index_merge_kernel, dim3((unsigned)rows), dim3(SEL_NT), 0, stream, p,
                       n_seg, ck, cp);
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
