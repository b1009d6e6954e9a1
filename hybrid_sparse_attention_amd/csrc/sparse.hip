// DSA sparse core attention of the MLA layers (ERNIE 5.5 Flash Base release blog, section
// 2.1: core attention runs only on the top-k positions chosen by the indexer; MLA heads are
// 256 wide for query/key and value).  bfloat16 latent rows are gathered by index, every
// listed position is one key (negative or out-of-range entries are skipped), order is
// irrelevant, and one latent row may serve as both key and value.
//
// Workgroup: one query row (all H heads share its index list) and a range of its list.
// Waves 0,1 / 2,3 take heads 0..31 / 32..63 (as MFMA columns) of the even / odd 32-key
// tiles; each pair of tiles is gathered together (coalesced 16-byte row reads, V transposed
// while staged), the two halves merge through LDS.  The products are the transposed ones
// (S^T = K Q^T, O^T = V^T P^T on v_mfma_f32_16x16x32_bf16) so the P fragment is the S^T
// accumulator itself.  Long lists of few query rows are split over several workgroups,
// whose partial (max, sum, O) a combine kernel merges.  The output gate runs afterwards as
// the gate GEMM in place (a per-row workgroup would have to read the whole gate matrix).
#include "common.h"
#include "kernels.h"

namespace lgsa {

namespace {

constexpr int D = 256;
constexpr int KT = 32;
constexpr int KS_LD = D + 8;
constexpr int VT_LD = KT + 8;
constexpr int KS_ELEMS = KT * KS_LD;
constexpr int VT_ELEMS = D * VT_LD;
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ int slot_key(int p) {
  const int g = p >> 3, j = p & 7;
  return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
}

__shared__ __attribute__((aligned(16))) uint16_t sp_smem[2 * KS_ELEMS + 2 * VT_ELEMS];
__shared__ int sp_idx[2 * KT];

struct WaveState {
  f32x4_t o[16][2];
  float m[2], l[2];
};

__device__ __forceinline__ void attend(WaveState& st, const Frag8 (&qf)[2][8],
                                       const uint16_t* ks, const uint16_t* vt,
                                       const int* tidx, float scale_log2, int lane) {
  const int l16 = lane & 15, g = lane >> 4;
  f32x4_t s[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) s[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    Frag8 ka[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
      ka[mb].u = *(const uint4*)(ks + (16 * mb + l16) * KS_LD + 32 * kk + 8 * g);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) s[mb][nb] = mfma_16x16x32(ka[mb], qf[nb][kk], s[mb][nb]);
  }
  bool valid[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) valid[mb][r] = tidx[16 * mb + 4 * g + r] >= 0;
  float alpha[2];
  Frag8 pf[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float x[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[mb][r] = valid[mb][r] ? s[mb][nb][r] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, x[mb][r]);
      }
    mx = wave_max16(mx);
    const float m_new = fmaxf(st.m[nb], mx);
    alpha[nb] = st.m[nb] == -INFINITY ? 0.f : fast_exp2(st.m[nb] - m_new);
    st.m[nb] = m_new;
    float p[2][4], psum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[mb][r] = x[mb][r] == -INFINITY ? 0.f : fast_exp2(x[mb][r] - m_new);
        psum += p[mb][r];
      }
    st.l[nb] = st.l[nb] * alpha[nb] + psum;
    pf[nb].u = make_uint4(pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                          pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3]));
  }
  if (__any((alpha[0] != 1.f) | (alpha[1] != 1.f))) {
#pragma unroll
    for (int cb = 0; cb < 16; ++cb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) st.o[cb][nb] *= alpha[nb];
  }
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) {
    Frag8 va;
    va.u = *(const uint4*)(vt + (16 * cb + l16) * VT_LD + 8 * g);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) st.o[cb][nb] = mfma_16x16x32(va, pf[nb], st.o[cb][nb]);
  }
}

__device__ __forceinline__ void store4(uint16_t* dst, const f32x4_t& v) {
  uint2 r;
  r.x = pack_bf16x2(v[0], v[1]);
  r.y = pack_bf16x2(v[2], v[3]);
  *(uint2*)dst = r;
}

// grid: (row r = b*Tq + i) x (head group of 64) x (split); n_split == 1 writes out directly
__global__ __launch_bounds__(256, 2) void sparse_kernel(SparseParams p, int n_split,
                                                        int chunk, float* part_o,
                                                        float* part_ml) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int n_hg = p.H / 64;
  const int sp = blockIdx.x % n_split;
  const int hg = (blockIdx.x / n_split) % n_hg;
  const int r = blockIdx.x / (n_split * n_hg);
  const int b = r / p.Tq;
  const int j_begin = sp * chunk, j_end = min(p.k, j_begin + chunk);
  const int half = wave >> 1;
  const int h0 = hg * 64 + 32 * (wave & 1);

  Frag8 qf[2][8];
  const uint16_t* qb = (const uint16_t*)p.q + (size_t)r * p.H * D;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const uint16_t* qr = qb + (size_t)(h0 + 16 * nb + l16) * D;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[nb][kk].u = *(const uint4*)(qr + 32 * kk + 8 * g);
  }
  WaveState st;
#pragma unroll
  for (int cb = 0; cb < 16; ++cb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) st.o[cb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  st.m[0] = st.m[1] = -INFINITY;
  st.l[0] = st.l[1] = 0.f;
  const float scale_log2 = p.scale * LOG2E;

  const int32_t* idx = p.idx + (size_t)r * p.k;
  const uint16_t* kl = (const uint16_t*)p.k_lat + (size_t)b * p.S * p.k_stride;
  const uint16_t* vl = (const uint16_t*)p.v_lat + (size_t)b * p.S * p.v_stride;
  for (int j0 = j_begin; j0 < j_end; j0 += 2 * KT) {
    // positions of the two tiles (-1: skipped)
    if (tid < 2 * KT) {
      const int j = j0 + tid;
      int s = j < j_end ? idx[j] : -1;
      if (s >= p.S) s = -1;
      sp_idx[tid] = s;
    }
    __syncthreads();
    // K rows: 64 rows x 32 chunks of 16 bytes, 8 per thread
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = tid + 256 * u;
      const int key = c >> 5, col = (c & 31) * 8;
      const int s = sp_idx[key];
      const uint4 v = s >= 0 ? *(const uint4*)(kl + (size_t)s * p.k_stride + col)
                             : make_uint4(0, 0, 0, 0);
      *(uint4*)(sp_smem + (key >> 5) * KS_ELEMS + (key & 31) * KS_LD + col) = v;
    }
    // V^T: thread -> tile u, slot group kg, column group cg; 8 rows, then an 8x8 transpose
    {
      const int u = tid >> 7, kg = tid & 3, cg = (tid >> 2) & 31;
      uint4 rows[8], cols[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int s = sp_idx[KT * u + slot_key(8 * kg + jj)];
        rows[jj] = s >= 0 ? *(const uint4*)(vl + (size_t)s * p.v_stride + 8 * cg)
                          : make_uint4(0, 0, 0, 0);
      }
      transpose8x8(rows, cols);
      uint16_t* vt = sp_smem + 2 * KS_ELEMS + u * VT_ELEMS;
#pragma unroll
      for (int i = 0; i < 8; ++i) *(uint4*)(vt + (8 * cg + i) * VT_LD + 8 * kg) = cols[i];
    }
    __syncthreads();
    if (j0 + KT * half < j_end)
      attend(st, qf, sp_smem + half * KS_ELEMS, sp_smem + 2 * KS_ELEMS + half * VT_ELEMS,
             sp_idx + KT * half, scale_log2, lane);
    __syncthreads();
  }

  // merge the two tile halves through LDS
  float* xo = (float*)sp_smem;              // [2][16][2][64][4] floats = 64 KB
  float* xml = xo + 2 * 16 * 2 * 64 * 4;    // [2][2][2][64]
  float lsum[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) lsum[nb] = wave_sum16(st.l[nb]);
  const int wv = wave & 1;
  if (half == 1) {
#pragma unroll
    for (int cb = 0; cb < 16; ++cb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        *(f32x4_t*)(xo + (((wv * 16 + cb) * 2 + nb) * 64 + lane) * 4) = st.o[cb][nb];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      xml[((wv * 2 + nb) * 2 + 0) * 64 + lane] = st.m[nb];
      xml[((wv * 2 + nb) * 2 + 1) * 64 + lane] = lsum[nb];
    }
  }
  __syncthreads();
  if (half == 1) return;
  float as[2], ao[2], mt[2], lt[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float mo = xml[((wv * 2 + nb) * 2 + 0) * 64 + lane];
    const float lo = xml[((wv * 2 + nb) * 2 + 1) * 64 + lane];
    mt[nb] = fmaxf(st.m[nb], mo);
    as[nb] = st.m[nb] == -INFINITY ? 0.f : fast_exp2(st.m[nb] - mt[nb]);
    ao[nb] = mo == -INFINITY ? 0.f : fast_exp2(mo - mt[nb]);
    lt[nb] = lsum[nb] * as[nb] + lo * ao[nb];
  }
#pragma unroll
  for (int cb = 0; cb < 16; ++cb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const f32x4_t other = *(const f32x4_t*)(xo + (((wv * 16 + cb) * 2 + nb) * 64 + lane) * 4);
      st.o[cb][nb] = st.o[cb][nb] * as[nb] + other * ao[nb];
    }
  if (n_split == 1) {
    uint16_t* out = (uint16_t*)p.out + (size_t)r * p.H * D;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float inv = lt[nb] > 0.f ? 1.f / lt[nb] : 0.f;
      uint16_t* orow = out + (size_t)(h0 + 16 * nb + l16) * D;
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) store4(orow + 16 * cb + 4 * g, st.o[cb][nb] * inv);
    }
    return;
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int hh = h0 + 16 * nb + l16;
    const size_t pr = ((size_t)r * n_split + sp) * p.H + hh;
    float* po = part_o + pr * D;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) *(f32x4_t*)(po + 16 * cb + 4 * g) = st.o[cb][nb];
    if (g == 0) {
      part_ml[pr * 2 + 0] = mt[nb];
      part_ml[pr * 2 + 1] = lt[nb];
    }
  }
}

__global__ __launch_bounds__(64) void sparse_combine_kernel(const float* __restrict__ part_o,
                                                            const float* __restrict__ part_ml,
                                                            uint16_t* __restrict__ out, int H,
                                                            int n_split) {
  const int rh = blockIdx.x;  // r * H + h
  const int r = rh / H, h = rh % H;
  float mt = -INFINITY;
  for (int s = 0; s < n_split; ++s)
    mt = fmaxf(mt, part_ml[(((size_t)r * n_split + s) * H + h) * 2]);
  float lt = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < n_split; ++s) {
    const size_t pr = ((size_t)r * n_split + s) * H + h;
    const float ms = part_ml[pr * 2];
    const float a = ms == -INFINITY ? 0.f : fast_exp2(ms - mt);
    lt += a * part_ml[pr * 2 + 1];
    const float4 v = *(const float4*)(part_o + pr * D + 4 * threadIdx.x);
    acc[0] += a * v.x;
    acc[1] += a * v.y;
    acc[2] += a * v.z;
    acc[3] += a * v.w;
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  uint2 o;
  o.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  o.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *(uint2*)(out + (size_t)rh * D + 4 * threadIdx.x) = o;
}

void sparse_plan(const SparseParams& p, int& n_split, int& chunk) {
  const long long wgs = (long long)p.B * p.Tq * (p.H / 64);
  long long want = wgs >= 512 ? 1 : (512 + wgs - 1) / wgs;
  const long long max_split = (p.k + 2 * KT - 1) / (2 * KT);
  n_split = (int)std::max<long long>(1, std::min(want, max_split));
  long long c = (p.k + n_split - 1) / n_split;
  c = (c + 2 * KT - 1) / (2 * KT) * (2 * KT);
  chunk = (int)c;
  n_split = (int)((p.k + chunk - 1) / chunk);
}

}  // namespace

size_t sparse_workspace(const SparseParams& p) {
  int n_split, chunk;
  sparse_plan(p, n_split, chunk);
  if (n_split == 1) return 0;
  const size_t rows = (size_t)p.B * p.Tq * n_split * p.H;
  return rows * D * sizeof(float) + rows * 2 * sizeof(float);
}

hipError_t launch_sparse(const SparseParams& p, hipStream_t stream) {
  const long long rows = (long long)p.B * p.Tq;
  if (rows == 0) return hipSuccess;
  int n_split, chunk;
  sparse_plan(p, n_split, chunk);
  float* part_o = (float*)p.ws;
  float* part_ml = part_o ? part_o + (size_t)rows * n_split * p.H * D : nullptr;
  const long long grid = rows * (p.H / 64) * n_split;
  hipLaunchKernelGGL(sparse_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p, n_split,
                     chunk, part_o, part_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (n_split > 1) {
    hipLaunchKernelGGL(sparse_combine_kernel, dim3((unsigned)(rows * p.H)), dim3(64), 0, stream,
                       part_o, part_ml, (uint16_t*)p.out, p.H, n_split);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.q_lat != nullptr)
    return launch_gate(p.q_lat, p.w_gate, p.out, p.out, (int)rows, p.d_lat, p.H * D, DT_BF16,
                       stream);
  return hipSuccess;
}

}  // namespace lgsa
