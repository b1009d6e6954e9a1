// Heavily Compressed Attention forward in float32 (ERNIE 5.5 Flash Base release blog,
// section 2.1; 128-token window per the xenospectrum.com article on ERNIE 5.5 Flash Base).
// Plain FMA kernel for the small fp32 configuration: one workgroup per query row, heads in
// turn, keys in chunks of 256 with an online softmax; one thread per key for the logits,
// threads over channels for the value sum.  The gate, when present, runs afterwards as the
// fp32 gate GEMM in place.
#include "common.h"
#include "kernels.h"

namespace lgsa {

namespace {

constexpr int NT = 256;

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  // wave reduction then across the four waves
  for (int o = 32; o > 0; o >>= 1) {
    const float x = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, x) : v + x;
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  const float a = red[0], b = red[1], c = red[2], d = red[3];
  return is_max ? fmaxf(fmaxf(a, b), fmaxf(c, d)) : (a + b) + (c + d);
}

__global__ __launch_bounds__(NT) void hca_f32_kernel(HcaParams p) {
  __shared__ float sq[512];
  __shared__ float sp[NT];
  __shared__ int srow[NT];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int row = blockIdx.x;  // b * Tq + i
  const int b = row / p.Tq, i = row % p.Tq;
  const int d = p.d;
  const int t = p.pos0[b] + i;
  const int ne = t >= 0 ? min(p.n_cap, (t + 1) / p.block) : 0;
  const int s_lo = max(0, t - p.window + 1);
  const int nw = t >= 0 ? t - s_lo + 1 : 0;
  const int nk = ne + nw;
  const float* kc = (const float*)p.kc + (size_t)b * p.n_cap * d;
  const float* vc = (const float*)p.vc + (size_t)b * p.n_cap * d;
  const float* kw = (const float*)p.k_win + (size_t)b * p.win_len * d;
  const float* vw = (const float*)p.v_win + (size_t)b * p.win_len * d;
  for (int h = 0; h < p.H; ++h) {
    const float* q = (const float*)p.q + ((size_t)row * p.H + h) * d;
    for (int c = tid; c < d; c += NT) sq[c] = q[c];
    float m = -INFINITY, l = 0.f;
    float acc[2] = {0.f, 0.f};  // channels tid and tid + 256
    for (int k0 = 0; k0 < nk; k0 += NT) {
      __syncthreads();
      const int j = k0 + tid;
      float logit = -INFINITY;
      if (j < nk) {
        const float* kr = j < ne ? kc + (size_t)j * d
                                 : kw + (size_t)((s_lo + (j - ne)) % p.win_len) * d;
        float s = 0.f;
        for (int c = 0; c < d; c += 4) {
          const float4 kv = *(const float4*)(kr + c);
          s = fmaf(sq[c], kv.x, s);
          s = fmaf(sq[c + 1], kv.y, s);
          s = fmaf(sq[c + 2], kv.z, s);
          s = fmaf(sq[c + 3], kv.w, s);
        }
        logit = s * p.scale;
        srow[tid] = j;
      }
      const float cm = block_reduce(logit, red, true);
      const float m_new = fmaxf(m, cm);
      const float alpha = m == -INFINITY ? 0.f : expf(m - m_new);
      const float pj = j < nk ? expf(logit - m_new) : 0.f;
      sp[tid] = pj;
      const float ps = block_reduce(pj, red, false);
      l = l * alpha + ps;
      m = m_new;
      const int cnt = min(NT, nk - k0);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c = tid + NT * u;
        if (c >= d) continue;
        float a = acc[u] * alpha;
        for (int jj = 0; jj < cnt; ++jj) {
          const int kj = srow[jj];
          const float* vr = kj < ne ? vc + (size_t)kj * d
                                    : vw + (size_t)((s_lo + (kj - ne)) % p.win_len) * d;
          a = fmaf(sp[jj], vr[c], a);
        }
        acc[u] = a;
      }
    }
    float* o = (float*)p.out + ((size_t)row * p.H + h) * d;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = tid + NT * u;
      if (c < d) o[c] = acc[u] * inv;
    }
    __syncthreads();
  }
}

}  // namespace

size_t hca_f32_workspace(const HcaParams&) { return 0; }

hipError_t launch_hca_f32(const HcaParams& p, hipStream_t stream) {
  const long long rows = (long long)p.B * p.Tq;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(hca_f32_kernel, dim3((unsigned)rows), dim3(NT), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.q_lat != nullptr) {
    e = launch_gate(p.q_lat, p.w_gate, p.out, p.out, (int)rows, p.d_lat, p.H * p.d, DT_F32,
                    stream);
    if (e != hipSuccess) return e;
  }
  if (p.vha_r > 0)  // the head mix of the gated output, in place
    return launch_vha(p.out, p.vha_u, p.vha_v, p.out, (int)rows, p.H, p.d, p.vha_r, DT_F32,
                      stream);
  return hipSuccess;
}

}  // namespace lgsa
