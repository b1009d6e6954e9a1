// DSA sparse core attention of the MLA layers (ERNIE 5.5 Flash Base release blog, section
// 2.1: core attention runs only on the top-k positions chosen by the indexer; MLA heads are
// 256 wide for query/key and value).  bfloat16 latent rows are gathered by index, every
// listed position is one key (negative or out-of-range entries are skipped), order is
// irrelevant, and one latent row may serve as both key and value.
//
// Workgroup: one query row (its H heads share the index list), 64 heads, and a range of the
// list.  Two waves take 32 heads each over the whole 256-wide head, as two blocks of 16 MFMA
// columns: Q in 64 registers, O in 128.  Every K or V fragment read from LDS feeds both blocks,
// which halves the LDS read traffic of 16 heads per wave; four workgroups fit a CU.  Keys come
// in tiles of 32 gathered rows, brought to LDS by LDS DMA (one instruction fetches two 512-byte
// rows) and double buffered.  When the value rows are the key rows the
// single tile serves both products: S^T = K Q^T reads it row-wise, O^T = V^T P^T reads it
// through the transposing LDS read, so each gathered row crosses the memory system once.
// The 16-byte chunks of a row are rotated (chunk c of row r at position
// (c + 2r + 16 (r & 1)) mod 32) so that both read patterns run at the LDS's full rate; the DMA
// applies the rotation by choosing which chunk each lane fetches.  Long lists of few query rows are split over several
// workgroups, whose partial (max, sum, O) a combine kernel merges.  The output gate runs
// afterwards as the gate GEMM in place (a per-row workgroup would have to read the whole gate
// matrix).
#include "common.h"
#include "kernels.h"
#include "sparse_tile.h"
#include "vha_tile.h"

namespace lgsa {

namespace {

using namespace sparse_tile;

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.69314718055994531f;
constexpr float LAZY = 8.0f;            // rescale O only when the max grows by more (log2)
constexpr float NEG_BIG = -1.0e30f;     // masked logit (finite: no inf - inf)
// Waves per workgroup: two of 32 heads when one gathered tile serves as keys and values, four
// of 16 heads when a second (value) tile is gathered beside it (its LDS then allows two
// workgroups per CU, and four waves keep eight waves on the CU).
template <bool ALIAS> constexpr int waves_of() { return ALIAS ? 2 : 4; }
// The key tiles double as the staging area of the epilogue's head mix: 64 head rows of 256
// bfloat16 channels, 32 to a tile, rows padded to 544 bytes (conflict-free transposing reads).
constexpr int MIX_ROW = 544;
constexpr int KTILE_BYTES = TILE > 32 * MIX_ROW ? TILE : 32 * MIX_ROW;

template <int NHB>
struct WaveState {
  f32x4_t o[NHB][16];  // o[hb][cb][r] = O[head 16hb + l16][16cb + 4g + r]
  float m[NHB];        // reference max (log2 domain)
  float l[NHB];        // running partial sum of this lane's keys
};

// kr = l16 * TROW and kc = g + 2 l16 + 16 (l16 & 1): key row 16mb + l16, chunk 4kk + g sits at
// position (4kk + kc) mod 32 (rows 16 apart share positions)
template <int NHB>
__device__ __forceinline__ void scores(f32x4_t (&s)[NHB][2], const Frag8 (&qf)[NHB][8],
                                       const char* kt, int kr, int kc) {
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) s[hb][0] = s[hb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int kc_t = opaque(kc);  // formed per tile, so the 8 positions are not kept live
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    Frag8 ka[2];
    const int off = kr + 16 * ((4 * kk + kc_t) & 31);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
      ka[mb].u = *(const uint4*)(kt + off + 16 * TROW * mb);
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) s[hb][mb] = mfma_16x16x32(ka[mb], qf[hb][kk], s[hb][mb]);
  }
}

template <int NHB>
__device__ __forceinline__ void softmax_pv(WaveState<NHB>& st, const f32x4_t (&s)[NHB][2],
                                           const char* vt, uint32_t valid, float scale_log2,
                                           int vrow, int vc, int lane) {
  const int g = lane >> 4;
  Frag8 pf[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    float x[2][4];  // [mb][r]: key 16mb + 4g + r
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        x[mb][r] = ((valid >> (16 * mb + 4 * g + r)) & 1u) ? s[hb][mb][r] * scale_log2 : NEG_BIG;
    float mx = x[0][0];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, x[mb][r]);
    const float m_new = fmaxf(st.m[hb], wave_max16(mx));
    if (__any(m_new > st.m[hb] + LAZY)) {
      const float alpha = fast_exp2(st.m[hb] - m_new);
      st.m[hb] = m_new;
      st.l[hb] *= alpha;
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) st.o[hb][cb] *= alpha;
    }
    float pr[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[mb][r] = fast_exp2(x[mb][r] - st.m[hb]);
        st.l[hb] += pr[mb][r];
      }
    pf[hb].u = make_uint4(pack_bf16x2(pr[0][0], pr[0][1]), pack_bf16x2(pr[0][2], pr[0][3]),
                          pack_bf16x2(pr[1][0], pr[1][1]), pack_bf16x2(pr[1][2], pr[1][3]));
  }
  // V^T fragment of column block cb: transposed reads of rows vr (slots 8g..8g+3) and
  // vr + 16 (slots 8g+4..8g+7), columns 16cb + 4(l16 % 4) .. +3 = chunk 2cb + vh, half
  // l16 & 1 of it, the chunk found at position (2cb + vc) mod 32, vc = vh + 2vr + 16 (vr & 1);
  // each fragment serves all the wave's head blocks
  const int vc_t = opaque(vc);  // formed per tile, so the 16 positions are not kept live
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) {
    const int pos = (2 * cb + vc_t) & 31;
    const char* a = vt + vrow + 16 * pos;
    Frag8 va;
    const uint2 lo = lds_read_tr16(a);
    const uint2 hi = lds_read_tr16(a + 16 * TROW);
    va.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) st.o[hb][cb] = mfma_16x16x32(va, pf[hb], st.o[hb][cb]);
  }
}

__device__ __forceinline__ void store4(uint16_t* dst, const f32x4_t& v) {
  uint2 r;
  r.x = pack_bf16x2(v[0], v[1]);
  r.y = pack_bf16x2(v[2], v[3]);
  *(uint2*)dst = r;
}

// grid: (row r = b*Tq + i) x (head group of 64) x (split); n_split == 1 writes out directly.
// ALIAS: the value rows are the key rows (one gathered tile per step); otherwise a second tile
// of value rows is gathered beside it.
// Two waves per SIMD: the register budget is 256 per lane.
template <bool ALIAS>
__global__ __launch_bounds__(64 * waves_of<ALIAS>()) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sparse_kernel(SparseParams p, int n_split, int chunk, float* part_o, float* part_ml) {
  constexpr int NW = waves_of<ALIAS>();
  constexpr int NHB = 64 / (16 * NW);  // 16-head blocks per wave
  __shared__ __attribute__((aligned(1024))) char kt0[KTILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char kt1[KTILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vt0[ALIAS ? 16 : TILE];
  __shared__ __attribute__((aligned(1024))) char vt1[ALIAS ? 16 : TILE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int n_hg = p.H / 64;
  const int sp = blockIdx.x % n_split;
  const int hg = (blockIdx.x / n_split) % n_hg;
  const int r = blockIdx.x / (n_split * n_hg);
  const int b = r / p.Tq;
  const int j_begin = sp * chunk, j_end = min(p.k, j_begin + chunk);
  const int n_tiles = max(0, (j_end - j_begin + KT - 1) / KT);
  const int h0 = hg * 64 + 16 * NHB * wave + l16;  // this lane's head in block 0 (MFMA column)

  Frag8 qf[NHB][8];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const uint16_t* qr = (const uint16_t*)p.q + ((size_t)r * p.H + h0 + 16 * hb) * D;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[hb][kk].u = *(const uint4*)(qr + 32 * kk + 8 * g);
  }
  WaveState<NHB> st;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) st.o[hb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    st.m[hb] = NEG_BIG;
    st.l[hb] = 0.f;
  }
  const float scale_log2 = p.scale * LOG2E;

  // lane-constant LDS offsets: key reads (row l16 / l16 + 16, chunk 4kk + g) and transposed
  // value reads (rows 4g + l16/4 and +16, chunk 2cb + (l16 & 3)/2, half l16 & 1)
  const int kr = l16 * TROW, kcol = g + 2 * l16 + 16 * (l16 & 1);
  const int vr = 4 * g + (l16 >> 2);
  const int vrow = vr * TROW + 8 * (l16 & 1);
  const int vcol = ((l16 & 3) >> 1) + 2 * vr + 16 * (vr & 1);

  const int32_t* idx = p.idx + (size_t)r * p.k;
  const uint16_t* kl = (const uint16_t*)p.k_lat + (size_t)b * p.S * p.k_stride;
  const uint16_t* vl = (const uint16_t*)p.v_lat + (size_t)b * p.S * p.v_stride;

  // prologue: tile 0 in flight, the positions of tile 1 loaded
  const int ix_cur = valid_ix(load_ix(idx, j_begin, j_end, lane), p.S);
  uint32_t valid_cur = (uint32_t)__ballot(ix_cur >= 0);
  if (n_tiles > 0) {
    gather_tile<NW>(kl, p.k_stride, ix_cur, kt0, wave, lane);
    if (!ALIAS) gather_tile<NW>(vl, p.v_stride, ix_cur, vt0, wave, lane);
  }
  int ix_nxt = load_ix(idx, j_begin + KT, j_end, lane);
  wait_all();
  __syncthreads();

  auto body = [&](int ti, const char* kc, const char* vc, char* kn, char* vn) {
    uint32_t valid_nxt = 0;
    if (ti + 1 < n_tiles) {
      const int ixv = valid_ix(ix_nxt, p.S);
      valid_nxt = (uint32_t)__ballot(ixv >= 0);
      gather_tile<NW>(kl, p.k_stride, ixv, kn, wave, lane);
      if (!ALIAS) gather_tile<NW>(vl, p.v_stride, ixv, vn, wave, lane);
    }
    const int ix_after = load_ix(idx, j_begin + KT * (ti + 2), j_end, lane);
    f32x4_t s[NHB][2];
    scores(s, qf, kc, kr, kcol);
    softmax_pv(st, s, ALIAS ? kc : vc, valid_cur, scale_log2, vrow, vcol, lane);
    wait_all();  // this wave's gathers of tile ti + 1 and the positions of tile ti + 2
    __syncthreads();
    valid_cur = valid_nxt;
    ix_nxt = ix_after;
  };
  for (int ti = 0; ti < n_tiles; ti += 2) {
    body(ti, kt0, vt0, kt1, vt1);
    if (ti + 1 < n_tiles) body(ti + 1, kt1, vt1, kt0, vt0);
  }

  // Epilogue.  When p.q_lat is set (the launcher passes it only with the head mix), out
  // already holds the gate factors sigmoid(q_lat W) of this row (written by the gate GEMM
  // before this kernel): the output is O * sigmoid(G).  With the head mix (VHA) that gated
  // output of all 64 heads is staged in the key tiles (the last barrier of the key loop has
  // freed them), mixed across heads in place and stored row by row.
  const bool gated = p.q_lat != nullptr;
  const bool mix = n_split == 1 && p.vha_r > 0;
  auto mrow = [&](int hl) -> char* { return (hl < 32 ? kt0 : kt1) + (hl & 31) * MIX_ROW; };
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const int h = h0 + 16 * hb;
    const float lt = wave_sum16(st.l[hb]);
    const bool seen = st.m[hb] > 0.5f * NEG_BIG;
    if (n_split == 1) {
      const float inv = (seen && lt > 0.f) ? 1.f / lt : 0.f;
      uint16_t* orow = (uint16_t*)p.out + ((size_t)r * p.H + h) * D;
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) {
        f32x4_t v = st.o[hb][cb] * inv;
        if (gated) {
          const uint2 sg = *(const uint2*)(orow + 16 * cb + 4 * g);
          v[0] *= __uint_as_float(sg.x << 16);
          v[1] *= __uint_as_float(sg.x & 0xFFFF0000u);
          v[2] *= __uint_as_float(sg.y << 16);
          v[3] *= __uint_as_float(sg.y & 0xFFFF0000u);
        }
        if (mix)
          store4((uint16_t*)(mrow(h - hg * 64) + (16 * cb + 4 * g) * 2), v);
        else
          store4(orow + 16 * cb + 4 * g, v);
      }
      if (p.lse != nullptr && g == 0)
        p.lse[(size_t)r * p.H + h] = inv > 0.f ? (st.m[hb] + __log2f(lt)) * LN2 : -INFINITY;
      continue;
    }
    const size_t pr = ((size_t)r * n_split + sp) * p.H + h;
    float* po = part_o + pr * D;
    // a split that saw no valid key contributes nothing: max -inf, sum 0, O 0
    const float keep = seen ? 1.f : 0.f;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) *(f32x4_t*)(po + 16 * cb + 4 * g) = st.o[hb][cb] * keep;
    if (g == 0) {
      part_ml[pr * 2 + 0] = seen ? st.m[hb] : -INFINITY;
      part_ml[pr * 2 + 1] = seen ? lt : 0.f;
    }
  }
  if (mix) {
    vha_tile::Factors f;
    vha_tile::load_factors(f, (const uint16_t*)p.vha_u, (const uint16_t*)p.vha_v, p.vha_r,
                           lane);
    __syncthreads();
    vha_tile::mix_blocks(mrow, f, (16 / NW) * wave, 16 / NW, lane);
    __syncthreads();
    // 64 rows of 512 bytes leave as 16-byte chunks
    uint16_t* out0 = (uint16_t*)p.out + ((size_t)r * p.H + hg * 64) * D;
    for (int c = tid; c < 64 * 32; c += 64 * NW)
      *(uint4*)(out0 + (size_t)(c >> 5) * D + 8 * (c & 31)) =
          *(const uint4*)(mrow(c >> 5) + 16 * (c & 31));
  }
}

// gated: out holds this row's gate factors (written before the attention kernel), which
// multiply the merged O.
__global__ __launch_bounds__(64) void sparse_combine_kernel(const float* __restrict__ part_o,
                                                            const float* __restrict__ part_ml,
                                                            uint16_t* __restrict__ out,
                                                            float* __restrict__ lse, int H,
                                                            int n_split, bool gated) {
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
  if (lse != nullptr && threadIdx.x == 0) lse[rh] = lt > 0.f ? (mt + __log2f(lt)) * LN2 : -INFINITY;
  float f[4] = {inv, inv, inv, inv};
  uint2* dst = (uint2*)(out + (size_t)rh * D + 4 * threadIdx.x);
  if (gated) {
    const uint2 sg = *dst;
    f[0] *= __uint_as_float(sg.x << 16);
    f[1] *= __uint_as_float(sg.x & 0xFFFF0000u);
    f[2] *= __uint_as_float(sg.y << 16);
    f[3] *= __uint_as_float(sg.y & 0xFFFF0000u);
  }
  uint2 o;
  o.x = pack_bf16x2(acc[0] * f[0], acc[1] * f[1]);
  o.y = pack_bf16x2(acc[2] * f[2], acc[3] * f[3]);
  *dst = o;
}

// Enough workgroups to fill the chip before a list is split, but at least four tiles per
// split: shorter pieces cost more in partial results and merging than they gain.
void sparse_plan(const SparseParams& p, int& n_split, int& chunk) {
  const long long wgs = (long long)p.B * p.Tq * (p.H / 64);
  const long long target = 1024;
  long long want = wgs >= target ? 1 : (target + wgs - 1) / wgs;
  const long long max_split = std::max<long long>(1, p.k / (4 * KT));
  n_split = (int)std::max<long long>(1, std::min(want, max_split));
  long long c = (p.k + n_split - 1) / n_split;
  c = (c + KT - 1) / KT * KT;
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
  hipError_t e;
  // With the head mix the gate must precede it inside the epilogue: the gate factors are
  // computed first, into out, where the epilogue reads them.  Without it the gate GEMM rescales
  // the attention output in place afterwards (the same bytes moved, measured 3% faster at the
  // DSA prefill shape).
  const bool gate_first = p.q_lat != nullptr && p.vha_r > 0;
  SparseParams pk = p;
  if (!gate_first) pk.q_lat = nullptr;  // the kernels read no gate factors
  if (gate_first) {
    e = launch_gate(p.q_lat, p.w_gate, nullptr, p.out, (int)rows, p.d_lat, p.H * D, DT_BF16,
                    stream);
    if (e != hipSuccess) return e;
  }
  const long long grid = rows * (p.H / 64) * n_split;
  const bool alias = p.v_lat == p.k_lat && p.v_stride == p.k_stride;
  if (alias)
    hipLaunchKernelGGL(sparse_kernel<true>, dim3((unsigned)grid), dim3(64 * waves_of<true>()), 0,
                       stream, pk, n_split, chunk, part_o, part_ml);
  else
    hipLaunchKernelGGL(sparse_kernel<false>, dim3((unsigned)grid), dim3(64 * waves_of<false>()), 0,
                       stream, pk, n_split, chunk, part_o, part_ml);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (n_split > 1) {
    hipLaunchKernelGGL(sparse_combine_kernel, dim3((unsigned)(rows * p.H)), dim3(64), 0, stream,
                       part_o, part_ml, (uint16_t*)p.out, p.lse, p.H, n_split, gate_first);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.q_lat != nullptr && !gate_first) {
    e = launch_gate(p.q_lat, p.w_gate, p.out, p.out, (int)rows, p.d_lat, p.H * D, DT_BF16,
                    stream);
    if (e != hipSuccess) return e;
  }
  // a merged row's head mix (the merge works per head) runs as its own pass
  if (p.vha_r > 0 && n_split > 1)
    return launch_vha(p.out, p.vha_u, p.vha_v, p.out, (int)rows, p.H, D, p.vha_r, DT_BF16,
                      stream);
  return hipSuccess;
}

}  // namespace lgsa

// ------------------------------------------------------------------ gather probe (measurement)
namespace lgsa {
namespace {

using namespace sparse_tile;

// The gathers of sparse_kernel<true> alone: one workgroup of two waves per index list, tiles of
// 32 listed rows brought to LDS by the same DMA pattern and double buffering.  So that the
// transfers are used, wave w adds up the first 64 words of tile row 16 w of every tile (rows 0
// and 16 are stored unrotated), uint32 with wrap-around: sums[list][w].
__global__ __launch_bounds__(128) void gather_probe_kernel(const uint16_t* __restrict__ rows,
                                                           long long stride, int S,
                                                           const int32_t* __restrict__ idx,
                                                           int k, uint32_t* __restrict__ sums) {
  __shared__ __attribute__((aligned(1024))) char t0[TILE];
  __shared__ __attribute__((aligned(1024))) char t1[TILE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t* list = idx + (size_t)blockIdx.x * k;
  const int n_tiles = (k + KT - 1) / KT;
  uint32_t sum = 0;
  if (n_tiles > 0) gather_tile<2>(rows, stride, valid_ix(load_ix(list, 0, k, lane), S), t0, wave, lane);
  int ix_nxt = load_ix(list, KT, k, lane);
  wait_all();
  __syncthreads();
  auto body = [&](int ti, const char* cur, char* nxt) {
    if (ti + 1 < n_tiles) gather_tile<2>(rows, stride, valid_ix(ix_nxt, S), nxt, wave, lane);
    const int ix_after = load_ix(list, KT * (ti + 2), k, lane);
    sum += *(const uint32_t*)(cur + 16 * wave * TROW + 4 * lane);
    wait_all();
    __syncthreads();
    ix_nxt = ix_after;
  };
  for (int ti = 0; ti < n_tiles; ti += 2) {
    body(ti, t0, t1);
    if (ti + 1 < n_tiles) body(ti + 1, t1, t0);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane == 0) sums[(size_t)blockIdx.x * 2 + wave] = sum;
}

}  // namespace

hipError_t launch_gather_probe(const void* rows, long long stride, int S, const int32_t* idx,
                               int n_lists, int k, uint32_t* sums, hipStream_t stream) {
  if (n_lists == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_probe_kernel, dim3((unsigned)n_lists), dim3(128), 0, stream,
                     (const uint16_t*)rows, stride, S, idx, k, sums);
  return hipGetLastError();
}

}  // namespace lgsa
