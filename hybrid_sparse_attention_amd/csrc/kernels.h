// Host-side launchers of the gfx950 kernels.  Arguments are validated by the C-ABI layer
// (api.cpp) before any of these is called; the launchers only size grids and enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lgsa {

enum { DT_F32 = 0, DT_BF16 = 1 };

hipError_t launch_compress(const void* k, const void* v, void* kc, void* vc, int B, int T,
                           int d, int block, int dt, hipStream_t stream);

// Decode-time cache appends (cache.hip).
hipError_t launch_hca_append(const int32_t* pos, const void* k_new, const void* v_new,
                             void* k_win, void* v_win, void* kc, void* vc, int B, int d,
                             int win_len, int n_cap, int block, int dt, hipStream_t stream);
hipError_t launch_dsa_append(const int32_t* pos, int B, int S, const float* k_idx_new,
                             float* k_idx, int di, const void* kv_new, void* kv_lat, int row,
                             long long stride, int dt, hipStream_t stream);

// Virtual Head Attention mixing step (vha.hip): out = o + U V^T o over the heads of each
// token; out may equal o.
hipError_t launch_vha(const void* o, const void* u, const void* v, void* out, int M, int H,
                      int d, int r, int dt, hipStream_t stream);

// out[m, n] = o[m, n] * sigmoid(q_lat[m, :] . w[:, n]); out may equal o.
// Backward, first step of the gate: do = dout * s into d_o, dG = dout * o * s * (1 - s) into dg.
hipError_t launch_gate_bwd_elem(const void* q_lat, const void* w, const void* o,
                                const void* dout, void* d_o, void* dg, int M, int d_lat, int N,
                                int dt, hipStream_t stream);
// C[m][n] = sum_k A(m, k) B(k, n) (see gemm.hip for the two operand layouts).
hipError_t launch_gemm(const void* a, long long lda, bool a_kmajor, const void* b,
                       long long ldb, bool b_kmajor, void* c, long long ldc, int M, int N, int K,
                       int dt, hipStream_t stream);
// bfloat16 with o == NULL: out = sigmoid(q_lat w), the gate factors alone.
hipError_t launch_gate(const void* q_lat, const void* w, const void* o, void* out, int M,
                       int d_lat, int N, int dt, hipStream_t stream);

struct HcaParams {
  int B, Tq, H, d;
  const void* q;
  const int32_t* pos0;
  int max_pos;
  const void* k_win;
  const void* v_win;
  int win_len, window;
  const void* kc;
  const void* vc;
  int n_cap, block;
  float scale;
  const void* q_lat;
  const void* w_gate;
  int d_lat;
  void* out;
  void* ws;
  size_t ws_bytes;
  float* lse;  // optional per-row log-sum-exp of the scaled logits (prefill kernel only)
  const void* vha_u;  // Virtual Head Attention factors [H, vha_r], applied to the gated output
  const void* vha_v;
  int vha_r;          // 0: no mixing
};

// Backward of HCA in prefill (every sequence from position 0, T query rows = T positions):
// the window rows are the sequence's own keys and values, the entries their block means.
struct HcaBwdParams {
  int B, T, H;  // d == 512, bfloat16
  const void* q;
  const void* k;
  const void* v;
  const void* kc;
  const void* vc;
  const void* out;
  const float* lse;
  const void* dout;
  int window, block, ne;  // ne = T / block entries
  float scale;
  void* dq;
  void* dk;
  void* dv;
  void* ws;
  size_t ws_bytes;
};
size_t hca_bwd_workspace(const HcaBwdParams& p);
hipError_t launch_hca_bwd(const HcaBwdParams& p, hipStream_t stream);
hipError_t launch_gemm_splitk_f32(const void* a, long long lda, bool a_kmajor, const void* b,
                                  long long ldb, bool b_kmajor, float* c, int M, int N, int K,
                                  int splits, float* part, hipStream_t stream);

// bfloat16, d == 512
size_t hca_bf16_workspace(const HcaParams& p);
hipError_t launch_hca_bf16(const HcaParams& p, hipStream_t stream);
// float32, d <= 512
size_t hca_f32_workspace(const HcaParams& p);
hipError_t launch_hca_f32(const HcaParams& p, hipStream_t stream);

struct IndexParams {
  int B, Tq, S, Hi, di, k;
  const float* q_idx;
  const float* w_idx;
  const float* k_idx;
  const int32_t* pos0;
  int max_pos;
  int32_t* idx_out;
  void* ws;
  size_t ws_bytes;
  int block;  // positions per key (>= 1): key s visible to position t iff s < (t + 1) / block
};

size_t index_workspace(const IndexParams& p);      // recommended size
size_t index_min_workspace(const IndexParams& p);  // smallest size a call accepts
hipError_t launch_index(const IndexParams& p, hipStream_t stream);

struct SparseParams {
  int B, Tq, H, d_qk, d_v, S, k;
  const void* q;
  const void* k_lat;
  long long k_stride;
  const void* v_lat;
  long long v_stride;
  const int32_t* idx;
  float scale;
  const void* q_lat;
  const void* w_gate;
  int d_lat;
  void* out;
  void* ws;
  size_t ws_bytes;
  float* lse;
  const void* vha_u;  // Virtual Head Attention factors [H, vha_r], applied to the gated output
  const void* vha_v;
  int vha_r;          // 0: no mixing
};

size_t sparse_workspace(const SparseParams& p);
// Measurement helper: the gathers of sparse attention alone (one checksum pair per list).
hipError_t launch_gather_probe(const void* rows, long long stride, int S, const int32_t* idx,
                               int n_lists, int k, uint32_t* sums, hipStream_t stream);
hipError_t launch_sparse(const SparseParams& p, hipStream_t stream);

struct SparseBwdParams {
  int B, Tq, H, S, k;
  const void* q;
  const void* k_lat;
  long long k_stride;
  const void* v_lat;
  long long v_stride;
  const int32_t* idx;
  float scale;
  const void* out;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;  // NULL: the value rows are the key rows
  void* ws;
  size_t ws_bytes;
};

size_t sparse_bwd_workspace(const SparseBwdParams& p);      // rows of a sequence at once, within a budget
size_t sparse_bwd_min_workspace(const SparseBwdParams& p);  // one row at a time
hipError_t launch_sparse_bwd(const SparseBwdParams& p, hipStream_t stream);

}  // namespace lgsa
