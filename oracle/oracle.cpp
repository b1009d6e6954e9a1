// Independent fp64 CPU oracle for the Latent-Gated Sparse Attention forward pass.
//
// TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline leg
// of the benchmark may load this library.  It shares no source with the HIP library and is
// built by g++ alone.  It is deliberately plain and slow: every function follows the
// definition it cites, one element at a time, with every input widened to double.
//
// Sources (cited by page title and section):
//   [blog 2.1]  ERNIE 5.5 Flash Base release blog, section 2.1 "Latent-Gated Sparse
//               Attention" (Japanese edition "BaiduがERNIE 5.5 Flash Baseを公開";
//               Chinese original "ERNIE 5.5 Flash Base 正式发布").
//   [xeno]      xenospectrum.com article on ERNIE 5.5 Flash Base, section
//               "活性140億パラメータと長文処理を支える仕組み" (37 HCA layers, a 128-token
//               uncompressed sliding window).
// Where the pages leave a step open, the reading taken here is the plainest one (block mean
// pool, complete blocks only, no de-duplication between window and compressed entries,
// lower index wins top-k ties, -0.0 equals +0.0); each such reading is listed in the
// project's design notes.
//
// Dtype codes for every tensor argument: 0 = float32, 1 = bfloat16 (raw uint16 bits),
// 2 = float64.  Index tensors are int32.  All outputs are float64.
// Every function returns 0 on success and a negative number on a bad argument.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

namespace {

enum { DT_F32 = 0, DT_BF16 = 1, DT_F64 = 2 };

// Reads element i of a tensor stored as dtype dt and returns it as a double.
// bfloat16 is the upper half of an IEEE float32, so its bits shift into place exactly.
double widen(const void* p, int dt, long long i) {
  if (dt == DT_F32) return (double)((const float*)p)[i];
  if (dt == DT_BF16) {
    uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    std::memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return ((const double*)p)[i];
}

bool dt_ok(int dt) { return dt == DT_F32 || dt == DT_BF16 || dt == DT_F64; }

double logistic(double g) { return 1.0 / (1.0 + std::exp(-g)); }

// Softmax attention of one query row over an explicit list of (key row, value row) offsets:
//   l_j = scale * <q, K_j>;  p_j = exp(l_j - max_j l_j);  O = sum_j p_j V_j / sum_j p_j.
// An empty list gives O = 0.
void attend(const void* q, int dt_q, long long q_off, long long dqk, long long dv,
            const void* kb, const void* vb, int dt_kv,
            const std::vector<long long>& koff, const std::vector<long long>& voff,
            double scale, double* o) {
  const size_t n = koff.size();
  for (long long j = 0; j < dv; ++j) o[j] = 0.0;
  if (n == 0) return;
  std::vector<double> qv(dqk), logit(n);
  for (long long c = 0; c < dqk; ++c) qv[c] = widen(q, dt_q, q_off + c);
  double m = -std::numeric_limits<double>::infinity();
  for (size_t j = 0; j < n; ++j) {
    double s = 0.0;
    for (long long c = 0; c < dqk; ++c) s += qv[c] * widen(kb, dt_kv, koff[j] + c);
    logit[j] = scale * s;
    m = std::max(m, logit[j]);
  }
  double l = 0.0;
  for (size_t j = 0; j < n; ++j) {
    const double p = std::exp(logit[j] - m);
    l += p;
    for (long long c = 0; c < dv; ++c) o[c] += p * widen(vb, dt_kv, voff[j] + c);
  }
  for (long long c = 0; c < dv; ++c) o[c] /= l;
}

// Low-rank output gate of [blog 2.1]: the attention output of query row `row` is multiplied,
// channel by channel, by sigma(q_lat[row] . W[:, n]) where n runs over the H*dv output
// channels (head-major).  q_lat has d_lat entries per row; W is [d_lat, H*dv] row-major.
// Each logit g[n] is summed over i in ascending order; the i loop is the outer one so that W
// is read row by row (every g[n] sees the same additions in the same order either way).
void apply_gate(const void* q_lat, const void* w, int dt_g, long long d_lat, long long n_out,
                long long row, double* o) {
  std::vector<double> g(n_out, 0.0);
  for (long long i = 0; i < d_lat; ++i) {
    const double qi = widen(q_lat, dt_g, row * d_lat + i);
    for (long long n = 0; n < n_out; ++n) g[n] += qi * widen(w, dt_g, i * n_out + n);
  }
  for (long long n = 0; n < n_out; ++n) o[n] *= logistic(g[n]);
}

}  // namespace

extern "C" {

// Block compressor of [blog 2.1] ("every 128 tokens become one cache entry"), read as a mean
// pool: entry e = (1/block) * sum_{i<block} x[e*block + i], over complete blocks only.
// x is [B, T, d]; out is [B, T/block, d].
int orc_hca_compress(const void* x, int dt, long long B, long long T, long long d,
                     long long block, double* out) {
  if (!x || !out || !dt_ok(dt) || B < 0 || T < 0 || d <= 0 || block <= 0) return -1;
  const long long ne = T / block;
#pragma omp parallel for collapse(2) schedule(static)
  for (long long b = 0; b < B; ++b)
    for (long long e = 0; e < ne; ++e)
      for (long long c = 0; c < d; ++c) {
        double s = 0.0;
        for (long long i = 0; i < block; ++i) s += widen(x, dt, (b * T + e * block + i) * d + c);
        out[(b * ne + e) * d + c] = s / (double)block;
      }
  return 0;
}

// Heavily Compressed Attention of [blog 2.1] with the window size of [xeno].
// Query row (b, i) sits at position t = pos0[b] + i and attends to
//   * compressed entry e of [kc, vc] for every e < n_cap with e*block + block - 1 <= t
//     (a block becomes visible once it is complete), and
//   * every raw position s with max(0, t - window + 1) <= s <= t, read from row s % win_len
//     of [k_win, v_win] (a ring buffer in decode; win_len = T in prefill).
// Both sets are used as they stand, also where they cover the same tokens.  All H query
// heads share the one key/value head.  If q_lat is non-null the output gate is applied.
// q [B,Tq,H,d]; k_win, v_win [B,win_len,d]; kc, vc [B,n_cap,d]; q_lat [B,Tq,d_lat];
// w_gate [d_lat, H*d]; rows lists flat query rows b*Tq + i; out is [n_rows, H, d].
int orc_hca_attn(const void* q, int dt_q, long long B, long long Tq, long long H, long long d,
                 const int* pos0, const void* k_win, const void* v_win, int dt_w,
                 long long win_len, long long window, const void* kc, const void* vc, int dt_c,
                 long long n_cap, long long block, double scale, const void* q_lat,
                 const void* w_gate, int dt_g, long long d_lat, const long long* rows,
                 long long n_rows, double* out) {
  if (!q || !pos0 || !k_win || !v_win || !out || !rows) return -1;
  if (!dt_ok(dt_q) || !dt_ok(dt_w) || (n_cap > 0 && (!kc || !vc || !dt_ok(dt_c)))) return -1;
  if (B <= 0 || Tq <= 0 || H <= 0 || d <= 0 || win_len <= 0 || window <= 0 || block <= 0)
    return -1;
  if (q_lat && (!w_gate || !dt_ok(dt_g) || d_lat <= 0)) return -1;
  for (long long r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= B * Tq) return -2;
  // Keys are taken from a mixed pair of buffers, so each visible key is addressed by a
  // (buffer, offset) pair; the compressed entries come first, then the window.
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long long r = 0; r < n_rows; ++r) {
    const long long row = rows[r], b = row / Tq, i = row % Tq;
    const long long t = (long long)pos0[b] + i;
    if (t < 0) {
#pragma omp atomic write
      err = -3;
      continue;
    }
    std::vector<long long> ce, ws;
    for (long long e = 0; e < n_cap; ++e)
      if (e * block + block - 1 <= t) ce.push_back(e);
    for (long long s = std::max(0LL, t - window + 1); s <= t; ++s) ws.push_back(s);
    const long long nk = (long long)(ce.size() + ws.size());
    // Gather the visible keys and values into contiguous float64 rows.
    std::vector<double> kk(nk * d), vv(nk * d);
    long long j = 0;
    for (long long e : ce) {
      for (long long c = 0; c < d; ++c) {
        kk[j * d + c] = widen(kc, dt_c, (b * n_cap + e) * d + c);
        vv[j * d + c] = widen(vc, dt_c, (b * n_cap + e) * d + c);
      }
      ++j;
    }
    for (long long s : ws) {
      const long long ring = s % win_len;
      for (long long c = 0; c < d; ++c) {
        kk[j * d + c] = widen(k_win, dt_w, (b * win_len + ring) * d + c);
        vv[j * d + c] = widen(v_win, dt_w, (b * win_len + ring) * d + c);
      }
      ++j;
    }
    std::vector<long long> off(nk);
    for (long long x = 0; x < nk; ++x) off[x] = x * d;
    double* o = out + r * H * d;
    for (long long h = 0; h < H; ++h)
      attend(q, dt_q, ((b * Tq + i) * H + h) * d, d, d, kk.data(), vv.data(), DT_F64, off, off,
             scale, o + h * d);
    if (q_lat) apply_gate(q_lat, w_gate, dt_g, d_lat, H * d, row, o);
  }
  return err;
}

// Stand-alone low-rank gate of [blog 2.1]: out[m, n] = o[m, n] * sigma(q_lat[m] . W[:, n]).
// q_lat [M, d_lat]; w [d_lat, N]; o [M, N]; out [n_rows, N] for the listed rows m.
int orc_latent_gate(const void* q_lat, int dt_l, const void* w, int dt_w, const void* o,
                    int dt_o, long long M, long long d_lat, long long N, const long long* rows,
                    long long n_rows, double* out) {
  if (!q_lat || !w || !o || !out || !rows || !dt_ok(dt_l) || !dt_ok(dt_w) || !dt_ok(dt_o))
    return -1;
  if (M < 0 || d_lat <= 0 || N <= 0) return -1;
  for (long long r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= M) return -2;
#pragma omp parallel for schedule(dynamic, 1)
  for (long long r = 0; r < n_rows; ++r) {
    const long long m = rows[r];
    std::vector<double> g(N, 0.0);  // g[n] summed over i in ascending order, W read by rows
    for (long long i = 0; i < d_lat; ++i) {
      const double qi = widen(q_lat, dt_l, m * d_lat + i);
      for (long long n = 0; n < N; ++n) g[n] += qi * widen(w, dt_w, i * N + n);
    }
    for (long long n = 0; n < N; ++n) out[r * N + n] = widen(o, dt_o, m * N + n) * logistic(g[n]);
  }
  return 0;
}

// Lightweight indexer of [blog 2.1] in the form taken here:
//   score(t, s) = sum_{h < Hi} w[t, h] * max(0, <q_I[t, h], k_I[s]>),
// evaluated in float64 from float32 inputs for s in [s0, s1) of query row (b, i).
// q_idx [B,Tq,Hi,di]; w_idx [B,Tq,Hi]; k_idx [B,S,di]; out has s1 - s0 entries.
int orc_dsa_scores(const float* q_idx, const float* w_idx, const float* k_idx, long long B,
                   long long Tq, long long S, long long Hi, long long di, long long b,
                   long long i, long long s0, long long s1, double* out) {
  if (!q_idx || !w_idx || !k_idx || !out) return -1;
  if (b < 0 || b >= B || i < 0 || i >= Tq || s0 < 0 || s1 > S || s0 > s1) return -2;
  for (long long s = s0; s < s1; ++s) {
    double score = 0.0;
    for (long long h = 0; h < Hi; ++h) {
      double dot = 0.0;
      for (long long c = 0; c < di; ++c)
        dot += (double)q_idx[((b * Tq + i) * Hi + h) * di + c] *
               (double)k_idx[(b * S + s) * di + c];
      score += (double)w_idx[(b * Tq + i) * Hi + h] * std::max(0.0, dot);
    }
    out[s - s0] = score + 0.0;  // adding +0.0 turns a -0.0 into +0.0
  }
  return 0;
}

// Per-query top-k of [blog 2.1]: among the keys visible to the query at t = pos0[b] + i,
// keep the k highest scores, the lower key winning a tie; when at most k keys are visible
// every one is kept.  With block == 1 the keys are token positions and key s is visible
// when s <= t (DSA).  With block > 1 key s is the compressed entry of positions
// block*s .. block*s + block - 1 (the compressed sparse variant of [blog 2.1]: history
// compressed, then a sparse part of it attended), visible once its block is complete,
// block*s + block - 1 <= t; there are (t + 1) / block of them, and that many keys must
// exist (at most S).  The kept keys are written in ascending order and the remaining slots
// hold -1.  kth_score[r] receives the k-th highest score (the selection threshold), or -inf
// when every visible key is kept.  idx_out is [n_rows, k] int32.
int orc_dsa_topk(const float* q_idx, const float* w_idx, const float* k_idx, long long B,
                 long long Tq, long long S, long long Hi, long long di, long long k,
                 long long block, const int* pos0, const long long* rows, long long n_rows,
                 int* idx_out, double* kth_score) {
  if (!q_idx || !w_idx || !k_idx || !pos0 || !rows || !idx_out || k <= 0 || block <= 0)
    return -1;
  for (long long r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= B * Tq) return -2;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long long r = 0; r < n_rows; ++r) {
    const long long b = rows[r] / Tq, i = rows[r] % Tq;
    const long long t = (long long)pos0[b] + i;
    int* dst = idx_out + r * k;
    const long long n = t < 0 ? 0 : (t + 1) / block;  // visible keys
    if (t < 0 || n > S) {
#pragma omp atomic write
      err = -3;
      continue;
    }
    std::vector<long long> keep;
    double kth = -std::numeric_limits<double>::infinity();
    if (n <= k) {
      for (long long s = 0; s < n; ++s) keep.push_back(s);
    } else {
      std::vector<double> sc(n);
      orc_dsa_scores(q_idx, w_idx, k_idx, B, Tq, S, Hi, di, b, i, 0, n, sc.data());
      std::vector<long long> order(n);
      for (long long s = 0; s < n; ++s) order[s] = s;
      // Higher score first; equal scores in ascending position order.
      std::sort(order.begin(), order.end(), [&](long long a, long long c) {
        if (sc[a] != sc[c]) return sc[a] > sc[c];
        return a < c;
      });
      keep.assign(order.begin(), order.begin() + k);
      kth = sc[order[k - 1]];
      std::sort(keep.begin(), keep.end());
    }
    for (long long j = 0; j < k; ++j) dst[j] = j < (long long)keep.size() ? (int)keep[j] : -1;
    if (kth_score) kth_score[r] = kth;
  }
  return err;
}

// Sparse core attention of [blog 2.1] (DSA in the MLA layers): query row (b, i), head h,
// attends with softmax to the latent rows listed in idx[b, i, :]; negative entries and
// entries >= S are skipped, every other entry is one key (listed twice, counted twice).
// The key of position s is k_lat[b*S*k_stride + s*k_stride + 0 .. dqk) and its value is
// v_lat[b*S*v_stride + s*v_stride + 0 .. dv); v_lat may be the same buffer as k_lat.
// q [B,Tq,H,dqk]; idx [B,Tq,k] int32; q_lat [B,Tq,d_lat]; w_gate [d_lat, H*dv];
// out [n_rows, H, dv].  With no valid entry the output row is zero.
int orc_sparse_attn(const void* q, int dt_q, long long B, long long Tq, long long H,
                    long long dqk, long long dv, const void* k_lat, long long k_stride,
                    const void* v_lat, long long v_stride, int dt_kv, long long S,
                    const int* idx, long long k, double scale, const void* q_lat,
                    const void* w_gate, int dt_g, long long d_lat, const long long* rows,
                    long long n_rows, double* out) {
  if (!q || !k_lat || !v_lat || !idx || !rows || !out || !dt_ok(dt_q) || !dt_ok(dt_kv))
    return -1;
  if (B <= 0 || Tq <= 0 || H <= 0 || dqk <= 0 || dv <= 0 || S <= 0 || k <= 0) return -1;
  if (k_stride < dqk || v_stride < dv) return -1;
  if (q_lat && (!w_gate || !dt_ok(dt_g) || d_lat <= 0)) return -1;
  for (long long r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= B * Tq) return -2;
#pragma omp parallel for schedule(dynamic, 1)
  for (long long r = 0; r < n_rows; ++r) {
    const long long row = rows[r], b = row / Tq;
    std::vector<long long> koff, voff;
    for (long long j = 0; j < k; ++j) {
      const long long s = idx[row * k + j];
      if (s < 0 || s >= S) continue;
      koff.push_back((b * S + s) * k_stride);
      voff.push_back((b * S + s) * v_stride);
    }
    double* o = out + r * H * dv;
    for (long long h = 0; h < H; ++h)
      attend(q, dt_q, (row * H + h) * dqk, dqk, dv, k_lat, v_lat, dt_kv, koff, voff, scale,
             o + h * dv);
    if (q_lat) apply_gate(q_lat, w_gate, dt_g, d_lat, H * dv, row, o);
  }
  return 0;
}

}  // extern "C"
