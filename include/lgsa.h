/*
 * lgsa.h -- C ABI of the Latent-Gated Sparse Attention forward library for AMD gfx950.
 *
 * The library implements the attention forward pass of the ERNIE 5.5 Flash layers as the
 * pages describe it:
 *   - Heavily Compressed Attention (HCA): each query attends densely to one cache entry per
 *     completed block of 128 tokens plus a window of the most recent raw tokens, with 512-wide
 *     heads (ERNIE 5.5 Flash Base release blog, section 2.1 "Latent-Gated Sparse Attention";
 *     the 128-token window size is from the xenospectrum.com article on ERNIE 5.5 Flash Base,
 *     long-context section);
 *   - DeepSeek Sparse Attention (DSA) in the MLA layers: a lightweight indexer scores every
 *     past position, and core attention with 256-wide heads runs only on the top-k positions
 *     (release blog, section 2.1);
 *   - the low-rank output gate: the attention output is multiplied by a gate computed from
 *     the query latent, which is 4x narrower than the hidden state (release blog, section
 *     2.1, "low-rank gated attention").
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers (memory of the current HIP device), row-major
 *     with the last dimension contiguous, unless a field says "host".
 *   - The caller owns every buffer.  The library allocates nothing, keeps no pointer after a
 *     call returns and never synchronises the stream: work is only enqueued on `stream`
 *     (a hipStream_t passed as void*; NULL means the default stream).  Buffers must stay
 *     alive until that work has completed.  Faults inside kernels surface at the caller's
 *     next synchronisation, as for any HIP call.
 *   - Scratch memory is passed in by the caller: query its size with the matching
 *     *_workspace() call.  A workspace pointer may be NULL only when the query returns 0.
 *   - Every call validates its arguments on the host before it enqueues anything; on error
 *     it returns a negative status, enqueues nothing, and lgsa_last_error() describes the
 *     problem.  No C++ exception crosses the ABI.
 *   - Results are deterministic: no floating-point atomics, two identical calls give
 *     bit-identical outputs.
 *   - Calls are thread-safe and re-entrant (the error message is thread-local).
 */
#ifndef LGSA_H
#define LGSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int lgsa_status;
#define LGSA_OK 0
#define LGSA_EINVAL (-1)       /* a pointer, size or relation between sizes is invalid */
#define LGSA_EUNSUPPORTED (-2) /* valid, but outside the shapes/dtypes the library implements */
#define LGSA_EWORKSPACE (-3)   /* workspace missing or smaller than the *_workspace query */
#define LGSA_EHIP (-4)         /* the HIP runtime refused a launch */

/* Element type of the floating-point tensors of a call. */
#define LGSA_F32 0
#define LGSA_BF16 1

/* Message of the last non-OK status returned on this thread ("" if none). */
const char* lgsa_last_error(void);

/* ---------------------------------------------------------------------------------------
 * hca_compress -- the HCA block compressor (release blog, section 2.1: every 128 tokens are
 * compressed into one cache entry).  The compressor is read as a mean pool over complete
 * blocks:  kc[b, e, :] = (1/block) * sum_{i<block} k[b, e*block + i, :], and likewise vc from
 * v.  Accumulation is in fp32; results are stored in `dt`.
 *   k, v   [B, T, d]            input keys and values (dt)
 *   kc, vc [B, T/block, d]      outputs (dt); a trailing incomplete block is not written
 *                               (kc, vc may be NULL when T < block: nothing is written)
 * Supported: dt LGSA_F32 (d % 4 == 0) or LGSA_BF16 (d % 8 == 0); block >= 1.
 * ------------------------------------------------------------------------------------- */
lgsa_status hca_compress(const void* k, const void* v, void* kc, void* vc, int B, int T, int d,
                         int block, int dt, void* stream);

/* ---------------------------------------------------------------------------------------
 * latent_gate -- the low-rank output gate (release blog, section 2.1):
 *     out[m, n] = o[m, n] * sigmoid( sum_i q_lat[m, i] * w_gate[i, n] )
 * with fp32 accumulation; sigmoid(g) = 1 / (1 + exp(-g)).
 *   q_lat  [M, d_lat]   query latent rows (dt)
 *   w_gate [d_lat, N]   gate projection (dt)
 *   o      [M, N]       attention output (dt);  out [M, N] (dt).  out may equal o.
 * Supported: LGSA_BF16 with d_lat % 64 == 0 and N % 16 == 0 (every tensor 16-byte
 * aligned); LGSA_F32 with any sizes.  M == 0 enqueues nothing.
 * ------------------------------------------------------------------------------------- */
lgsa_status latent_gate(const void* q_lat, const void* w_gate, const void* o, void* out, int M,
                        int d_lat, int N, int dt, void* stream);

/* ---------------------------------------------------------------------------------------
 * latent_gate_bwd -- backward of latent_gate (the chain rule of its definition): with
 * G = q_lat w_gate and s = sigmoid(G), so that out = o * s, and dout the gradient of a loss
 * with respect to out,
 *     d_o = dout * s,   dG = dout * o * s * (1 - s),   dq_lat = dG w_gate^T,   dw_gate = q_lat^T dG.
 *   q_lat [M, d_lat], w_gate [d_lat, N], o and dout [M, N] (dt, read);
 *   d_o [M, N], dq_lat [M, d_lat], dw_gate [d_lat, N] (dt, written; d_o may equal dout).
 * G is recomputed, not stored by the forward.  dG is kept in the workspace, in dt:
 * latent_gate_bwd_workspace() bytes (M * N elements).  fp32 accumulation; the bf16 path rounds
 * dG to bf16 before the two products.  Supported: as latent_gate (LGSA_BF16: d_lat % 64 == 0,
 * N % 16 == 0, every pointer 16-byte aligned).  Errors: LGSA_EINVAL for NULL or misaligned
 * pointers and bad sizes, LGSA_EWORKSPACE for a missing or short workspace; nothing is
 * enqueued on error.  M == 0 writes zeros to dw_gate.
 * --------------------------------------------------------------------------------------- */
lgsa_status latent_gate_bwd(const void* q_lat, const void* w_gate, const void* o,
                            const void* dout, void* d_o, void* dq_lat, void* dw_gate, int M,
                            int d_lat, int N, int dt, void* workspace, size_t workspace_bytes,
                            void* stream);
lgsa_status latent_gate_bwd_workspace(int M, int d_lat, int N, int dt, size_t* bytes);

/* ---------------------------------------------------------------------------------------
 * hca_attn_fwd -- Heavily Compressed Attention forward (release blog, section 2.1; window
 * size from the xenospectrum.com article).  Query row i of sequence b sits at position
 * t = pos0[b] + i and attends, with one shared key/value head for all H query heads, to
 *   - compressed entry e < n_cap when e*block + block - 1 <= t (its block is complete), and
 *   - raw position s for max(0, t - window + 1) <= s <= t, read from row s % win_len of
 *     k_win / v_win (prefill: win_len = T and the raw k, v; decode: a ring of >= window rows).
 * Both sets are used as they stand, also where they cover the same tokens.
 *   O[b,i,h,:] = sum_j softmax_j(scale * <q[b,i,h,:], key_j>) * value_j
 * and, when q_lat is non-NULL, out = O * sigmoid(q_lat[b,i,:] . w_gate[:, h*d + c]);
 * otherwise out = O.  bf16 prefill (Tq > 1) computes the gate in the attention kernel's own
 * epilogue (O never goes to memory).  bf16 decode (Tq == 1) with B <= 64 and d_lat == 1024
 * merges the key splits of the attention in the gate kernel's epilogue, which multiplies the
 * merged O, rounded to bf16, by sigmoid(q_lat W).  Other decode shapes and fp32 run the gate
 * GEMM as a second kernel that rescales out in place, exactly what latent_gate(q_lat, w_gate,
 * out, out, B*Tq, d_lat, H*d) does.  All give the result of the unfused calls: O stored in the
 * output type, then latent_gate.
 * --------------------------------------------------------------------------------------- */
typedef struct {
  int dt;              /* LGSA_F32 or LGSA_BF16: q, k_win, v_win, kc, vc, q_lat, w_gate, out */
  int B, Tq, H, d;     /* sequences, query rows per sequence, query heads, head dim */
  const void* q;       /* [B, Tq, H, d] */
  const int32_t* pos0; /* device [B]: position of query row 0 of each sequence (>= 0) */
  int max_pos;         /* host: an upper bound of pos0[b] + Tq - 1 over b (sizes the launch
                          and is checked against n_cap and win_len) */
  const void* k_win;   /* [B, win_len, d] raw keys, position p in row p % win_len */
  const void* v_win;   /* [B, win_len, d] raw values, same rows */
  int win_len;         /* rows of k_win / v_win (>= window) */
  int window;          /* raw window length (128 for ERNIE 5.5 Flash), >= 1 */
  const void* kc;      /* [B, n_cap, d] compressed keys (may be NULL when n_cap == 0) */
  const void* vc;      /* [B, n_cap, d] compressed values */
  int n_cap;           /* entries held in kc / vc (>= 0); entries e >= n_cap are absent */
  int block;           /* tokens per compressed entry (128 for ERNIE 5.5 Flash), >= 1 */
  float scale;         /* logit scale, normally 1/sqrt(d) */
  const void* q_lat;   /* [B, Tq, d_lat] or NULL (ungated) */
  const void* w_gate;  /* [d_lat, H*d] or NULL; NULL exactly when q_lat is NULL */
  int d_lat;           /* query-latent width (1024 for ERNIE 5.5 Flash) */
  void* out;           /* [B, Tq, H, d] */
  void* workspace;     /* scratch, hca_attn_fwd_workspace() bytes */
  size_t workspace_bytes;
  float* lse;          /* NULL, or [B, Tq, H] fp32: ln sum_j exp(scale <q, key_j>) of every row
                          (-inf for a row with no visible key), for hca_attn_bwd; bf16 with
                          Tq > 1 only */
  const void* vha_u;   /* Virtual Head Attention (release blog, section 2.1: a light low-rank */
  const void* vha_v;   /* mix across heads with an identity skip) of the gated output:        */
  int vha_rank;        /* out[h] <- out[h] + sum_h' (U V^T)[h, h'] out[h'], U = vha_u and
                          V = vha_v [H, vha_rank] (dt); vha_rank 0 (and NULL factors) turns it
                          off, at most 16; bf16 needs H == 64.  It runs as a pass of its own
                          after the attention kernels, in place (as vha_mix does). */
} lgsa_hca_args;
/* Validation: every size >= 1 (n_cap >= 0); unless max_pos < win_len (no window row wraps
 * around the ring), win_len >= window + Tq - 1: a call of Tq rows reads positions
 * pos0 - window + 1 .. pos0 + Tq - 1 of a sequence, which must sit in distinct ring rows (a
 * decode call, Tq == 1, needs win_len >= window); max_pos >= Tq - 1; kc / vc non-NULL when
 * n_cap > 0.
 * Entries e >= n_cap are absent: a query sees min(n_cap, (t + 1) / block) entries.
 * Supported: LGSA_BF16 with d == 512 and d_lat % 64 == 0; LGSA_F32 with d <= 512, d % 4 == 0;
 * every tensor 16-byte aligned.
 * Positions beyond max_pos or below 0 never cause an out-of-bounds access: a row whose
 * position is negative has no visible key and produces zeros. */
lgsa_status hca_attn_fwd(const lgsa_hca_args* a, void* stream);
lgsa_status hca_attn_fwd_workspace(const lgsa_hca_args* a, size_t* bytes);

/* ---------------------------------------------------------------------------------------
 * hca_attn_fwd_static -- hca_attn_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments, validation, kernels and result as hca_attn_fwd, except that a->workspace and
 * a->workspace_bytes are ignored: the scratch (the decode path's split partials) comes from a
 * device array of LGSA_STATIC_SCRATCH_BYTES that the library holds on every GPU it runs on,
 * until the process ends.  The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).  A call whose hca_attn_fwd_workspace() exceeds LGSA_STATIC_SCRATCH_BYTES
 * returns LGSA_EWORKSPACE and enqueues nothing (prefill needs no scratch; decode of up to 128
 * sequences of 64 heads, at any context, fits).  Every call on one GPU shares that GPU's
 * array: calls ordered on one stream are safe, but calls that overlap in time on one GPU
 * (other streams, other threads) race on it.  Each call writes every scratch entry it later
 * reads, so the array needs no clearing.  LGSA_EHIP if the array's address cannot be obtained.
 * --------------------------------------------------------------------------------------- */
#define LGSA_STATIC_SCRATCH_BYTES (40u << 20)
lgsa_status hca_attn_fwd_static(const lgsa_hca_args* a, void* stream);

/* ---------------------------------------------------------------------------------------
 * hca_attn_bwd -- backward of hca_attn_fwd in prefill (the chain rule of its definition;
 * training runs whole sequences): every sequence b holds T positions from position 0, query
 * row i sits at position i, the window rows are the sequence's own k, v (win_len = T) and the
 * entries kc, vc are their block means (hca_compress).  With P the softmax of each row's
 * scaled logits over its keys (rebuilt from the forward's lse), dP = dO V^T and
 * D = rowsum(dO * O):
 *     dS = P (dP - D),   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO,
 * and an entry's gradient reaches each position of its block divided by block, so dk, dv
 * hold the gradients of the raw k, v (through the window and through the pooling).  A gated
 * layer runs latent_gate_bwd first and passes its d_o here as dout (out is then the ungated O).
 * --------------------------------------------------------------------------------------- */
typedef struct {
  int dt;              /* LGSA_BF16 */
  int B, T, H, d;      /* sequences, positions (= query rows) per sequence, heads, head dim */
  const void* q;       /* [B, T, H, d] */
  const void* k;       /* [B, T, d] raw keys */
  const void* v;       /* [B, T, d] raw values */
  const void* kc;      /* [B, T / block, d] entries (block means of k); NULL when T < block */
  const void* vc;      /* [B, T / block, d] */
  const void* out;     /* [B, T, H, d] the forward's output O (ungated) */
  const float* lse;    /* [B, T, H] the forward's log-sum-exp (hca_attn_fwd with lse) */
  const void* dout;    /* [B, T, H, d] gradient of the loss with respect to O */
  int window, block;   /* as in the forward */
  float scale;         /* as in the forward */
  void* dq;            /* [B, T, H, d] */
  void* dk;            /* [B, T, d] */
  void* dv;            /* [B, T, d] */
  void* workspace;     /* scratch, hca_attn_bwd_workspace() bytes (P and dS of every row and
                          key are kept there in bf16) */
  size_t workspace_bytes;
} lgsa_hca_bwd_args;
/* Supported: LGSA_BF16, d == 512, H % 4 == 0, 1 <= window <= 512, block >= 1, every tensor
 * 16-byte aligned.  Errors: LGSA_EINVAL (NULL, misaligned, bad sizes), LGSA_EUNSUPPORTED,
 * LGSA_EWORKSPACE; nothing is enqueued on error.  Deterministic (no atomics). */
lgsa_status hca_attn_bwd(const lgsa_hca_bwd_args* a, void* stream);
lgsa_status hca_attn_bwd_workspace(const lgsa_hca_bwd_args* a, size_t* bytes);

/* ---------------------------------------------------------------------------------------
 * dsa_index_topk -- the DSA lightweight indexer and per-query top-k (release blog, section
 * 2.1: the indexer scores the past positions of each query and core attention runs only on
 * the k highest-scoring ones).  The indexer form taken here is
 *     score(t, s) = sum_{h<Hi} w_idx[b,i,h] * max(0, <q_idx[b,i,h,:], k_idx[b,s,:]>)
 * computed in fp32 for every visible key s of the query at position t = pos0[b] + i.  With
 * block == 1 key s is token position s and is visible when s <= t.  With block > 1 (the
 * compressed sparse attention variant, release blog section 2.1: history compressed 4x, then
 * a sparse part of it attended) key s is the entry summarising positions block*s ..
 * block*s + block - 1 and is visible once that block is complete: block*s + block - 1 <= t,
 * i.e. s < (t + 1) / block.  The k highest scores are kept (every visible key when there are
 * at most k); a tie is won by the lower key index; -0.0 counts as +0.0.  idx_out[b,i,:]
 * lists the kept keys in ascending order and holds -1 in the remaining slots.
 * --------------------------------------------------------------------------------------- */
typedef struct {
  int B, Tq, S;          /* sequences, query rows per sequence, key positions held */
  int Hi, di, k;         /* indexer heads, indexer head dim, positions kept per query */
  const float* q_idx;    /* [B, Tq, Hi, di] fp32 */
  const float* w_idx;    /* [B, Tq, Hi] fp32 */
  const float* k_idx;    /* [B, S, di] fp32 */
  const int32_t* pos0;   /* device [B] */
  int max_pos;           /* host: upper bound of pos0[b] + Tq - 1; must be < S */
  int32_t* idx_out;      /* [B, Tq, k] int32 */
  void* workspace;       /* scratch, dsa_index_topk_workspace() bytes */
  size_t workspace_bytes;
  int block;             /* positions per key (see above); 0 is read as 1 */
} lgsa_index_args;
/* Supported: di == 64, 1 <= Hi <= 4, 1 <= k <= 4096, S >= 1, block >= 0; (max_pos + 1) / block
 * <= S (the visible keys of every row exist); q_idx and k_idx 16-byte aligned.  A position
 * beyond max_pos (caller broke the promise) is clamped for reading; it never reads out of
 * bounds. */
lgsa_status dsa_index_topk(const lgsa_index_args* a, void* stream);
lgsa_status dsa_index_topk_workspace(const lgsa_index_args* a, size_t* bytes);

/* ---------------------------------------------------------------------------------------
 * sparse_attn_fwd -- DSA sparse core attention in the MLA layers (release blog, section 2.1:
 * core attention only on the selected positions; 256-wide heads for query/key and value).
 * For query row (b, i) and head h, with the positions listed in idx[b,i,:] (entries < 0 or
 * >= S are skipped, every other entry is one key, order is irrelevant):
 *   O[b,i,h,:] = sum_j softmax_j(scale * <q[b,i,h,:], K_j>) * V_j
 *   K_j = k_lat[b*S*k_row_stride + s_j*k_row_stride + 0 .. d_qk)
 *   V_j = v_lat[b*S*v_row_stride + s_j*v_row_stride + 0 .. d_v)     (v_lat may equal k_lat)
 * and, when q_lat is non-NULL, out = O * sigmoid(q_lat[b,i,:] . w_gate[:, h*d_v + c]).
 * A row with no valid entry produces zeros.
 * --------------------------------------------------------------------------------------- */
typedef struct {
  int dt;                /* LGSA_BF16 */
  int B, Tq, H, d_qk, d_v, S, k;
  const void* q;         /* [B, Tq, H, d_qk] */
  const void* k_lat;     /* [B, S, k_row_stride] latent key rows */
  long long k_row_stride;/* elements between consecutive positions (>= d_qk) */
  const void* v_lat;     /* [B, S, v_row_stride] latent value rows (may equal k_lat) */
  long long v_row_stride;
  const int32_t* idx;    /* [B, Tq, k] int32 */
  float scale;           /* normally 1/sqrt(d_qk) */
  const void* q_lat;     /* [B, Tq, d_lat] or NULL */
  const void* w_gate;    /* [d_lat, H*d_v] or NULL */
  int d_lat;
  void* out;             /* [B, Tq, H, d_v] */
  void* workspace;       /* scratch, sparse_attn_fwd_workspace() bytes */
  size_t workspace_bytes;
  float* lse;            /* [B, Tq, H] or NULL: natural log of each row's softmax denominator
                            over its scaled logits (-inf for a row with no valid entry), for
                            sparse_attn_bwd */
  const void* vha_u;     /* Virtual Head Attention (release blog, section 2.1: a light low-rank */
  const void* vha_v;     /* mix across heads with an identity skip) of the gated output:       */
  int vha_rank;          /* out[h] <- out[h] + sum_h' (U V^T)[h, h'] out[h'], U = vha_u,
                            V = vha_v [H, vha_rank] bf16; 0 turns it off, at most 16; H == 64 */
} lgsa_sparse_args;
/* Supported: LGSA_BF16, d_qk == d_v == 256, H % 64 == 0, row strides % 8 == 0,
 * d_lat % 64 == 0; every tensor 16-byte aligned.  Gated without the head mix, the gate GEMM
 * runs after the attention kernel and rescales out in place.  With the head mix, a GEMM first
 * writes the gate factors sigmoid(q_lat w_gate) into out; the attention kernel's epilogue
 * multiplies them into O, mixes the heads (a workgroup holds all 64 heads of its query row)
 * and writes out over them.  A query row whose list is split over several workgroups (few
 * rows, long lists) is merged, gated, by a combine kernel, and its head mix then runs as a
 * pass of its own. */
lgsa_status sparse_attn_fwd(const lgsa_sparse_args* a, void* stream);
lgsa_status sparse_attn_fwd_workspace(const lgsa_sparse_args* a, size_t* bytes);

/* Compressed sparse attention (release blog, section 2.1: history compressed 4x, then a sparse
 * part of it attended) has no entry point of its own: a caller composes it from the calls
 * above, on one stream.
 *   1. hca_compress(k, v, kc, vc, B, T, 256, block = 4, LGSA_BF16): pooled keys and values,
 *      [B, T / 4, 256], used as separate key and value rows;
 *   2. hca_compress(k_idx, k_idx, kic, kic2, B, T, 64, 4, LGSA_F32): pooled indexer keys
 *      (kic2 receives the same values and may be discarded);
 *   3. dsa_index_topk with k_idx = kic, S = T / 4 and block = 4: query t sees the entries whose
 *      block is complete, s < (t + 1) / 4, and keeps the top k;
 *   4. sparse_attn_fwd with k_lat = kc, v_lat = vc (row strides 256), S = T / 4, the lists of
 *      step 3 and, when gated, q_lat and w_gate.
 * The binding's csa_attn_fwd does exactly this. */

/* ---------------------------------------------------------------------------------------
 * sparse_attn_bwd -- backward of sparse_attn_fwd (the chain rule of its definition; the
 * pages' training is the reason to have it).  For query row (b, i), head h, the listed keys
 * K_j, values V_j, P the softmax of the row's scaled logits (rebuilt from the forward's lse),
 * dP_j = <dO, V_j> and D = <dO, O>:
 *     dS_j = P_j (dP_j - D),   dq = scale sum_j dS_j K_j,
 *     row s_j of dk gains scale sum_h dS_j q_h,   row s_j of dv gains sum_h P_j dO_h,
 * summed over every (row, entry) that lists s_j (an entry listed twice counts twice; skipped
 * entries contribute nothing; rows no entry lists get zeros).  When v_lat is k_lat the two
 * gradients land on the same latent row: dk then holds their sum on its first d_qk columns and
 * dv must be NULL.  A gated layer runs latent_gate_bwd first and passes its d_o as dout.
 * Deterministic: the contributions of every (row, entry) are written to slots ordered by key
 * and then by row, and each key's slots are summed in that order (fp32).
 * --------------------------------------------------------------------------------------- */
typedef struct {
  int dt;                /* LGSA_BF16 */
  int B, Tq, H, d_qk, d_v, S, k;
  const void* q;         /* [B, Tq, H, d_qk] */
  const void* k_lat;     /* [B, S, k_row_stride] */
  long long k_row_stride;
  const void* v_lat;     /* [B, S, v_row_stride] (may equal k_lat) */
  long long v_row_stride;
  const int32_t* idx;    /* [B, Tq, k] as in the forward */
  float scale;           /* as in the forward */
  const void* out;       /* [B, Tq, H, d_v] the forward's output O (ungated) */
  const float* lse;      /* [B, Tq, H] the forward's log-sum-exp */
  const void* dout;      /* [B, Tq, H, d_v] gradient of the loss with respect to O */
  void* dq;              /* [B, Tq, H, d_qk] */
  void* dk;              /* [B, S, d_qk] gradient of the key columns of every latent row */
  void* dv;              /* [B, S, d_v] gradient of the value columns; NULL when v_lat == k_lat */
  void* workspace;       /* scratch: sparse_attn_bwd_workspace() bytes hold the slot order
                            and the contributions of up to a sequence's rows at a time (within
                            about 8 GiB); less, down to the size for one row, makes the call
                            take fewer rows at a time (same result up to summation order) */
  size_t workspace_bytes;
} lgsa_sparse_bwd_args;
/* Supported: LGSA_BF16, d_qk == d_v == 256, H % 64 == 0, row strides % 8 == 0, S <= 2^26,
 * k * H / 64 <= 2^24; q, the latent rows, out, dout, dq, dk, dv 16-byte aligned; lse, idx 4-byte
 * aligned.  dq, dk, dv are overwritten (dk and dv entirely).  Errors as for sparse_attn_fwd
 * (LGSA_EINVAL, LGSA_EUNSUPPORTED); LGSA_EWORKSPACE when the workspace is below the size for one
 * row.  Runs on the given stream; the workspace must stay untouched until the call completes. */
lgsa_status sparse_attn_bwd(const lgsa_sparse_bwd_args* a, void* stream);
lgsa_status sparse_attn_bwd_workspace(const lgsa_sparse_bwd_args* a, size_t* bytes);

/* ---------------------------------------------------------------------------------------
 * vha_mix -- Virtual Head Attention (release blog, section 2.1: after attention, a light
 * low-rank mixing step across heads with an identity skip connection, so that heads share
 * information).  Read as, per token m and channel c of the head dimension,
 *     out[m, h, c] = o[m, h, c] + sum_{h'} (U V^T)[h, h'] * o[m, h', c]
 * with U = u, V = v of shape [H, r] (the pages give neither the rank nor the weights), applied
 * to the gated attention output.  Computed as z = V^T o[m] (rank r) and out = o[m] + U z,
 * accumulating in fp32; on the bfloat16 path z is rounded to bfloat16 before the second
 * product.
 *   o, out [M, H, d] (dt); out may equal o.   u, v [H, r] (dt)
 * Supported: LGSA_BF16 with H == 64, d % 256 == 0, 1 <= r <= 16 (o, out 16-byte aligned);
 * LGSA_F32 with H >= 1, d >= 1, 1 <= r <= 16.  M == 0 enqueues nothing.
 * ------------------------------------------------------------------------------------- */
lgsa_status vha_mix(const void* o, const void* u, const void* v, void* out, int M, int H, int d,
                    int r, int dt, void* stream);

/* ---------------------------------------------------------------------------------------
 * hca_cache_append -- decode-time maintenance of an HCA layer's cache (release blog,
 * section 2.1: one compressed entry per completed block of 128 tokens plus a window of recent
 * raw tokens; window size from the xenospectrum.com article, long-context section).  For
 * every sequence b whose new token sits at position t = pos[b] >= 0:
 *   - k_new[b] and v_new[b] are written to row t % win_len of the rings k_win and v_win;
 *   - when t completes its block (t % block == block - 1) and e = t / block < n_cap, the
 *     entry kc[b, e] = (1/block) * (sum of the block's keys) is written, and vc[b, e] from the
 *     values.  The block's first block - 1 rows are read from the ring (row p % win_len for
 *     position p) and its last row from k_new / v_new.  The sum runs in fp32 in the order
 *     hca_compress uses, so an entry completed here is bit-identical to the one hca_compress
 *     makes from the same rows.
 * Sequences with pos[b] < 0 are left untouched.  This runs before the decode attention of the
 * same token, which sees the token itself and, at a block's last token, the new entry.
 * --------------------------------------------------------------------------------------- */
typedef struct {
  int dt;              /* LGSA_F32 or LGSA_BF16: every tensor of the call */
  int B, d;            /* sequences, row width */
  const int32_t* pos;  /* device [B]: position of each sequence's new token */
  const void* k_new;   /* [B, d] key of the new token */
  const void* v_new;   /* [B, d] value of the new token */
  void* k_win;         /* [B, win_len, d] ring of raw keys: position p in row p % win_len */
  void* v_win;         /* [B, win_len, d] ring of raw values, same rows */
  int win_len;         /* rows of each ring (>= 1) */
  void* kc;            /* [B, n_cap, d] compressed keys (may be NULL when n_cap == 0) */
  void* vc;            /* [B, n_cap, d] compressed values */
  int n_cap;           /* entries held in kc / vc (>= 0); entries e >= n_cap are not written */
  int block;           /* tokens per compressed entry (128 for ERNIE 5.5 Flash), >= 1 */
} lgsa_hca_append_args;
/* Validation: B >= 0, d >= 1, win_len >= 1, block >= 1, n_cap >= 0; when n_cap > 0, kc and vc
 * non-NULL and win_len >= block (the ring must hold a whole block).  Supported: LGSA_F32 with
 * d % 4 == 0 or LGSA_BF16 with d % 8 == 0; every tensor 16-byte aligned.  Ring rows are always
 * in range; the caller keeps the block's earlier rows in the ring (they were appended by the
 * previous block - 1 calls or by a prefill). */
lgsa_status hca_cache_append(const lgsa_hca_append_args* a, void* stream);

/* ---------------------------------------------------------------------------------------
 * dsa_cache_append -- decode-time append to a DSA layer's caches (release blog, section 2.1:
 * the indexer scores every past position and sparse attention gathers the latent rows of the
 * selected ones).  For every sequence b with 0 <= t = pos[b] < S:
 *   k_idx[b, t, :] = k_idx_new[b, :]   and   kv_lat[b*S*stride + t*stride + 0 .. row) = kv_new[b, :]
 * Other sequences are left untouched.
 * --------------------------------------------------------------------------------------- */
typedef struct {
  int dt;                  /* LGSA_F32 or LGSA_BF16: element type of kv_new and kv_lat */
  int B, S;                /* sequences, positions held per sequence */
  const int32_t* pos;      /* device [B]: position of each sequence's new token */
  const float* k_idx_new;  /* [B, di] fp32 indexer key of the new token */
  float* k_idx;            /* [B, S, di] fp32 indexer keys */
  int di;                  /* indexer head dim */
  const void* kv_new;      /* [B, row] latent row of the new token */
  void* kv_lat;            /* [B, S, kv_row_stride] latent rows */
  int row;                 /* elements of a latent row */
  long long kv_row_stride; /* elements between consecutive positions (>= row) */
} lgsa_dsa_append_args;
/* Validation: B >= 0, S >= 1, di >= 1, row >= 1, kv_row_stride >= row.  Supported: di % 4 == 0;
 * row and kv_row_stride multiples of 8 (bf16) or 4 (f32); every tensor 16-byte aligned. */
lgsa_status dsa_cache_append(const lgsa_dsa_append_args* a, void* stream);

/* ---------------------------------------------------------------------------------------
 * sparse_gather_probe -- measurement helper, not a step of the method: the gathers of
 * sparse_attn_fwd alone (its DMA pattern, tiles of 32 listed rows double buffered in LDS, one
 * workgroup per list), with no arithmetic, so that the rate at which listed 512-byte latent
 * rows can be gathered (the bound of sparse attention's data movement) can be timed.
 *   rows [S, row_stride] bf16 (the first 256 elements of a row are gathered); idx [n_lists, k]
 *   int32 (entries < 0 or >= S, and slots past k in the last tile, read row 0); sums
 *   [n_lists, 2] uint32, written so that the transfers are used: sums[l][w] adds up, with
 *   wrap-around, the first 64 32-bit words of the row listed in slot 32 t + 16 w of every
 *   tile t of list l.
 * Errors: LGSA_EINVAL for NULL or misaligned pointers and bad sizes, LGSA_EUNSUPPORTED for a
 * row stride below 256 or not a multiple of 8.
 * --------------------------------------------------------------------------------------- */
lgsa_status sparse_gather_probe(const void* rows, long long row_stride, int S,
                                const int32_t* idx, int n_lists, int k, uint32_t* sums,
                                void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LGSA_H */
