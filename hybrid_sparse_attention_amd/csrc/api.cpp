// C ABI of the Latent-Gated Sparse Attention library (declared in include/lgsa.h).
// Every entry point validates its arguments on the host before it touches the HIP runtime,
// so every error path is exercised without a GPU; then it hands over to the launchers.
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/lgsa.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

lgsa_status fail(lgsa_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

lgsa_status ok() {
  g_err.clear();
  return LGSA_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

lgsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(LGSA_EHIP, "%s: HIP launch failed: %s", what, hipGetErrorString(e));
}

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

lgsa::HcaParams to_params(const lgsa_hca_args* a) {
  lgsa::HcaParams p;
  p.B = a->B;
  p.Tq = a->Tq;
  p.H = a->H;
  p.d = a->d;
  p.q = a->q;
  p.pos0 = a->pos0;
  p.max_pos = a->max_pos;
  p.k_win = a->k_win;
  p.v_win = a->v_win;
  p.win_len = a->win_len;
  p.window = a->window;
  p.kc = a->kc;
  p.vc = a->vc;
  p.n_cap = a->n_cap;
  p.block = a->block;
  p.scale = a->scale;
  p.q_lat = a->q_lat;
  p.w_gate = a->w_gate;
  p.d_lat = a->d_lat;
  p.out = a->out;
  p.lse = a->lse;
  p.ws = a->workspace;
  p.ws_bytes = a->workspace_bytes;
  p.vha_u = a->vha_u;
  p.vha_v = a->vha_v;
  p.vha_r = a->vha_rank;
  return p;
}

// The optional head mix (VHA) of an attention call: rank 0 turns it off; otherwise both
// factors [H, rank] in the call's dtype, rank <= 16, and 64 heads on the bfloat16 path.
lgsa_status check_vha(const char* who, int dt, int H, const void* u, const void* v, int rank) {
  REQUIRE(rank >= 0 && rank <= 16, LGSA_EUNSUPPORTED, "%s: vha_rank must be in 0..16 (got %d)",
          who, rank);
  if (rank == 0) return LGSA_OK;
  REQUIRE(u != nullptr && v != nullptr, LGSA_EINVAL,
          "%s: vha_u and vha_v must be non-NULL when vha_rank > 0", who);
  REQUIRE(dt != LGSA_BF16 || H == 64, LGSA_EUNSUPPORTED,
          "%s: the bf16 head mix needs H == 64 (got %d)", who, H);
  const uintptr_t al = dt == LGSA_BF16 ? 2 : 4;
  REQUIRE(aligned(u, al) && aligned(v, al), LGSA_EINVAL,
          "%s: vha_u and vha_v must be aligned to their element size", who);
  return LGSA_OK;
}

lgsa_status check_hca(const lgsa_hca_args* a) {
  REQUIRE(a != nullptr, LGSA_EINVAL, "hca_attn_fwd: args is NULL");
  REQUIRE(a->dt == LGSA_F32 || a->dt == LGSA_BF16, LGSA_EINVAL, "hca_attn_fwd: unknown dt %d",
          a->dt);
  REQUIRE(a->B >= 1 && a->Tq >= 1 && a->H >= 1 && a->d >= 1, LGSA_EINVAL,
          "hca_attn_fwd: B, Tq, H, d must be >= 1 (got %d, %d, %d, %d)", a->B, a->Tq, a->H,
          a->d);
  REQUIRE(a->q && a->pos0 && a->k_win && a->v_win && a->out, LGSA_EINVAL,
          "hca_attn_fwd: q, pos0, k_win, v_win and out must be non-NULL");
  REQUIRE(a->win_len >= 1 && a->window >= 1, LGSA_EINVAL,
          "hca_attn_fwd: win_len and window must be >= 1");
  // the window rows a call reads must not alias in the ring: either no position reaches past
  // its end, or it holds the window of the first row plus the call's other Tq - 1 rows
  // (positions pos0 - window + 1 .. pos0 + Tq - 1 of one sequence)
  REQUIRE(a->max_pos < a->win_len || (long long)a->win_len >= (long long)a->window + a->Tq - 1,
          LGSA_EINVAL,
          "hca_attn_fwd: k_win/v_win hold %d rows, fewer than window + Tq - 1 = %lld, and "
          "positions reach past them", a->win_len, (long long)a->window + a->Tq - 1);
  REQUIRE(a->block >= 1, LGSA_EINVAL, "hca_attn_fwd: block must be >= 1");
  REQUIRE(a->lse == nullptr || (a->dt == LGSA_BF16 && a->Tq > 1), LGSA_EUNSUPPORTED,
          "hca_attn_fwd: lse is written by the bf16 path with Tq > 1 only");
  REQUIRE(a->n_cap >= 0, LGSA_EINVAL, "hca_attn_fwd: n_cap must be >= 0");
  REQUIRE(a->n_cap == 0 || (a->kc && a->vc), LGSA_EINVAL,
          "hca_attn_fwd: kc and vc must be non-NULL when n_cap > 0");
  REQUIRE(a->max_pos >= a->Tq - 1, LGSA_EINVAL,
          "hca_attn_fwd: max_pos (%d) is below Tq - 1 (%d)", a->max_pos, a->Tq - 1);
  REQUIRE(std::isfinite(a->scale), LGSA_EINVAL, "hca_attn_fwd: scale is not finite");
  REQUIRE((a->q_lat == nullptr) == (a->w_gate == nullptr), LGSA_EINVAL,
          "hca_attn_fwd: q_lat and w_gate must be both NULL or both non-NULL");
  REQUIRE(a->q_lat == nullptr || a->d_lat >= 1, LGSA_EINVAL,
          "hca_attn_fwd: d_lat must be >= 1 when gated");
  if (a->dt == LGSA_BF16) {
    REQUIRE(a->d == 512, LGSA_EUNSUPPORTED, "hca_attn_fwd: bf16 supports d == 512 (got %d)",
            a->d);
    REQUIRE(a->q_lat == nullptr || a->d_lat % 64 == 0, LGSA_EUNSUPPORTED,
            "hca_attn_fwd: bf16 gate needs d_lat %% 64 == 0 (got %d)", a->d_lat);
    const void* ptrs[] = {a->q, a->k_win, a->v_win, a->kc, a->vc, a->q_lat, a->w_gate, a->out};
    for (const void* p : ptrs)
      REQUIRE(aligned(p, 16), LGSA_EINVAL, "hca_attn_fwd: tensors must be 16-byte aligned");
  } else {
    REQUIRE(a->d <= 512 && a->d % 4 == 0, LGSA_EUNSUPPORTED,
            "hca_attn_fwd: f32 supports d <= 512 with d %% 4 == 0 (got %d)", a->d);
    const void* ptrs[] = {a->q, a->k_win, a->v_win, a->kc, a->vc, a->out};
    for (const void* p : ptrs)
      REQUIRE(aligned(p, 16), LGSA_EINVAL, "hca_attn_fwd: tensors must be 16-byte aligned");
  }
  return check_vha("hca_attn_fwd", a->dt, a->H, a->vha_u, a->vha_v, a->vha_rank);
}

size_t hca_ws(const lgsa_hca_args* a) {
  const lgsa::HcaParams p = to_params(a);
  return a->dt == LGSA_BF16 ? lgsa::hca_bf16_workspace(p) : lgsa::hca_f32_workspace(p);
}

lgsa::IndexParams to_params(const lgsa_index_args* a) {
  lgsa::IndexParams p;
  p.B = a->B;
  p.Tq = a->Tq;
  p.S = a->S;
  p.Hi = a->Hi;
  p.di = a->di;
  p.k = a->k;
  p.q_idx = a->q_idx;
  p.w_idx = a->w_idx;
  p.k_idx = a->k_idx;
  p.pos0 = a->pos0;
  p.max_pos = a->max_pos;
  p.idx_out = a->idx_out;
  p.ws = a->workspace;
  p.ws_bytes = a->workspace_bytes;
  p.block = a->block == 0 ? 1 : a->block;
  return p;
}

lgsa_status check_index(const lgsa_index_args* a) {
  REQUIRE(a != nullptr, LGSA_EINVAL, "dsa_index_topk: args is NULL");
  REQUIRE(a->B >= 1 && a->Tq >= 1 && a->S >= 1, LGSA_EINVAL,
          "dsa_index_topk: B, Tq, S must be >= 1");
  REQUIRE(a->Hi >= 1 && a->di >= 1 && a->k >= 1, LGSA_EINVAL,
          "dsa_index_topk: Hi, di, k must be >= 1");
  REQUIRE(a->q_idx && a->w_idx && a->k_idx && a->pos0 && a->idx_out, LGSA_EINVAL,
          "dsa_index_topk: q_idx, w_idx, k_idx, pos0 and idx_out must be non-NULL");
  REQUIRE(a->max_pos >= a->Tq - 1, LGSA_EINVAL,
          "dsa_index_topk: max_pos (%d) is below Tq - 1 (%d)", a->max_pos, a->Tq - 1);
  REQUIRE(a->block >= 0, LGSA_EINVAL, "dsa_index_topk: block must be >= 0 (got %d)", a->block);
  REQUIRE(((long long)a->max_pos + 1) / (a->block == 0 ? 1 : a->block) <= a->S, LGSA_EINVAL,
          "dsa_index_topk: max_pos (%d) needs (max_pos + 1) / block keys but S is %d: every "
          "visible key must exist", a->max_pos, a->S);
  REQUIRE(a->di == 64, LGSA_EUNSUPPORTED, "dsa_index_topk: di must be 64 (got %d)", a->di);
  REQUIRE(a->Hi <= 4, LGSA_EUNSUPPORTED, "dsa_index_topk: Hi must be <= 4 (got %d)", a->Hi);
  REQUIRE(a->k <= 4096, LGSA_EUNSUPPORTED, "dsa_index_topk: k must be <= 4096 (got %d)", a->k);
  REQUIRE(aligned(a->q_idx, 16) && aligned(a->k_idx, 16), LGSA_EINVAL,
          "dsa_index_topk: q_idx and k_idx must be 16-byte aligned");
  return LGSA_OK;
}

lgsa::SparseParams to_params(const lgsa_sparse_args* a) {
  lgsa::SparseParams p;
  p.B = a->B;
  p.Tq = a->Tq;
  p.H = a->H;
  p.d_qk = a->d_qk;
  p.d_v = a->d_v;
  p.S = a->S;
  p.k = a->k;
  p.q = a->q;
  p.k_lat = a->k_lat;
  p.k_stride = a->k_row_stride;
  p.v_lat = a->v_lat;
  p.v_stride = a->v_row_stride;
  p.idx = a->idx;
  p.scale = a->scale;
  p.q_lat = a->q_lat;
  p.w_gate = a->w_gate;
  p.d_lat = a->d_lat;
  p.out = a->out;
  p.ws = a->workspace;
  p.ws_bytes = a->workspace_bytes;
  p.lse = a->lse;
  p.vha_u = a->vha_u;
  p.vha_v = a->vha_v;
  p.vha_r = a->vha_rank;
  return p;
}

lgsa_status check_sparse(const lgsa_sparse_args* a) {
  REQUIRE(a != nullptr, LGSA_EINVAL, "sparse_attn_fwd: args is NULL");
  REQUIRE(a->dt == LGSA_F32 || a->dt == LGSA_BF16, LGSA_EINVAL,
          "sparse_attn_fwd: unknown dt %d", a->dt);
  REQUIRE(a->B >= 1 && a->Tq >= 1 && a->H >= 1 && a->d_qk >= 1 && a->d_v >= 1 && a->S >= 1 &&
              a->k >= 1,
          LGSA_EINVAL, "sparse_attn_fwd: B, Tq, H, d_qk, d_v, S, k must be >= 1");
  REQUIRE(a->q && a->k_lat && a->v_lat && a->idx && a->out, LGSA_EINVAL,
          "sparse_attn_fwd: q, k_lat, v_lat, idx and out must be non-NULL");
  REQUIRE(a->k_row_stride >= a->d_qk && a->v_row_stride >= a->d_v, LGSA_EINVAL,
          "sparse_attn_fwd: row strides must be >= the head dims");
  REQUIRE(std::isfinite(a->scale), LGSA_EINVAL, "sparse_attn_fwd: scale is not finite");
  REQUIRE((a->q_lat == nullptr) == (a->w_gate == nullptr), LGSA_EINVAL,
          "sparse_attn_fwd: q_lat and w_gate must be both NULL or both non-NULL");
  REQUIRE(a->q_lat == nullptr || a->d_lat >= 1, LGSA_EINVAL,
          "sparse_attn_fwd: d_lat must be >= 1 when gated");
  REQUIRE(a->dt == LGSA_BF16, LGSA_EUNSUPPORTED, "sparse_attn_fwd: only bf16 is built");
  REQUIRE(a->d_qk == 256 && a->d_v == 256, LGSA_EUNSUPPORTED,
          "sparse_attn_fwd: d_qk and d_v must be 256 (got %d, %d)", a->d_qk, a->d_v);
  REQUIRE(a->H % 64 == 0, LGSA_EUNSUPPORTED, "sparse_attn_fwd: H must be a multiple of 64");
  REQUIRE(a->k_row_stride % 8 == 0 && a->v_row_stride % 8 == 0, LGSA_EUNSUPPORTED,
          "sparse_attn_fwd: row strides must be multiples of 8 elements");
  REQUIRE(a->q_lat == nullptr || a->d_lat % 64 == 0, LGSA_EUNSUPPORTED,
          "sparse_attn_fwd: gate needs d_lat %% 64 == 0 (got %d)", a->d_lat);
  const void* ptrs[] = {a->q, a->k_lat, a->v_lat, a->q_lat, a->w_gate, a->out};
  for (const void* p : ptrs)
    REQUIRE(aligned(p, 16), LGSA_EINVAL, "sparse_attn_fwd: tensors must be 16-byte aligned");
  return check_vha("sparse_attn_fwd", a->dt, a->H, a->vha_u, a->vha_v, a->vha_rank);
}

lgsa_status check_workspace(const char* name, const void* ws, size_t have, size_t need) {
  REQUIRE(have >= need, LGSA_EWORKSPACE, "%s: workspace of %zu bytes is below the %zu needed",
          name, have, need);
  REQUIRE(need == 0 || ws != nullptr, LGSA_EWORKSPACE, "%s: workspace is NULL", name);
  REQUIRE(need == 0 || aligned(ws, 16), LGSA_EWORKSPACE, "%s: workspace must be 16-byte aligned",
          name);
  return LGSA_OK;
}

lgsa::SparseBwdParams to_params(const lgsa_sparse_bwd_args* a) {
  lgsa::SparseBwdParams p;
  p.B = a->B;
  p.Tq = a->Tq;
  p.H = a->H;
  p.S = a->S;
  p.k = a->k;
  p.q = a->q;
  p.k_lat = a->k_lat;
  p.k_stride = a->k_row_stride;
  p.v_lat = a->v_lat;
  p.v_stride = a->v_row_stride;
  p.idx = a->idx;
  p.scale = a->scale;
  p.out = a->out;
  p.lse = a->lse;
  p.dout = a->dout;
  p.dq = a->dq;
  p.dk = a->dk;
  p.dv = a->dv;
  p.ws = a->workspace;
  p.ws_bytes = a->workspace_bytes;
  return p;
}

lgsa_status check_sparse_bwd(const lgsa_sparse_bwd_args* a) {
  REQUIRE(a != nullptr, LGSA_EINVAL, "sparse_attn_bwd: args is NULL");
  REQUIRE(a->dt == LGSA_BF16, LGSA_EUNSUPPORTED, "sparse_attn_bwd: only LGSA_BF16 is supported");
  REQUIRE(a->B >= 1 && a->Tq >= 1 && a->H >= 1 && a->d_qk >= 1 && a->d_v >= 1 && a->S >= 1 &&
              a->k >= 1,
          LGSA_EINVAL, "sparse_attn_bwd: B, Tq, H, d_qk, d_v, S, k must be >= 1");
  REQUIRE(a->q && a->k_lat && a->v_lat && a->idx && a->out && a->lse && a->dout && a->dq && a->dk,
          LGSA_EINVAL, "sparse_attn_bwd: q, k_lat, v_lat, idx, out, lse, dout, dq and dk must be "
          "non-NULL");
  REQUIRE(a->dv != nullptr || (a->v_lat == a->k_lat && a->v_row_stride == a->k_row_stride),
          LGSA_EINVAL, "sparse_attn_bwd: dv may be NULL only when v_lat is k_lat");
  REQUIRE(a->k_row_stride >= a->d_qk && a->v_row_stride >= a->d_v, LGSA_EINVAL,
          "sparse_attn_bwd: row strides must be >= the head dims");
  REQUIRE(std::isfinite(a->scale), LGSA_EINVAL, "sparse_attn_bwd: scale is not finite");
  REQUIRE(a->d_qk == 256 && a->d_v == 256, LGSA_EUNSUPPORTED,
          "sparse_attn_bwd: d_qk and d_v must be 256 (got %d, %d)", a->d_qk, a->d_v);
  REQUIRE(a->H % 64 == 0, LGSA_EUNSUPPORTED, "sparse_attn_bwd: H must be a multiple of 64");
  REQUIRE(a->k_row_stride % 8 == 0 && a->v_row_stride % 8 == 0, LGSA_EUNSUPPORTED,
          "sparse_attn_bwd: row strides must be multiples of 8 elements");
  REQUIRE(a->S <= (1 << 26), LGSA_EUNSUPPORTED, "sparse_attn_bwd: S must be <= 2^26");
  REQUIRE((long long)a->k * (a->H / 64) <= (1 << 24), LGSA_EUNSUPPORTED,
          "sparse_attn_bwd: k * H / 64 must be <= 2^24");
  const void* ptrs[] = {a->q, a->k_lat, a->v_lat, a->out, a->dout, a->dq, a->dk, a->dv};
  for (const void* p : ptrs)
    REQUIRE(aligned(p, 16), LGSA_EINVAL, "sparse_attn_bwd: tensors must be 16-byte aligned");
  REQUIRE(aligned(a->lse, 4) && aligned(a->idx, 4), LGSA_EINVAL,
          "sparse_attn_bwd: lse and idx must be 4-byte aligned");
  return LGSA_OK;
}

lgsa::HcaBwdParams to_params(const lgsa_hca_bwd_args* a) {
  lgsa::HcaBwdParams p;
  p.B = a->B;
  p.T = a->T;
  p.H = a->H;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.kc = a->kc;
  p.vc = a->vc;
  p.out = a->out;
  p.lse = a->lse;
  p.dout = a->dout;
  p.window = a->window;
  p.block = a->block;
  p.ne = a->block >= 1 ? a->T / a->block : 0;
  p.scale = a->scale;
  p.dq = a->dq;
  p.dk = a->dk;
  p.dv = a->dv;
  p.ws = a->workspace;
  p.ws_bytes = a->workspace_bytes;
  return p;
}

lgsa_status check_hca_bwd(const lgsa_hca_bwd_args* a) {
  REQUIRE(a != nullptr, LGSA_EINVAL, "hca_attn_bwd: args is NULL");
  REQUIRE(a->dt == LGSA_BF16, LGSA_EUNSUPPORTED, "hca_attn_bwd: only LGSA_BF16 is supported");
  REQUIRE(a->B >= 1 && a->T >= 1 && a->H >= 1 && a->d >= 1, LGSA_EINVAL,
          "hca_attn_bwd: B, T, H, d must be >= 1");
  REQUIRE(a->d == 512, LGSA_EUNSUPPORTED, "hca_attn_bwd: d must be 512 (got %d)", a->d);
  REQUIRE(a->H % 4 == 0, LGSA_EUNSUPPORTED, "hca_attn_bwd: H must be a multiple of 4");
  REQUIRE(a->window >= 1 && a->window <= 512 && a->block >= 1, LGSA_EINVAL,
          "hca_attn_bwd: window must be in [1, 512] and block >= 1");
  REQUIRE(std::isfinite(a->scale), LGSA_EINVAL, "hca_attn_bwd: scale is not finite");
  REQUIRE(a->q && a->k && a->v && a->out && a->lse && a->dout && a->dq && a->dk && a->dv,
          LGSA_EINVAL, "hca_attn_bwd: q, k, v, out, lse, dout, dq, dk, dv must be non-NULL");
  REQUIRE(a->T < a->block || (a->kc && a->vc), LGSA_EINVAL,
          "hca_attn_bwd: kc and vc must be non-NULL when a block is complete");
  for (const void* p : {a->q, a->k, a->v, a->kc, a->vc, a->out, (const void*)a->lse, a->dout,
                        (const void*)a->dq, (const void*)a->dk, (const void*)a->dv})
    REQUIRE(aligned(p, 16), LGSA_EINVAL, "hca_attn_bwd: tensors must be 16-byte aligned");
  return LGSA_OK;
}

}  // namespace

extern "C" {

const char* lgsa_last_error(void) { return g_err.c_str(); }

lgsa_status hca_compress(const void* k, const void* v, void* kc, void* vc, int B, int T, int d,
                         int block, int dt, void* stream) {
  REQUIRE(dt == LGSA_F32 || dt == LGSA_BF16, LGSA_EINVAL, "hca_compress: unknown dt %d", dt);
  REQUIRE(B >= 0 && T >= 0, LGSA_EINVAL, "hca_compress: B and T must be >= 0");
  REQUIRE(d >= 1 && block >= 1, LGSA_EINVAL, "hca_compress: d and block must be >= 1");
  REQUIRE(k && v, LGSA_EINVAL, "hca_compress: k and v must be non-NULL");
  REQUIRE((kc && vc) || T / block == 0 || B == 0, LGSA_EINVAL,
          "hca_compress: kc and vc must be non-NULL when a block is complete");
  REQUIRE(d % (dt == LGSA_BF16 ? 8 : 4) == 0, LGSA_EUNSUPPORTED,
          "hca_compress: d must be a multiple of %d for this dtype", dt == LGSA_BF16 ? 8 : 4);
  REQUIRE(aligned(k, 16) && aligned(v, 16) && aligned(kc, 16) && aligned(vc, 16), LGSA_EINVAL,
          "hca_compress: tensors must be 16-byte aligned");
  return hip_status(lgsa::launch_compress(k, v, kc, vc, B, T, d, block, dt, (hipStream_t)stream),
                    "hca_compress");
}

lgsa_status vha_mix(const void* o, const void* u, const void* v, void* out, int M, int H, int d,
                    int r, int dt, void* stream) {
  REQUIRE(dt == LGSA_F32 || dt == LGSA_BF16, LGSA_EINVAL, "vha_mix: unknown dt %d", dt);
  REQUIRE(M >= 0 && H >= 1 && d >= 1 && r >= 1, LGSA_EINVAL,
          "vha_mix: M must be >= 0 and H, d, r >= 1");
  REQUIRE(o && u && v && out, LGSA_EINVAL, "vha_mix: o, u, v and out must be non-NULL");
  REQUIRE(r <= 16, LGSA_EUNSUPPORTED, "vha_mix: rank r must be <= 16 (got %d)", r);
  if (dt == LGSA_BF16) {
    REQUIRE(H == 64 && d % 256 == 0, LGSA_EUNSUPPORTED,
            "vha_mix: bf16 needs H == 64 and d %% 256 == 0 (got %d, %d)", H, d);
    REQUIRE(aligned(o, 16) && aligned(out, 16), LGSA_EINVAL,
            "vha_mix: o and out must be 16-byte aligned");
  }
  return hip_status(lgsa::launch_vha(o, u, v, out, M, H, d, r, dt, (hipStream_t)stream),
                    "vha_mix");
}

lgsa_status hca_cache_append(const lgsa_hca_append_args* a, void* stream) {
  REQUIRE(a != nullptr, LGSA_EINVAL, "hca_cache_append: args is NULL");
  REQUIRE(a->dt == LGSA_F32 || a->dt == LGSA_BF16, LGSA_EINVAL,
          "hca_cache_append: unknown dt %d", a->dt);
  REQUIRE(a->B >= 0 && a->n_cap >= 0, LGSA_EINVAL, "hca_cache_append: B and n_cap must be >= 0");
  REQUIRE(a->d >= 1 && a->win_len >= 1 && a->block >= 1, LGSA_EINVAL,
          "hca_cache_append: d, win_len and block must be >= 1");
  REQUIRE(a->pos && a->k_new && a->v_new && a->k_win && a->v_win, LGSA_EINVAL,
          "hca_cache_append: pos, k_new, v_new, k_win and v_win must be non-NULL");
  REQUIRE(a->n_cap == 0 || (a->kc && a->vc), LGSA_EINVAL,
          "hca_cache_append: kc and vc must be non-NULL when n_cap > 0");
  REQUIRE(a->n_cap == 0 || a->win_len >= a->block, LGSA_EINVAL,
          "hca_cache_append: the ring (win_len %d) must hold a whole block (%d) when n_cap > 0",
          a->win_len, a->block);
  REQUIRE(a->d % (a->dt == LGSA_BF16 ? 8 : 4) == 0, LGSA_EUNSUPPORTED,
          "hca_cache_append: d must be a multiple of %d for this dtype",
          a->dt == LGSA_BF16 ? 8 : 4);
  REQUIRE(aligned(a->k_new, 16) && aligned(a->v_new, 16) && aligned(a->k_win, 16) &&
              aligned(a->v_win, 16) && aligned(a->kc, 16) && aligned(a->vc, 16),
          LGSA_EINVAL, "hca_cache_append: tensors must be 16-byte aligned");
  return hip_status(lgsa::launch_hca_append(a->pos, a->k_new, a->v_new, a->k_win, a->v_win,
                                            a->kc, a->vc, a->B, a->d, a->win_len, a->n_cap,
                                            a->block, a->dt, (hipStream_t)stream),
                    "hca_cache_append");
}

lgsa_status dsa_cache_append(const lgsa_dsa_append_args* a, void* stream) {
  REQUIRE(a != nullptr, LGSA_EINVAL, "dsa_cache_append: args is NULL");
  REQUIRE(a->dt == LGSA_F32 || a->dt == LGSA_BF16, LGSA_EINVAL,
          "dsa_cache_append: unknown dt %d", a->dt);
  REQUIRE(a->B >= 0 && a->S >= 1 && a->di >= 1 && a->row >= 1, LGSA_EINVAL,
          "dsa_cache_append: B must be >= 0 and S, di, row >= 1");
  REQUIRE(a->kv_row_stride >= a->row, LGSA_EINVAL,
          "dsa_cache_append: kv_row_stride (%lld) must be >= row (%d)", a->kv_row_stride, a->row);
  REQUIRE(a->pos && a->k_idx_new && a->k_idx && a->kv_new && a->kv_lat, LGSA_EINVAL,
          "dsa_cache_append: pos, k_idx_new, k_idx, kv_new and kv_lat must be non-NULL");
  const int vec = a->dt == LGSA_BF16 ? 8 : 4;
  REQUIRE(a->di % 4 == 0 && a->row % vec == 0 && a->kv_row_stride % vec == 0, LGSA_EUNSUPPORTED,
          "dsa_cache_append: di must be a multiple of 4 and row, kv_row_stride of %d", vec);
  REQUIRE(aligned(a->k_idx_new, 16) && aligned(a->k_idx, 16) && aligned(a->kv_new, 16) &&
              aligned(a->kv_lat, 16),
          LGSA_EINVAL, "dsa_cache_append: tensors must be 16-byte aligned");
  return hip_status(lgsa::launch_dsa_append(a->pos, a->B, a->S, a->k_idx_new, a->k_idx, a->di,
                                            a->kv_new, a->kv_lat, a->row, a->kv_row_stride,
                                            a->dt, (hipStream_t)stream),
                    "dsa_cache_append");
}

lgsa_status latent_gate(const void* q_lat, const void* w_gate, const void* o, void* out, int M,
                        int d_lat, int N, int dt, void* stream) {
  REQUIRE(dt == LGSA_F32 || dt == LGSA_BF16, LGSA_EINVAL, "latent_gate: unknown dt %d", dt);
  REQUIRE(M >= 0 && d_lat >= 1 && N >= 1, LGSA_EINVAL,
          "latent_gate: M must be >= 0 and d_lat, N >= 1");
  REQUIRE(q_lat && w_gate && o && out, LGSA_EINVAL,
          "latent_gate: q_lat, w_gate, o, out must be non-NULL");
  if (dt == LGSA_BF16) {
    REQUIRE(d_lat % 64 == 0 && N % 16 == 0, LGSA_EUNSUPPORTED,
            "latent_gate: bf16 needs d_lat %% 64 == 0 and N %% 16 == 0 (got %d, %d)", d_lat, N);
    REQUIRE(aligned(q_lat, 16) && aligned(w_gate, 16) && aligned(o, 16) && aligned(out, 16),
            LGSA_EINVAL, "latent_gate: bf16 tensors must be 16-byte aligned");
  }
  return hip_status(lgsa::launch_gate(q_lat, w_gate, o, out, M, d_lat, N, dt,
                                      (hipStream_t)stream),
                    "latent_gate");
}

lgsa_status latent_gate_bwd_workspace(int M, int d_lat, int N, int dt, size_t* bytes) {
  REQUIRE(bytes != nullptr, LGSA_EINVAL, "latent_gate_bwd_workspace: bytes is NULL");
  REQUIRE(dt == LGSA_F32 || dt == LGSA_BF16, LGSA_EINVAL, "latent_gate_bwd: unknown dt %d", dt);
  REQUIRE(M >= 0 && d_lat >= 1 && N >= 1, LGSA_EINVAL,
          "latent_gate_bwd: M must be >= 0 and d_lat, N >= 1");
  *bytes = (size_t)M * (size_t)N * (dt == LGSA_BF16 ? 2 : 4);
  return ok();
}

lgsa_status latent_gate_bwd(const void* q_lat, const void* w_gate, const void* o,
                            const void* dout, void* d_o, void* dq_lat, void* dw_gate, int M,
                            int d_lat, int N, int dt, void* workspace, size_t workspace_bytes,
                            void* stream) {
  size_t need = 0;
  const lgsa_status s = latent_gate_bwd_workspace(M, d_lat, N, dt, &need);
  if (s != LGSA_OK) return s;
  REQUIRE(q_lat && w_gate && o && dout && d_o && dq_lat && dw_gate, LGSA_EINVAL,
          "latent_gate_bwd: q_lat, w_gate, o, dout, d_o, dq_lat, dw_gate must be non-NULL");
  if (dt == LGSA_BF16) {
    REQUIRE(d_lat % 64 == 0 && N % 16 == 0, LGSA_EUNSUPPORTED,
            "latent_gate_bwd: bf16 needs d_lat %% 64 == 0 and N %% 16 == 0 (got %d, %d)", d_lat,
            N);
  }
  REQUIRE(aligned(q_lat, 16) && aligned(w_gate, 16) && aligned(o, 16) && aligned(dout, 16) &&
              aligned(d_o, 16) && aligned(dq_lat, 16) && aligned(dw_gate, 16),
          LGSA_EINVAL, "latent_gate_bwd: every tensor must be 16-byte aligned");
  const lgsa_status w = check_workspace("latent_gate_bwd", workspace, workspace_bytes, need);
  if (w != LGSA_OK) return w;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = lgsa::launch_gate_bwd_elem(q_lat, w_gate, o, dout, d_o, workspace, M, d_lat,
                                            N, dt, st);
  // dq_lat [M, d_lat] = dG [M, N] (k-contiguous) x W^T (W rows are d_lat, k-contiguous)
  if (e == hipSuccess)
    e = lgsa::launch_gemm(workspace, N, false, w_gate, N, false, dq_lat, d_lat, M, d_lat, N, dt,
                          st);
  // dw_gate [d_lat, N] = q_lat^T (k-major, k = rows of q_lat) x dG (k-major)
  if (e == hipSuccess)
    e = lgsa::launch_gemm(q_lat, d_lat, true, workspace, N, true, dw_gate, N, d_lat, N, M, dt,
                          st);
  return hip_status(e, "latent_gate_bwd");
}

lgsa_status sparse_attn_bwd_workspace(const lgsa_sparse_bwd_args* a, size_t* bytes) {
  REQUIRE(bytes != nullptr, LGSA_EINVAL, "sparse_attn_bwd_workspace: bytes is NULL");
  const lgsa_status s = check_sparse_bwd(a);
  if (s != LGSA_OK) return s;
  *bytes = lgsa::sparse_bwd_workspace(to_params(a));
  return LGSA_OK;
}

lgsa_status sparse_attn_bwd(const lgsa_sparse_bwd_args* a, void* stream) {
  const lgsa_status s = check_sparse_bwd(a);
  if (s != LGSA_OK) return s;
  const lgsa::SparseBwdParams p = to_params(a);
  const lgsa_status w = check_workspace("sparse_attn_bwd", a->workspace, a->workspace_bytes,
                                        lgsa::sparse_bwd_min_workspace(p));
  if (w != LGSA_OK) return w;
  return hip_status(lgsa::launch_sparse_bwd(p, (hipStream_t)stream), "sparse_attn_bwd");
}

lgsa_status hca_attn_bwd_workspace(const lgsa_hca_bwd_args* a, size_t* bytes) {
  REQUIRE(bytes != nullptr, LGSA_EINVAL, "hca_attn_bwd_workspace: bytes is NULL");
  const lgsa_status s = check_hca_bwd(a);
  if (s != LGSA_OK) return s;
  *bytes = lgsa::hca_bwd_workspace(to_params(a));
  return ok();
}

lgsa_status hca_attn_bwd(const lgsa_hca_bwd_args* a, void* stream) {
  const lgsa_status s = check_hca_bwd(a);
  if (s != LGSA_OK) return s;
  const lgsa::HcaBwdParams p = to_params(a);
  const lgsa_status w = check_workspace("hca_attn_bwd", a->workspace, a->workspace_bytes,
                                        lgsa::hca_bwd_workspace(p));
  if (w != LGSA_OK) return w;
  return hip_status(lgsa::launch_hca_bwd(p, (hipStream_t)stream), "hca_attn_bwd");
}

lgsa_status hca_attn_fwd_workspace(const lgsa_hca_args* a, size_t* bytes) {
  REQUIRE(bytes != nullptr, LGSA_EINVAL, "hca_attn_fwd_workspace: bytes is NULL");
  const lgsa_status s = check_hca(a);
  if (s != LGSA_OK) return s;
  *bytes = hca_ws(a);
  return ok();
}

lgsa_status hca_attn_fwd(const lgsa_hca_args* a, void* stream) {
  const lgsa_status s = check_hca(a);
  if (s != LGSA_OK) return s;
  const lgsa_status w = check_workspace("hca_attn_fwd", a->workspace, a->workspace_bytes,
                                        hca_ws(a));
  if (w != LGSA_OK) return w;
  const lgsa::HcaParams p = to_params(a);
  const hipError_t e = a->dt == LGSA_BF16 ? lgsa::launch_hca_bf16(p, (hipStream_t)stream)
                                          : lgsa::launch_hca_f32(p, (hipStream_t)stream);
  return hip_status(e, "hca_attn_fwd");
}

// ------------------------------------------------------------------ allocation-free variant
// hca_attn_fwd_static takes its scratch from `scratch`, a file-scope device array that every
// GPU the library runs on holds until the process ends.  In host code the array's name is a
// host-side stand-in, not a device address: its device address on the current GPU is looked up
// once per device (first call on that device, with the device current) and kept in
// g_scratch_dev, which is what the launch receives.
namespace {

static __device__ __align__(256) unsigned char scratch[LGSA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

lgsa_status static_scratch(const char* who, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LGSA_EHIP, "%s: hipGetDevice failed: %s", who, hipGetErrorString(e));
  REQUIRE(dev >= 0 && dev < kMaxDevices, LGSA_EUNSUPPORTED,
          "%s: device ordinal %d is beyond the %d devices the static scratch tracks", who, dev,
          kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(LGSA_EHIP, "%s: hipGetSymbolAddress of the static scratch failed: %s", who,
                  hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return LGSA_OK;
}

}  // namespace

lgsa_status hca_attn_fwd_static(const lgsa_hca_args* a, void* stream) {
  const lgsa_status s = check_hca(a);
  if (s != LGSA_OK) return s;
  const size_t need = hca_ws(a);
  REQUIRE(need <= (size_t)LGSA_STATIC_SCRATCH_BYTES, LGSA_EWORKSPACE,
          "hca_attn_fwd_static: the call needs %zu bytes of scratch, more than the %zu the "
          "library holds per GPU (LGSA_STATIC_SCRATCH_BYTES); use hca_attn_fwd with a workspace",
          need, (size_t)LGSA_STATIC_SCRATCH_BYTES);
  lgsa::HcaParams p = to_params(a);
  p.ws = nullptr;
  p.ws_bytes = 0;
  if (need > 0) {
    const lgsa_status g = static_scratch("hca_attn_fwd_static", &p.ws);
    if (g != LGSA_OK) return g;
    p.ws_bytes = (size_t)LGSA_STATIC_SCRATCH_BYTES;
  }
  const hipError_t e = a->dt == LGSA_BF16 ? lgsa::launch_hca_bf16(p, (hipStream_t)stream)
                                          : lgsa::launch_hca_f32(p, (hipStream_t)stream);
  return hip_status(e, "hca_attn_fwd_static");
}

lgsa_status dsa_index_topk_workspace(const lgsa_index_args* a, size_t* bytes) {
  REQUIRE(bytes != nullptr, LGSA_EINVAL, "dsa_index_topk_workspace: bytes is NULL");
  const lgsa_status s = check_index(a);
  if (s != LGSA_OK) return s;
  *bytes = lgsa::index_workspace(to_params(a));
  return ok();
}

lgsa_status dsa_index_topk(const lgsa_index_args* a, void* stream) {
  const lgsa_status s = check_index(a);
  if (s != LGSA_OK) return s;
  const lgsa::IndexParams p = to_params(a);
  // the prefill path streams queries through the workspace in chunks, so it needs one row
  // of scores at least; the decode path needs exactly what the query reports
  const size_t need = lgsa::index_min_workspace(p);
  const lgsa_status w = check_workspace("dsa_index_topk", a->workspace, a->workspace_bytes, need);
  if (w != LGSA_OK) return w;
  return hip_status(lgsa::launch_index(p, (hipStream_t)stream), "dsa_index_topk");
}

lgsa_status sparse_attn_fwd_workspace(const lgsa_sparse_args* a, size_t* bytes) {
  REQUIRE(bytes != nullptr, LGSA_EINVAL, "sparse_attn_fwd_workspace: bytes is NULL");
  const lgsa_status s = check_sparse(a);
  if (s != LGSA_OK) return s;
  *bytes = lgsa::sparse_workspace(to_params(a));
  return ok();
}

lgsa_status sparse_attn_fwd(const lgsa_sparse_args* a, void* stream) {
  const lgsa_status s = check_sparse(a);
  if (s != LGSA_OK) return s;
  const lgsa::SparseParams p = to_params(a);
  const lgsa_status w = check_workspace("sparse_attn_fwd", a->workspace, a->workspace_bytes,
                                        lgsa::sparse_workspace(p));
  if (w != LGSA_OK) return w;
  return hip_status(lgsa::launch_sparse(p, (hipStream_t)stream), "sparse_attn_fwd");
}

lgsa_status sparse_gather_probe(const void* rows, long long row_stride, int S,
                                const int32_t* idx, int n_lists, int k, uint32_t* sums,
                                void* stream) {
  REQUIRE(rows && idx && sums, LGSA_EINVAL,
          "sparse_gather_probe: rows, idx and sums must be non-NULL");
  REQUIRE(S >= 1 && n_lists >= 0 && k >= 1, LGSA_EINVAL,
          "sparse_gather_probe: S, k must be >= 1 and n_lists >= 0");
  REQUIRE(row_stride >= 256 && row_stride % 8 == 0, LGSA_EUNSUPPORTED,
          "sparse_gather_probe: row_stride must be >= 256 and a multiple of 8 (got %lld)",
          row_stride);
  REQUIRE(aligned(rows, 16) && aligned(idx, 4) && aligned(sums, 4), LGSA_EINVAL,
          "sparse_gather_probe: rows must be 16-byte aligned, idx and sums 4-byte aligned");
  return hip_status(lgsa::launch_gather_probe(rows, row_stride, S, idx, n_lists, k, sums,
                                              (hipStream_t)stream),
                    "sparse_gather_probe");
}

}  // extern "C"
