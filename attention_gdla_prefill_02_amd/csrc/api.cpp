// C ABI of libgdla: argument checks, workspace carving and the launch
// sequence of one GDLA layer (prefill), one decode step, and the latent
// expansion.  Every check runs before the first launch, so a non-OK return
// has enqueued nothing.  Nothing here allocates or synchronizes.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/gdla.h"
#include "backward.h"
#include "decode.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

gdla_status fail(gdla_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

gdla_status hip_fail(hipError_t e, const char* where) {
  return fail(GDLA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Dims {
  int64_t d, rq, rkv, nN, g, dn, dr, dv, nS, H, dqk, ndown, nq, ngate;
  int elt;   // bytes per element of the config dtype
};

Dims dims_of(const gdla_config* c) {
  Dims D;
  D.d = c->d_model; D.rq = c->q_rank; D.rkv = c->kv_rank; D.nN = c->n_noise; D.g = c->group;
  D.dn = c->d_nope; D.dr = c->d_rope; D.dv = c->d_v;
  D.nS = D.g * D.nN; D.H = D.nS + D.nN; D.dqk = D.dn + D.dr;
  D.ndown = D.rq + D.rkv + D.dr + D.nS;
  D.nq = D.H * D.dqk;
  D.ngate = D.nS * D.dv;
  D.elt = c->dtype == GDLA_BF16 ? 2 : 4;
  return D;
}

// Shape checks shared by every entry point.
gdla_status check_config(const gdla_config* c) {
  if (!c) return fail(GDLA_ERR_INVALID_ARG, "cfg is NULL");
  if (c->dtype != GDLA_BF16 && c->dtype != GDLA_FP32) return fail(GDLA_ERR_INVALID_ARG, "unknown dtype %d", (int)c->dtype);
  if (c->d_model <= 0 || c->q_rank <= 0 || c->kv_rank <= 0 || c->n_noise <= 0 || c->group <= 0 ||
      c->d_nope <= 0 || c->d_rope <= 0 || c->d_v <= 0)
    return fail(GDLA_ERR_INVALID_ARG, "every dimension must be positive");
  if (c->d_rope % 2) return fail(GDLA_ERR_INVALID_ARG, "d_rope must be even (got %d)", c->d_rope);
  if (!(c->rope_base > 0.f) || !std::isfinite(c->rope_base)) return fail(GDLA_ERR_INVALID_ARG, "rope_base must be positive");
  if (!(c->rms_eps >= 0.f) || !std::isfinite(c->rms_eps)) return fail(GDLA_ERR_INVALID_ARG, "rms_eps must be >= 0");
  if (std::isnan(c->yarn_factor)) return fail(GDLA_ERR_INVALID_ARG, "yarn_factor is NaN");
  if (c->yarn_factor > 1.f &&
      !(std::isfinite(c->yarn_factor) && c->yarn_orig_len > 0 && std::isfinite(c->yarn_beta_fast) &&
        c->yarn_beta_slow > 0.f && c->yarn_beta_fast > c->yarn_beta_slow))
    return fail(GDLA_ERR_INVALID_ARG, "YaRN needs a finite factor, yarn_orig_len > 0 and beta_fast > beta_slow > 0");
  if (c->yarn_temperature != GDLA_YARN_TEMP_ROTARY && c->yarn_temperature != GDLA_YARN_TEMP_LOGIT)
    return fail(GDLA_ERR_INVALID_ARG, "unknown yarn_temperature %d", (int)c->yarn_temperature);
  const int64_t H = (int64_t)c->group * c->n_noise + c->n_noise;
  if (H * (c->d_nope + c->d_rope) > (1 << 24)) return fail(GDLA_ERR_INVALID_ARG, "too many query heads");
  if (c->dtype == GDLA_BF16) {
    if (c->d_nope != 128 || c->d_rope != 64 || c->d_v != 128)
      return fail(GDLA_ERR_UNSUPPORTED, "bf16 path needs d_nope=128, d_rope=64, d_v=128 (got %d, %d, %d)",
                  c->d_nope, c->d_rope, c->d_v);
    if (c->group > 4) return fail(GDLA_ERR_UNSUPPORTED, "bf16 path supports group <= 4 (got %d)", c->group);
    if (c->d_model % 64 || c->q_rank % 64 || c->kv_rank % 64)
      return fail(GDLA_ERR_UNSUPPORTED, "bf16 path needs d_model, q_rank, kv_rank multiples of 64");
  } else {
    if (c->d_nope + c->d_rope > 256 || c->d_v > 256)
      return fail(GDLA_ERR_UNSUPPORTED, "fp32 path needs d_nope + d_rope <= 256 and d_v <= 256");
  }
  return GDLA_OK;
}

// Prefill workspace: every intermediate of the layer, each 256-byte aligned,
// for a stream of T tokens; plan_bytes for the packed attention's work list.
struct PrefillLayout {
  size_t down, cqn, ckvn, kr, lam, rope, q, gate, kc, vt, z, plan, blas, total;
  int64_t vt_ld;
};

PrefillLayout prefill_layout(const Dims& D, int64_t T, size_t plan_bytes) {
  PrefillLayout P;
  const int e = D.elt;
  P.vt_ld = (T + 63) / 64 * 64;
  size_t o = 0;
  P.down = o; o = align256(o + (size_t)T * D.ndown * 4);
  P.cqn = o;  o = align256(o + (size_t)T * D.rq * e);
  P.ckvn = o; o = align256(o + (size_t)T * D.rkv * 2 * e);
  P.kr = o;   o = align256(o + (size_t)T * D.dr * e);
  P.lam = o;  o = align256(o + (size_t)T * D.nS * 4);
  P.rope = o; o = align256(o + (size_t)T * D.dr * 4);
  P.q = o;    o = align256(o + (size_t)T * D.nq * e);
  P.gate = o; o = align256(o + (size_t)T * D.ngate * 4);
  P.kc = o;   o = align256(o + (size_t)T * D.nN * D.dn * e);
  P.vt = o;   o = align256(o + (size_t)D.nN * D.dv * P.vt_ld * e);
  P.z = o;    o = align256(o + (size_t)T * D.nS * D.dv * e);
  P.plan = o; o = align256(o + plan_bytes);
  P.blas = o; o = align256(o + (D.elt == 2 ? gdla::blas_workspace_bytes() : 0));   // hipBLASLt's workspace (bf16)
  P.total = o;
  return P;
}

constexpr int64_t PACKED_MAX_T = (int64_t)1 << 20;

// Workspace of a packed call; 0 when the sizes are outside the supported range.
size_t packed_plan_bytes(const gdla_config* c, int32_t n_seq, int64_t T) {
  if (c->dtype != GDLA_BF16) return 0;
  return gdla::attn_plan_bytes(n_seq, T, c->group);
}

gdla_status check_weights(const gdla_weights* w) {
  if (!w) return fail(GDLA_ERR_INVALID_ARG, "weights is NULL");
  const void* ps[] = {w->w_dq, w->g_q, w->w_dkv, w->g_kv, w->w_lambda, w->w_uq, w->w_ukv, w->w_gate, w->w_o};
  const char* names[] = {"w_dq", "g_q", "w_dkv", "g_kv", "w_lambda", "w_uq", "w_ukv", "w_gate", "w_o"};
  for (int i = 0; i < 9; ++i) {
    if (!ps[i]) return fail(GDLA_ERR_INVALID_ARG, "weight %s is NULL", names[i]);
    if (!aligned16(ps[i])) return fail(GDLA_ERR_INVALID_ARG, "weight %s is not 16-byte aligned", names[i]);
  }
  return GDLA_OK;
}

gdla_status check_paged(const gdla_paged_cache* c) {
  if (!c->pages || !c->block_table) return fail(GDLA_ERR_INVALID_ARG, "cache pages and block_table must be non-NULL");
  if (!aligned16(c->pages) || ((uintptr_t)c->block_table & 3))
    return fail(GDLA_ERR_INVALID_ARG, "cache pages must be 16-byte aligned, block_table 4-byte aligned");
  if (c->page_rows < 32 || (c->page_rows & (c->page_rows - 1)))
    return fail(GDLA_ERR_INVALID_ARG, "page_rows must be a power of two >= 32 (got %d)", c->page_rows);
  if (c->max_pages <= 0 || c->num_pages <= 0)
    return fail(GDLA_ERR_INVALID_ARG, "max_pages and num_pages must be positive");
  if ((int64_t)c->page_rows * c->max_pages > ((int64_t)1 << 30))
    return fail(GDLA_ERR_INVALID_ARG, "page_rows * max_pages beyond 2^30 positions");
  return GDLA_OK;
}

gdla::CacheView paged_view(const gdla_paged_cache* c) {
  return gdla::CacheView{c->pages, c->block_table, c->page_rows, c->max_pages, c->num_pages};
}

// The sequences of one prefill call: B of L rows each (cu == nullptr) or a
// packed stream (cu, nseq, per-sequence first positions).
struct Stream {
  int64_t T;
  int B, L;
  int64_t pos_offset;
  const int32_t* cu;
  int nseq;
  const int32_t* seq_pos;
};

// Launch sequence of one layer; every argument has been checked.
gdla_status run_prefill(const gdla_config* cfg, const gdla_weights* w, const Stream& S, const void* x, void* y,
                        const void* residual, const gdla::CacheView& cache, char* ws, const PrefillLayout& P,
                        hipStream_t s, uint32_t stages) {
  using namespace gdla;
  const Dims D = dims_of(cfg);
  const bool bf = cfg->dtype == GDLA_BF16;
  const int64_t T = S.T;
  const int e = D.elt;
  auto gemm = bf ? gemm_bf16 : gemm_f32;
  hipError_t err;

  // 1. fused down-projection: [c_Q | c_KV k_R | lambda logit] = x [W_DQ; W_DKV; W_l]^T (fp32 out)
  if (stages & GDLA_STAGE_DOWN) {
    GemmArgs g{};
    g.A = x; g.lda = D.d;
    g.B = w->w_dq; g.ldb = D.d;
    g.B2 = w->w_dkv; g.nb2 = (int)D.rq;
    g.B3 = w->w_lambda; g.nb3 = (int)(D.rq + D.rkv + D.dr);
    g.C = ws + P.down; g.ldc = D.ndown;
    g.M = (int)T; g.N = (int)D.ndown; g.K = (int)D.d; g.batch = 1; g.epi = EPI_F32;
    if ((err = gemm(g, s)) != hipSuccess) return hip_fail(err, "down-projection");
  }
  // 2. row prep: norms, rotary key, lambda, RoPE table, cache rows
  if (stages & GDLA_STAGE_PREP) {
    RowPrepArgs r{};
    r.down = (const float*)(ws + P.down); r.ld_down = D.ndown;
    r.T = T; r.L = S.L; r.pos_offset = S.pos_offset;
    r.cu = S.cu; r.nseq = S.nseq; r.seq_pos = S.seq_pos;
    r.q_rank = (int)D.rq; r.kv_rank = (int)D.rkv; r.d_rope = (int)D.dr; r.nS = (int)D.nS;
    r.g_q = w->g_q; r.g_kv = w->g_kv; r.eps = cfg->rms_eps;
    set_rope(r, cfg->rope_base, cfg->window, cfg->yarn_factor, cfg->yarn_orig_len, cfg->yarn_beta_fast,
             cfg->yarn_beta_slow, cfg->yarn_temperature);
    r.cqn = ws + P.cqn; r.ckvn = ws + P.ckvn; r.kr = ws + P.kr; r.lam = (float*)(ws + P.lam);
    r.rope = (float*)(ws + P.rope); r.cache = cache;
    r.split_kv = bf;
    r.kr_f16 = bf;   // the attention's rotary keys in fp16 (the cache rows stay bf16)
    if ((err = rowprep(r, bf, s)) != hipSuccess) return hip_fail(err, "row prep");
  }
  // 3. latent expansion: K^C = c_KVn W_UK^T (token-major), V^T = W_UV c_KVn^T
  //    (token t in column t).  bf16: c_KVn enters as [hi | lo] over K =
  //    2*kv_rank against the weight read twice (K wrap), so the expansion does
  //    not round the latent.
  if (stages & GDLA_STAGE_EXPAND) {
    const int64_t kk = bf ? 2 * D.rkv : D.rkv;
    GemmArgs g{};
    g.A = ws + P.ckvn; g.lda = kk;
    g.B = w->w_ukv; g.ldb = D.rkv; g.kwrapB = bf ? (int)D.rkv : 0;
    g.C = ws + P.kc; g.ldc = D.nN * D.dn;
    g.M = (int)T; g.N = (int)(D.nN * D.dn); g.K = (int)kk; g.batch = 1; g.epi = EPI_STORE;
    g.out_f16 = bf;   // content keys in fp16 (score operand)
    if ((err = gemm(g, s)) != hipSuccess) return hip_fail(err, "latent expand (keys)");
    GemmArgs v{};
    v.A = (const char*)w->w_ukv + (size_t)D.nN * D.dn * D.rkv * e; v.lda = D.rkv;
    v.kwrapA = bf ? (int)D.rkv : 0;
    v.B = ws + P.ckvn; v.ldb = kk;
    v.C = ws + P.vt; v.ldc = P.vt_ld;
    v.M = (int)(D.nN * D.dv); v.N = (int)T; v.K = (int)kk; v.batch = 1; v.epi = EPI_STORE;
    v.Npad = (int)P.vt_ld;   // the attention kernel reads whole 32-key tiles: pad with zeros
    if ((err = gemm(v, s)) != hipSuccess) return hip_fail(err, "latent expand (values)");
  }
  // 4. query up-projection with RoPE on the rotary parts, and the sigmoid gate
  //    (fp32): [Q | G] = c_Qn [W_UQ; W_G]^T
  if (stages & GDLA_STAGE_QG) {
    if (bf) {
      GemmArgs g{};
      g.A = ws + P.cqn; g.lda = D.rq;
      g.B = w->w_uq; g.ldb = D.rq;
      g.B2 = w->w_gate; g.nb2 = (int)D.nq;
      g.C = ws + P.q; g.ldc = D.nq;
      g.G = (float*)(ws + P.gate); g.ldg = D.ngate;
      g.M = (int)T; g.N = (int)(D.nq + D.ngate); g.K = (int)D.rq; g.batch = 1; g.epi = EPI_QG;
      g.out_f16 = true;   // queries in fp16 (score operand); the gate stays fp32
      g.rope = (const float*)(ws + P.rope); g.q_cols = (int)D.nq;
      g.d_qk = (int)D.dqk; g.d_nope = (int)D.dn; g.d_rope = (int)D.dr;
      if ((err = gemm(g, s)) != hipSuccess) return hip_fail(err, "query/gate projection");
    } else {
      GemmArgs g{};
      g.A = ws + P.cqn; g.lda = D.rq;
      g.B = w->w_uq; g.ldb = D.rq;
      g.C = ws + P.q; g.ldc = D.nq;
      g.M = (int)T; g.N = (int)D.nq; g.K = (int)D.rq; g.batch = 1; g.epi = EPI_STORE;
      if ((err = gemm(g, s)) != hipSuccess) return hip_fail(err, "query projection");
      g.B = w->w_gate; g.C = ws + P.gate; g.ldc = D.ngate; g.N = (int)D.ngate;
      if ((err = gemm(g, s)) != hipSuccess) return hip_fail(err, "gate projection");
      if ((err = qg_finish((float*)(ws + P.q), D.nq, (float*)(ws + P.gate), D.ngate, T, (int)D.H, (int)D.ngate,
                           (int)D.dqk, (int)D.dn, (int)D.dr, (const float*)(ws + P.rope), s)) != hipSuccess)
        return hip_fail(err, "query/gate finish");
    }
  }
  // 5. attention, signal + noise heads, fused differential and gate (a packed
  //    bf16 stream first builds its work list)
  if (stages & GDLA_STAGE_ATTN) {
    AttnArgs a{};
    a.q = ws + P.q; a.ld_q = D.nq;
    a.gate = (const float*)(ws + P.gate); a.ld_gate = D.ngate;
    a.kc = ws + P.kc; a.ld_kc = D.nN * D.dn;
    a.kr = ws + P.kr;
    a.vt = ws + P.vt; a.ld_vt = P.vt_ld;
    a.lam = (const float*)(ws + P.lam);
    a.z = ws + P.z;
    a.T = T; a.B = S.B; a.L = S.L;
    a.cu = S.cu; a.nseq = S.nseq;
    a.nN = (int)D.nN; a.g = (int)D.g; a.window = cfg->window;
    a.d_nope = (int)D.dn; a.d_rope = (int)D.dr; a.d_v = (int)D.dv;
    a.scale = (float)(yarn_logit_multiplier(cfg->yarn_factor, cfg->window, cfg->yarn_temperature) /
                      std::sqrt((double)D.dqk));
    a.qk_f16 = bf;
    if (bf && S.cu) {
      int* plan = (int*)(ws + P.plan);
      if ((err = attn_plan(S.cu, S.nseq, T, (int)D.g, plan, s)) != hipSuccess) return hip_fail(err, "attention plan");
      a.plan = plan;
      a.items_cap = attn_plan_items(S.nseq, T, (int)D.g);
    }
    if ((err = bf ? attn_bf16(a, s) : attn_f32(a, s)) != hipSuccess) return hip_fail(err, "attention");
  }
  // 6. output projection (+ residual): hipBLASLt for bf16 (a plain GEMM; the
  //    residual is its C term), the library's GEMM otherwise or as the fallback
  if (stages & GDLA_STAGE_OUT) {
    if (bf) {
      err = blas_gemm(ws + P.z, D.nS * D.dv, w->w_o, D.nS * D.dv, residual, D.d, y, D.d, (int)T, (int)D.d,
                      (int)(D.nS * D.dv), false, ws + P.blas, blas_workspace_bytes(), s);
      if (err == hipSuccess) return GDLA_OK;
      if (err != hipErrorNotSupported) return hip_fail(err, "output projection (hipBLASLt)");
    }
    GemmArgs g{};
    g.A = ws + P.z; g.lda = D.nS * D.dv;
    g.B = w->w_o; g.ldb = D.nS * D.dv;
    g.C = y; g.ldc = D.d;
    g.R = residual; g.ldr = D.d;
    g.M = (int)T; g.N = (int)D.d; g.K = (int)(D.nS * D.dv); g.batch = 1; g.epi = EPI_STORE;
    if ((err = gemm(g, s)) != hipSuccess) return hip_fail(err, "output projection");
  }
  return GDLA_OK;
}

}  // namespace

namespace gdla {

// thread-local error detail for entry points outside this file
gdla_status report_error(gdla_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}
}  // namespace gdla

extern "C" {

const char* gdla_status_string(gdla_status s) {
  switch (s) {
    case GDLA_OK: return "GDLA_OK";
    case GDLA_ERR_INVALID_ARG: return "GDLA_ERR_INVALID_ARG";
    case GDLA_ERR_UNSUPPORTED: return "GDLA_ERR_UNSUPPORTED";
    case GDLA_ERR_WORKSPACE: return "GDLA_ERR_WORKSPACE";
    case GDLA_ERR_HIP: return "GDLA_ERR_HIP";
  }
  return "GDLA_ERR_UNKNOWN";
}

const char* gdla_last_error(void) { return g_err; }

int32_t gdla_version(void) { return 104; }   // 1.04: YaRN temperature setting in gdla_config

size_t gdla_prefill_workspace_size(const gdla_config* cfg, int32_t B, int32_t L) {
  if (check_config(cfg) != GDLA_OK || B < 0 || L < 0) return 0;
  return prefill_layout(dims_of(cfg), (int64_t)B * L, 0).total;
}

gdla_status gdla_prefill_workspace_layout(const gdla_config* cfg, int32_t B, int32_t L, gdla_prefill_layout* out) {
  gdla_status st = check_config(cfg);
  if (st != GDLA_OK) return st;
  if (!out) return fail(GDLA_ERR_INVALID_ARG, "out is NULL");
  if (B < 0 || L < 0) return fail(GDLA_ERR_INVALID_ARG, "B and L must be >= 0");
  const PrefillLayout P = prefill_layout(dims_of(cfg), (int64_t)B * L, 0);
  out->down = P.down; out->cqn = P.cqn; out->ckvn = P.ckvn; out->kr = P.kr; out->lam = P.lam;
  out->rope = P.rope; out->q = P.q; out->gate = P.gate; out->kc = P.kc; out->vt = P.vt; out->z = P.z;
  return GDLA_OK;
}

gdla_status gdla_prefill(const gdla_config* cfg, const gdla_weights* w, int32_t B, int32_t L, int64_t pos_offset,
                         const void* x, void* y, const void* residual, void* cache, int32_t cache_capacity,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return gdla_prefill_stages(cfg, w, B, L, pos_offset, x, y, residual, cache, cache_capacity, workspace,
                             workspace_bytes, stream, GDLA_STAGE_ALL);
}

gdla_status gdla_prefill_stages(const gdla_config* cfg, const gdla_weights* w, int32_t B, int32_t L,
                                int64_t pos_offset, const void* x, void* y, const void* residual, void* cache,
                                int32_t cache_capacity, void* workspace, size_t workspace_bytes, void* stream,
                                uint32_t stages) {
  gdla_status st = check_config(cfg);
  if (st != GDLA_OK) return st;
  if (B < 0 || L < 0) return fail(GDLA_ERR_INVALID_ARG, "B and L must be >= 0 (got %d, %d)", B, L);
  if (pos_offset < 0) return fail(GDLA_ERR_INVALID_ARG, "pos_offset must be >= 0");
  if (stages & ~(uint32_t)GDLA_STAGE_ALL) return fail(GDLA_ERR_INVALID_ARG, "unknown stage bits 0x%x", stages);
  if (B == 0 || L == 0) return GDLA_OK;
  const bool bf = cfg->dtype == GDLA_BF16;
  if (!bf && L > 8192) return fail(GDLA_ERR_UNSUPPORTED, "fp32 path supports L <= 8192 (got %d)", L);
  if ((int64_t)B * L > ((int64_t)1 << 31) / 8) return fail(GDLA_ERR_UNSUPPORTED, "B*L too large");
  st = check_weights(w);
  if (st != GDLA_OK) return st;
  if (!x || !y) return fail(GDLA_ERR_INVALID_ARG, "x and y must be non-NULL");
  if (!aligned16(x) || !aligned16(y) || (residual && !aligned16(residual)) || (cache && !aligned16(cache)))
    return fail(GDLA_ERR_INVALID_ARG, "x, y, residual and cache must be 16-byte aligned");
  if (x == y) return fail(GDLA_ERR_INVALID_ARG, "y must not alias x");
  if (cache && (int64_t)cache_capacity < pos_offset + L)
    return fail(GDLA_ERR_INVALID_ARG, "cache_capacity %d < pos_offset + L = %lld", cache_capacity,
                (long long)(pos_offset + L));
  if (pos_offset + L > (int64_t)1 << 30) return fail(GDLA_ERR_INVALID_ARG, "positions beyond 2^30");
  const PrefillLayout P = prefill_layout(dims_of(cfg), (int64_t)B * L, 0);
  if (!workspace) return fail(GDLA_ERR_WORKSPACE, "workspace is NULL (needs %zu bytes)", P.total);
  if (((uintptr_t)workspace & 255) != 0) return fail(GDLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < P.total)
    return fail(GDLA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, P.total);
  const Stream S{(int64_t)B * L, B, L, pos_offset, nullptr, 0, nullptr};
  const gdla::CacheView view{cache, nullptr, cache_capacity, 1, B};
  return run_prefill(cfg, w, S, x, y, residual, view, (char*)workspace, P, (hipStream_t)stream, stages);
}

size_t gdla_prefill_packed_workspace_size(const gdla_config* cfg, int32_t n_seq, int64_t T) {
  if (check_config(cfg) != GDLA_OK || n_seq < 0 || T < 0) return 0;
  const bool bf = cfg->dtype == GDLA_BF16;
  if (T > (bf ? PACKED_MAX_T : 8192) || n_seq > PACKED_MAX_T) return 0;
  const size_t plan = packed_plan_bytes(cfg, n_seq, T);
  if (bf && plan == 0) return 0;
  return prefill_layout(dims_of(cfg), T, plan).total;
}

gdla_status gdla_prefill_packed(const gdla_config* cfg, const gdla_weights* w, int32_t n_seq, int64_t T,
                                const int32_t* cu_seqlens, const int32_t* pos_offsets, const void* x, void* y,
                                const void* residual, const gdla_paged_cache* cache, void* workspace,
                                size_t workspace_bytes, void* stream) {
  gdla_status st = check_config(cfg);
  if (st != GDLA_OK) return st;
  if (n_seq < 0 || T < 0) return fail(GDLA_ERR_INVALID_ARG, "n_seq and T must be >= 0");
  if (T == 0) return GDLA_OK;
  if (n_seq == 0) return fail(GDLA_ERR_INVALID_ARG, "T = %lld tokens but no sequences", (long long)T);
  const bool bf = cfg->dtype == GDLA_BF16;
  if (T > (bf ? PACKED_MAX_T : 8192))
    return fail(GDLA_ERR_UNSUPPORTED, "packed prefill supports T <= %lld (got %lld)", (long long)(bf ? PACKED_MAX_T : 8192),
                (long long)T);
  if (n_seq > PACKED_MAX_T) return fail(GDLA_ERR_UNSUPPORTED, "packed prefill supports n_seq <= 2^20");
  st = check_weights(w);
  if (st != GDLA_OK) return st;
  if (!x || !y || !cu_seqlens) return fail(GDLA_ERR_INVALID_ARG, "x, y and cu_seqlens must be non-NULL");
  if (!aligned16(x) || !aligned16(y) || (residual && !aligned16(residual)))
    return fail(GDLA_ERR_INVALID_ARG, "x, y and residual must be 16-byte aligned");
  if (((uintptr_t)cu_seqlens & 3) || ((uintptr_t)pos_offsets & 3))
    return fail(GDLA_ERR_INVALID_ARG, "cu_seqlens and pos_offsets must be 4-byte aligned");
  if (x == y) return fail(GDLA_ERR_INVALID_ARG, "y must not alias x");
  if (cache && (st = check_paged(cache)) != GDLA_OK) return st;
  const PrefillLayout P = prefill_layout(dims_of(cfg), T, packed_plan_bytes(cfg, n_seq, T));
  if (!workspace) return fail(GDLA_ERR_WORKSPACE, "workspace is NULL (needs %zu bytes)", P.total);
  if (((uintptr_t)workspace & 255) != 0) return fail(GDLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < P.total)
    return fail(GDLA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, P.total);
  const Stream S{T, 0, 0, 0, cu_seqlens, n_seq, pos_offsets};
  const gdla::CacheView view = cache ? paged_view(cache) : gdla::CacheView{nullptr, nullptr, 1, 1, 0};
  return run_prefill(cfg, w, S, x, y, residual, view, (char*)workspace, P, (hipStream_t)stream, GDLA_STAGE_ALL);
}

gdla_status gdla_latent_expand(const gdla_config* cfg, int64_t T, const void* c_kv, int64_t ld_c, const void* g_kv,
                               const void* w_ukv, void* k_nope, void* v, void* c_norm, void* stream) {
  using namespace gdla;
  gdla_status st = check_config(cfg);
  if (st != GDLA_OK) return st;
  if (T < 0) return fail(GDLA_ERR_INVALID_ARG, "T must be >= 0");
  if (T == 0) return GDLA_OK;
  if (T > ((int64_t)1 << 31) / 8) return fail(GDLA_ERR_UNSUPPORTED, "T too large");
  if (ld_c < cfg->kv_rank) return fail(GDLA_ERR_INVALID_ARG, "ld_c (%lld) < kv_rank (%d)", (long long)ld_c, cfg->kv_rank);
  if (!c_kv || !g_kv || !w_ukv || !k_nope || !v || !c_norm)
    return fail(GDLA_ERR_INVALID_ARG, "c_kv, g_kv, w_ukv, k_nope, v and c_norm must be non-NULL");
  const void* ps[] = {c_kv, g_kv, w_ukv, k_nope, v, c_norm};
  for (const void* p : ps)
    if (!aligned16(p)) return fail(GDLA_ERR_INVALID_ARG, "all pointers must be 16-byte aligned");
  const Dims D = dims_of(cfg);
  if ((ld_c * D.elt) % 16) return fail(GDLA_ERR_INVALID_ARG, "ld_c rows must be 16-byte multiples");
  const bool bf = cfg->dtype == GDLA_BF16;
  hipStream_t s = (hipStream_t)stream;
  hipError_t err;
  LatentNormArgs n{c_kv, ld_c, T, (int)D.rkv, g_kv, cfg->rms_eps, c_norm, nullptr};
  if ((err = latent_norm(n, bf, s)) != hipSuccess) return hip_fail(err, "latent norm");
  auto gemm = bf ? gemm_bf16 : gemm_f32;
  GemmArgs g{};
  g.A = c_norm; g.lda = D.rkv;
  g.B = w_ukv; g.ldb = D.rkv;
  g.C = k_nope; g.ldc = D.nN * D.dn;
  g.M = (int)T; g.N = (int)(D.nN * D.dn); g.K = (int)D.rkv; g.batch = 1; g.epi = EPI_STORE;
  if ((err = gemm(g, s)) != hipSuccess) return hip_fail(err, "latent expand (keys)");
  g.B = (const char*)w_ukv + (size_t)D.nN * D.dn * D.rkv * D.elt;
  g.C = v; g.ldc = D.nN * D.dv; g.N = (int)(D.nN * D.dv);
  if ((err = gemm(g, s)) != hipSuccess) return hip_fail(err, "latent expand (values)");
  return GDLA_OK;
}

size_t gdla_decode_workspace_size(const gdla_config* cfg, int32_t B) {
  if (check_config(cfg) != GDLA_OK || B < 0 || !gdla::decode_supported(cfg)) return 0;
  return gdla::decode_workspace_bytes(cfg, B);
}

namespace {

// Checks shared by the dense and paged decode entry points (everything but the cache).
gdla_status check_decode(const gdla_config* cfg, const gdla_weights* w, int32_t B, const void* x, void* y,
                         const int32_t* cache_lens, void* workspace, size_t workspace_bytes) {
  gdla_status st = check_config(cfg);
  if (st != GDLA_OK) return st;
  if (cfg->dtype != GDLA_BF16) return fail(GDLA_ERR_UNSUPPORTED, "decode is bf16 only");
  if (!gdla::decode_supported(cfg))
    return fail(GDLA_ERR_UNSUPPORTED, "decode needs kv_rank in {128, 256, 512} and at most 80 query heads");
  if (B < 0) return fail(GDLA_ERR_INVALID_ARG, "B must be >= 0");
  if (B == 0) return GDLA_OK;
  st = check_weights(w);
  if (st != GDLA_OK) return st;
  if (!x || !y || !cache_lens) return fail(GDLA_ERR_INVALID_ARG, "x, y and cache_lens must be non-NULL");
  if (!aligned16(x) || !aligned16(y) || ((uintptr_t)cache_lens & 3))
    return fail(GDLA_ERR_INVALID_ARG, "x, y must be 16-byte aligned, cache_lens 4-byte aligned");
  const size_t need = gdla::decode_workspace_bytes(cfg, B);
  if (!workspace) return fail(GDLA_ERR_WORKSPACE, "workspace is NULL (needs %zu bytes)", need);
  if (((uintptr_t)workspace & 255) != 0) return fail(GDLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < need) return fail(GDLA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  return GDLA_OK;
}

}  // namespace

gdla_status gdla_decode(const gdla_config* cfg, const gdla_weights* w, int32_t B, const void* x, void* y, void* cache,
                        const int32_t* cache_lens, int32_t capacity, void* workspace, size_t workspace_bytes,
                        void* stream) {
  gdla_status st = check_decode(cfg, w, B, x, y, cache_lens, workspace, workspace_bytes);
  if (st != GDLA_OK || B == 0) return st;
  if (capacity <= 0) return fail(GDLA_ERR_INVALID_ARG, "capacity must be positive");
  if (!cache) return fail(GDLA_ERR_INVALID_ARG, "cache must be non-NULL");
  if (!aligned16(cache)) return fail(GDLA_ERR_INVALID_ARG, "cache must be 16-byte aligned");
  const gdla::CacheView view{cache, nullptr, capacity, 1, B};
  hipError_t err = gdla::decode_step(cfg, w, B, x, y, view, cache_lens, workspace, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "decode");
  return GDLA_OK;
}

gdla_status gdla_decode_paged(const gdla_config* cfg, const gdla_weights* w, int32_t B, const void* x, void* y,
                              const gdla_paged_cache* cache, const int32_t* cache_lens, void* workspace,
                              size_t workspace_bytes, void* stream) {
  gdla_status st = check_decode(cfg, w, B, x, y, cache_lens, workspace, workspace_bytes);
  if (st != GDLA_OK || B == 0) return st;
  if (!cache) return fail(GDLA_ERR_INVALID_ARG, "cache must be non-NULL");
  if ((st = check_paged(cache)) != GDLA_OK) return st;
  if ((int64_t)B * cache->max_pages > ((int64_t)1 << 28))
    return fail(GDLA_ERR_UNSUPPORTED, "B * max_pages beyond 2^28 block-table entries");
  hipError_t err = gdla::decode_step(cfg, w, B, x, y, paged_view(cache), cache_lens, workspace, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "decode");
  return GDLA_OK;
}

namespace {

gdla::BwdDims bwd_dims(const gdla_config* c) {
  const Dims D = dims_of(c);
  return gdla::BwdDims{D.d, D.rq, D.rkv, D.nN, D.g, D.dn, D.dr, D.dv, D.nS, D.H, D.dqk, D.ndown, D.nq, D.ngate};
}

gdla_status check_backward_shape(const gdla_config* cfg, int32_t B, int32_t L) {
  gdla_status st = check_config(cfg);
  if (st != GDLA_OK) return st;
  if (cfg->dtype != GDLA_BF16) return fail(GDLA_ERR_UNSUPPORTED, "backward is bf16 only");
  if (cfg->q_rank + cfg->kv_rank > 2048) return fail(GDLA_ERR_UNSUPPORTED, "backward needs q_rank + kv_rank <= 2048");
  if (B < 0 || L < 0) return fail(GDLA_ERR_INVALID_ARG, "B and L must be >= 0 (got %d, %d)", B, L);
  if ((int64_t)B * L > ((int64_t)1 << 22)) return fail(GDLA_ERR_UNSUPPORTED, "backward supports B*L <= 2^22");
  return GDLA_OK;
}

}  // namespace

size_t gdla_backward_workspace_size(const gdla_config* cfg, int32_t B, int32_t L) {
  if (check_backward_shape(cfg, B, L) != GDLA_OK) return 0;
  return gdla::backward_layout(bwd_dims(cfg), (int64_t)B * L).total;
}

namespace {

// Pointer and workspace checks shared by the uniform and the packed backward.
gdla_status check_backward_buffers(const gdla_weights* w, const void* x, const void* dy, void* dx,
                                   const gdla_grads* grads, void* workspace, size_t workspace_bytes, size_t need) {
  gdla_status st = check_weights(w);
  if (st != GDLA_OK) return st;
  if (!x || !dy || !dx || !grads) return fail(GDLA_ERR_INVALID_ARG, "x, dy, dx and grads must be non-NULL");
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dx))
    return fail(GDLA_ERR_INVALID_ARG, "x, dy and dx must be 16-byte aligned");
  if (dx == x || dx == dy) return fail(GDLA_ERR_INVALID_ARG, "dx must not alias x or dy");
  const float* gp[] = {grads->w_dq, grads->g_q, grads->w_dkv, grads->g_kv, grads->w_lambda,
                       grads->w_uq, grads->w_ukv, grads->w_gate, grads->w_o};
  for (const float* p : gp) {
    if (!p) return fail(GDLA_ERR_INVALID_ARG, "every gradient pointer must be non-NULL");
    if (!aligned16(p)) return fail(GDLA_ERR_INVALID_ARG, "gradient buffers must be 16-byte aligned");
  }
  if (!workspace) return fail(GDLA_ERR_WORKSPACE, "workspace is NULL (needs %zu bytes)", need);
  if (((uintptr_t)workspace & 255) != 0) return fail(GDLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < need) return fail(GDLA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  return GDLA_OK;
}

gdla_status check_backward_packed_shape(const gdla_config* cfg, int32_t n_seq, int64_t T) {
  gdla_status st = check_backward_shape(cfg, 0, 0);
  if (st != GDLA_OK) return st;
  if (n_seq < 0 || T < 0) return fail(GDLA_ERR_INVALID_ARG, "n_seq and T must be >= 0");
  if (T > ((int64_t)1 << 22)) return fail(GDLA_ERR_UNSUPPORTED, "packed backward supports T <= 2^22");
  if (n_seq > (1 << 20)) return fail(GDLA_ERR_UNSUPPORTED, "packed backward supports n_seq <= 2^20");
  return GDLA_OK;
}

}  // namespace

gdla_status gdla_backward(const gdla_config* cfg, const gdla_weights* w, int32_t B, int32_t L, int64_t pos_offset,
                          const void* x, const void* dy, void* dx, const gdla_grads* grads, void* workspace,
                          size_t workspace_bytes, void* stream) {
  gdla_status st = check_backward_shape(cfg, B, L);
  if (st != GDLA_OK) return st;
  if (pos_offset < 0) return fail(GDLA_ERR_INVALID_ARG, "pos_offset must be >= 0");
  if (B == 0 || L == 0) return GDLA_OK;
  if (pos_offset + L > (int64_t)1 << 30) return fail(GDLA_ERR_INVALID_ARG, "positions beyond 2^30");
  const gdla::BwdDims D = bwd_dims(cfg);
  const gdla::BackwardLayout P = gdla::backward_layout(D, (int64_t)B * L);
  st = check_backward_buffers(w, x, dy, dx, grads, workspace, workspace_bytes, P.total);
  if (st != GDLA_OK) return st;
  const gdla::BwdCall c{cfg, w, grads, B, L, (int64_t)B * L, pos_offset, x, dy, dx, workspace, nullptr, nullptr, 0};
  hipError_t err = gdla::backward_step(D, P, c, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "backward");
  return GDLA_OK;
}

size_t gdla_backward_packed_workspace_size(const gdla_config* cfg, int32_t n_seq, int64_t T) {
  if (check_backward_packed_shape(cfg, n_seq, T) != GDLA_OK || n_seq == 0) return 0;
  return gdla::backward_layout(bwd_dims(cfg), T, n_seq).total;
}

gdla_status gdla_backward_packed(const gdla_config* cfg, const gdla_weights* w, int32_t n_seq, int64_t T,
                                 const int32_t* cu_seqlens, const int32_t* pos_offsets, const void* x,
                                 const void* dy, void* dx, const gdla_grads* grads, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  gdla_status st = check_backward_packed_shape(cfg, n_seq, T);
  if (st != GDLA_OK) return st;
  if (T == 0) return GDLA_OK;
  if (n_seq == 0) return fail(GDLA_ERR_INVALID_ARG, "T = %lld tokens but no sequences", (long long)T);
  if (!cu_seqlens) return fail(GDLA_ERR_INVALID_ARG, "cu_seqlens must be non-NULL");
  if (((uintptr_t)cu_seqlens & 3) || ((uintptr_t)pos_offsets & 3))
    return fail(GDLA_ERR_INVALID_ARG, "cu_seqlens and pos_offsets must be 4-byte aligned");
  const gdla::BwdDims D = bwd_dims(cfg);
  const gdla::BackwardLayout P = gdla::backward_layout(D, T, n_seq);
  if (P.total == 0) return fail(GDLA_ERR_UNSUPPORTED, "stream too long for the work-list kernel");
  st = check_backward_buffers(w, x, dy, dx, grads, workspace, workspace_bytes, P.total);
  if (st != GDLA_OK) return st;
  const gdla::BwdCall c{cfg, w, grads, 0, 0, T, 0, x, dy, dx, workspace, cu_seqlens, pos_offsets, n_seq};
  hipError_t err = gdla::backward_step(D, P, c, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "packed backward");
  return GDLA_OK;
}

}  // extern "C"
