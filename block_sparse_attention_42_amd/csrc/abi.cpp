// Host side of the C ABI declared in include/bsa.h: argument validation,
// derived geometry and kernel dispatch.  Every check runs before any launch,
// so a non-OK status means nothing was enqueued.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/bsa.h"
#include "bsa_internal.h"

namespace {

thread_local std::string g_last_error;

bsa_status fail(bsa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
bsa_status fail(bsa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

bsa_status ok() {
  g_last_error.clear();
  return BSA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Derived {
  int64_t S;
  int32_t nqb, nkb;
  int32_t f0_first, f0_last;
  int32_t text_last;
};

// Geometry checks shared by every entry point.
bsa_status check_geometry(const bsa_geometry* g, Derived* d) {
  if (!g) return fail(BSA_ERR_INVALID_ARGUMENT, "geometry is NULL");
  if (g->B < 1 || g->H < 1) return fail(BSA_ERR_INVALID_ARGUMENT, "B=%d and H=%d must be >= 1", g->B, g->H);
  if (g->text_len < 0 || g->frames < 0 || g->latent_h < 0 || g->latent_w < 0)
    return fail(BSA_ERR_INVALID_ARGUMENT, "text_len, frames, latent_h, latent_w must be >= 0");
  if (g->head_dim != 64 && g->head_dim != 128)
    return fail(BSA_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", g->head_dim);
  if (g->q_block != 32 && g->q_block != 64)
    return fail(BSA_ERR_UNSUPPORTED, "q_block %d unsupported (32 or 64)", g->q_block);
  if (g->k_block != 16 && g->k_block != 32 && g->k_block != 64)
    return fail(BSA_ERR_UNSUPPORTED, "k_block %d unsupported (16, 32 or 64)", g->k_block);
  const int64_t S = (int64_t)g->text_len + (int64_t)g->frames * g->latent_h * g->latent_w;
  if (S < 1) return fail(BSA_ERR_INVALID_ARGUMENT, "sequence is empty (S = %lld)", (long long)S);
  const int64_t nqb = (S + g->q_block - 1) / g->q_block;
  const int64_t nkb = (S + g->k_block - 1) / g->k_block;
  if (nqb > (1 << 30) || nkb > (1 << 30)) return fail(BSA_ERR_UNSUPPORTED, "sequence too long");
  const int64_t need = std::max(nqb * g->q_block, nkb * g->k_block);
  if (g->seq_alloc < need)
    return fail(BSA_ERR_INVALID_ARGUMENT, "seq_alloc %lld < %lld (blocks of the padded sequence)",
                (long long)g->seq_alloc, (long long)need);
  if ((int64_t)g->B * g->H > (1 << 24)) return fail(BSA_ERR_UNSUPPORTED, "B*H too large");
  // every launch covers at most B*H*max(nqb, nkb) block rows, counted in 32 bits
  if ((int64_t)g->B * g->H * std::max(nqb, nkb) > 0x7fffffffLL)
    return fail(BSA_ERR_UNSUPPORTED, "B*H*max(nqb, nkb) = %lld block rows exceed one launch",
                (long long)((int64_t)g->B * g->H * std::max(nqb, nkb)));
  d->S = S;
  d->nqb = (int32_t)nqb;
  d->nkb = (int32_t)nkb;
  // frame-0 query blocks: frame-0 page, sec. 4
  if (g->frames > 0 && g->latent_h * g->latent_w > 0) {
    const int64_t start = g->text_len;
    const int64_t end = start + (int64_t)g->latent_h * g->latent_w;
    d->f0_first = (int32_t)(start / g->q_block);
    d->f0_last = (int32_t)((end - 1) / g->q_block);
  } else {
    d->f0_first = d->f0_last = -1;
  }
  d->text_last = g->text_len > 0 ? (int32_t)((g->text_len - 1) / g->k_block) : -1;
  return BSA_OK;
}

int32_t topk_of(const bsa_mask_params* p, int32_t nkb) {
  if (p->topk > 0) return p->topk < nkb ? p->topk : nkb;
  double k = std::ceil(p->keep_ratio * (double)nkb);
  if (k < 1) k = 1;
  if (k > nkb) k = nkb;
  return (int32_t)k;
}

bsa_status check_params(const bsa_mask_params* p, const Derived& d) {
  if (!p) return fail(BSA_ERR_INVALID_ARGUMENT, "mask params are NULL");
  if (p->mode != BSA_SELECT_TOPK && p->mode != BSA_SELECT_SAMPLE)
    return fail(BSA_ERR_INVALID_ARGUMENT, "unknown selection mode %d", p->mode);
  if (p->topk < 0) return fail(BSA_ERR_INVALID_ARGUMENT, "topk %d < 0", p->topk);
  const bool ratio_used = p->mode == BSA_SELECT_SAMPLE || p->topk == 0;
  if (ratio_used && !(std::isfinite(p->keep_ratio) && p->keep_ratio > 0.0 && p->keep_ratio <= 1.0))
    return fail(BSA_ERR_INVALID_ARGUMENT, "keep_ratio %g must be in (0, 1]", p->keep_ratio);
  (void)d;
  return BSA_OK;
}

}  // namespace

extern "C" {

int32_t bsa_abi_version(void) { return BSA_ABI_VERSION; }

const char* bsa_status_string(int32_t s) {
  switch (s) {
    case BSA_OK: return "ok";
    case BSA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case BSA_ERR_UNSUPPORTED: return "unsupported";
    case BSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* bsa_last_error(void) { return g_last_error.c_str(); }

bsa_status bsa_derive(const bsa_geometry* g, const bsa_mask_params* p, bsa_derived* out) {
  if (!out) return fail(BSA_ERR_INVALID_ARGUMENT, "out is NULL");
  Derived d;
  bsa_status s = check_geometry(g, &d);
  if (s != BSA_OK) return s;
  std::memset(out, 0, sizeof *out);
  out->S = d.S;
  out->nqb = d.nqb;
  out->nkb = d.nkb;
  out->frame0_first = d.f0_first;
  out->frame0_last = d.f0_last;
  out->text_last = d.text_last;
  if (p) {
    s = check_params(p, d);
    if (s != BSA_OK) return s;
    out->topk = topk_of(p, d.nkb);
    out->expected = (float)(p->keep_ratio * (double)d.nkb);
  }
  return ok();
}

bsa_status bsa_pool_blocks(const void* x, int32_t dtype, const bsa_geometry* g, int32_t block,
                           float* pooled, void* stream) {
  Derived d;
  bsa_status s = check_geometry(g, &d);
  if (s != BSA_OK) return s;
  if (dtype != BSA_DTYPE_BF16 && dtype != BSA_DTYPE_F32)
    return fail(BSA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (block != g->q_block && block != g->k_block)
    return fail(BSA_ERR_INVALID_ARGUMENT, "block %d is neither q_block nor k_block", block);
  if (!x || !pooled) return fail(BSA_ERR_INVALID_ARGUMENT, "x and pooled must not be NULL");
  if (!aligned16(x) || !aligned16(pooled))
    return fail(BSA_ERR_INVALID_ARGUMENT, "x and pooled must be 16-byte aligned");
  bsa::PoolArgs a;
  a.x = x;
  a.out = pooled;
  a.seq_alloc = g->seq_alloc;
  a.S = d.S;
  a.BH = g->B * g->H;
  a.D = g->head_dim;
  a.block = block;
  a.nb = (int32_t)((d.S + block - 1) / block);
  hipError_t e = bsa::launch_pool(a, dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BSA_ERR_HIP, "pool launch: %s", hipGetErrorString(e));
  return ok();
}

bsa_status bsa_pool_qk(const void* q, const void* k, int32_t dtype, const bsa_geometry* g, float* q_pooled,
                       float* k_pooled, void* stream) {
  Derived d;
  bsa_status s = check_geometry(g, &d);
  if (s != BSA_OK) return s;
  if (dtype != BSA_DTYPE_BF16 && dtype != BSA_DTYPE_F32)
    return fail(BSA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (!q || !k || !q_pooled || !k_pooled)
    return fail(BSA_ERR_INVALID_ARGUMENT, "q, k, q_pooled and k_pooled must not be NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_pooled) || !aligned16(k_pooled))
    return fail(BSA_ERR_INVALID_ARGUMENT, "q, k, q_pooled and k_pooled must be 16-byte aligned");
  bsa::PoolArgs a[2];
  const void* x[2] = {q, k};
  float* out[2] = {q_pooled, k_pooled};
  const int32_t block[2] = {g->q_block, g->k_block};
  for (int j = 0; j < 2; ++j) {
    a[j].x = x[j];
    a[j].out = out[j];
    a[j].seq_alloc = g->seq_alloc;
    a[j].S = d.S;
    a[j].BH = g->B * g->H;
    a[j].D = g->head_dim;
    a[j].block = block[j];
    a[j].nb = (int32_t)((d.S + block[j] - 1) / block[j]);
  }
  hipError_t e = bsa::launch_pool_jobs(a, 2, dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BSA_ERR_HIP, "pool launch: %s", hipGetErrorString(e));
  return ok();
}

bsa_status bsa_build_mask(const float* q_pooled, const float* k_pooled, const bsa_geometry* g,
                          const bsa_mask_params* p, uint8_t* mask, int32_t* kv_cnt,
                          int32_t* kv_idx, float* log_w, void* stream) {
  Derived d;
  bsa_status s = check_geometry(g, &d);
  if (s != BSA_OK) return s;
  s = check_params(p, d);
  if (s != BSA_OK) return s;
  if (!q_pooled || !k_pooled || !kv_cnt || !kv_idx)
    return fail(BSA_ERR_INVALID_ARGUMENT, "q_pooled, k_pooled, kv_cnt and kv_idx must not be NULL");
  if (!aligned16(q_pooled) || !aligned16(k_pooled) || !aligned16(kv_cnt) || !aligned16(kv_idx) ||
      (mask && !aligned16(mask)) || (log_w && !aligned16(log_w)))
    return fail(BSA_ERR_INVALID_ARGUMENT, "device buffers must be 16-byte aligned");
  if (p->mode == BSA_SELECT_SAMPLE && !log_w)
    return fail(BSA_ERR_INVALID_ARGUMENT, "sampling needs log_w");
  const int32_t nkb_max = p->mode == BSA_SELECT_SAMPLE ? 2048 : 8192;
  if (d.nkb > nkb_max)
    return fail(BSA_ERR_UNSUPPORTED, "nkb %d > %d for this selection mode", d.nkb, nkb_max);
  bsa::MaskArgs a;
  a.qp = q_pooled;
  a.kp = k_pooled;
  a.mask = mask;
  a.cnt = kv_cnt;
  a.idx = kv_idx;
  a.logw = log_w;
  a.H = g->H;
  a.BH = g->B * g->H;
  a.nqb = d.nqb;
  a.nkb = d.nkb;
  a.D = g->head_dim;
  a.mode = p->mode;
  a.topk = topk_of(p, d.nkb);
  a.expected = (float)(p->keep_ratio * (double)d.nkb);
  a.scale = (float)(1.0 / std::sqrt((double)g->head_dim));
  a.log_cluster = p->log_cluster ? 1 : 0;
  const int64_t n_last = d.S - (int64_t)(d.nkb - 1) * g->k_block;
  a.ln_full = (float)std::log((double)g->k_block);
  a.ln_last = (float)std::log((double)n_last);
  a.frame0_first = p->frame0_dense ? d.f0_first : -1;
  a.frame0_last = p->frame0_dense ? d.f0_last : -1;
  a.text_last = p->text_columns ? d.text_last : -1;
  a.seed = p->seed;
  a.imp = nullptr;
  hipError_t e = bsa::launch_mask(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BSA_ERR_HIP, "mask launch: %s", hipGetErrorString(e));
  return ok();
}

bsa_status bsa_cluster_importance(const void* q, int32_t dtype, const float* k_pooled,
                                  const bsa_geometry* g, int32_t n_clusters, int32_t iters,
                                  int32_t log_cluster, float* importance, void* stream) {
  Derived d;
  bsa_status s = check_geometry(g, &d);
  if (s != BSA_OK) return s;
  if (dtype != BSA_DTYPE_BF16 && dtype != BSA_DTYPE_F32)
    return fail(BSA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (!q || !k_pooled || !importance)
    return fail(BSA_ERR_INVALID_ARGUMENT, "q, k_pooled and importance must not be NULL");
  if (!aligned16(q) || !aligned16(k_pooled) || !aligned16(importance))
    return fail(BSA_ERR_INVALID_ARGUMENT, "device buffers must be 16-byte aligned");
  if (n_clusters < 1 || n_clusters > 8)
    return fail(BSA_ERR_INVALID_ARGUMENT, "n_clusters %d must be in 1..8", n_clusters);
  if (iters < 0 || iters > 16) return fail(BSA_ERR_INVALID_ARGUMENT, "iters %d must be in 0..16", iters);
  if (d.nkb > 8192 || (int64_t)n_clusters * d.nkb > 16384)
    return fail(BSA_ERR_UNSUPPORTED, "n_clusters * nkb = %lld > 16384 (or nkb > 8192)",
                (long long)n_clusters * d.nkb);
  if ((int64_t)g->B * g->H * d.nqb > 0x7fffffffLL)
    return fail(BSA_ERR_UNSUPPORTED, "too many query blocks for one launch");
  bsa::ImpArgs a;
  a.q = q;
  a.kp = k_pooled;
  a.imp = importance;
  a.seq_alloc = g->seq_alloc;
  a.S = d.S;
  a.BH = g->B * g->H;
  a.nqb = d.nqb;
  a.nkb = d.nkb;
  a.D = g->head_dim;
  a.q_block = g->q_block;
  a.C = n_clusters;
  a.T = iters;
  a.scale = (float)(1.0 / std::sqrt((double)g->head_dim));
  a.log_cluster = log_cluster ? 1 : 0;
  const int64_t n_last = d.S - (int64_t)(d.nkb - 1) * g->k_block;
  a.ln_full = (float)std::log((double)g->k_block);
  a.ln_last = (float)std::log((double)n_last);
  a.G = bsa::importance_group(n_clusters, d.nkb, d.nqb);
  a.area_a = 0;
  if (bsa::importance_lds_bytes(a) > 96 * 1024) return fail(BSA_ERR_UNSUPPORTED, "LDS budget exceeded");
  hipError_t e = bsa::launch_importance(a, dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BSA_ERR_HIP, "importance launch: %s", hipGetErrorString(e));
  return ok();
}

bsa_status bsa_select_blocks(const float* importance, const bsa_geometry* g, const bsa_mask_params* p,
                             uint8_t* mask, int32_t* kv_cnt, int32_t* kv_idx, float* log_w,
                             void* stream) {
  Derived d;
  bsa_status s = check_geometry(g, &d);
  if (s != BSA_OK) return s;
  s = check_params(p, d);
  if (s != BSA_OK) return s;
  if (!importance || !kv_cnt || !kv_idx)
    return fail(BSA_ERR_INVALID_ARGUMENT, "importance, kv_cnt and kv_idx must not be NULL");
  if (!aligned16(importance) || !aligned16(kv_cnt) || !aligned16(kv_idx) ||
      (mask && !aligned16(mask)) || (log_w && !aligned16(log_w)))
    return fail(BSA_ERR_INVALID_ARGUMENT, "device buffers must be 16-byte aligned");
  if (p->mode == BSA_SELECT_SAMPLE && !log_w)
    return fail(BSA_ERR_INVALID_ARGUMENT, "sampling needs log_w");
  const int32_t nkb_max = p->mode == BSA_SELECT_SAMPLE ? 2048 : 8192;
  if (d.nkb > nkb_max)
    return fail(BSA_ERR_UNSUPPORTED, "nkb %d > %d for this selection mode", d.nkb, nkb_max);
  bsa::MaskArgs a = {};
  a.imp = importance;
  a.mask = mask;
  a.cnt = kv_cnt;
  a.idx = kv_idx;
  a.logw = log_w;
  a.H = g->H;
  a.BH = g->B * g->H;
  a.nqb = d.nqb;
  a.nkb = d.nkb;
  a.D = g->head_dim;
  a.mode = p->mode;
  a.topk = topk_of(p, d.nkb);
  a.expected = (float)(p->keep_ratio * (double)d.nkb);
  a.frame0_first = p->frame0_dense ? d.f0_first : -1;
  a.frame0_last = p->frame0_dense ? d.f0_last : -1;
  a.text_last = p->text_columns ? d.text_last : -1;
  a.seed = p->seed;
  hipError_t e = bsa::launch_mask(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BSA_ERR_HIP, "selection launch: %s", hipGetErrorString(e));
  return ok();
}

bsa_status bsa_top_p_workspace_bytes(const bsa_geometry* g, int64_t* bytes) {
  if (!bytes) return fail(BSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  Derived d;
  bsa_status s = check_geometry(g, &d);
  if (s != BSA_OK) return s;
  *bytes = bsa::topp_workspace_bytes((int64_t)g->B * g->H, g->B, d.nqb, d.nkb);
  return ok();
}

bsa_status bsa_select_top_p(const float* scores, const float* v_pooled, const bsa_geometry* g,
                            const bsa_topp_params* tp, double* head_entropy, void* workspace,
                            int64_t workspace_bytes, uint8_t* mask, int32_t* kv_cnt, int32_t* kv_idx,
                            void* stream) {
  Derived d;
  bsa_status s = check_geometry(g, &d);
  if (s != BSA_OK) return s;
  if (!tp) return fail(BSA_ERR_INVALID_ARGUMENT, "top-p params are NULL");
  if (tp->domain < BSA_DOMAIN_ROW || tp->domain > BSA_DOMAIN_EG)
    return fail(BSA_ERR_INVALID_ARGUMENT, "unknown domain %d", tp->domain);
  if (!(std::isfinite(tp->top_p) && tp->top_p > 0.0 && tp->top_p <= 1.0))
    return fail(BSA_ERR_INVALID_ARGUMENT, "top_p %g must be in (0, 1]", tp->top_p);
  if (!(std::isfinite(tp->entropy_eps) && tp->entropy_eps > 0.0f))
    return fail(BSA_ERR_INVALID_ARGUMENT, "entropy_eps must be finite and > 0");
  if (!scores || !workspace || !kv_cnt || !kv_idx)
    return fail(BSA_ERR_INVALID_ARGUMENT, "scores, workspace, kv_cnt and kv_idx must not be NULL");
  if (tp->value_aware && !v_pooled) return fail(BSA_ERR_INVALID_ARGUMENT, "value-aware scores need v_pooled");
  if (!aligned16(scores) || !aligned16(workspace) || !aligned16(kv_cnt) || !aligned16(kv_idx) ||
      (mask && !aligned16(mask)) || (head_entropy && !aligned16(head_entropy)) ||
      (tp->value_aware && !aligned16(v_pooled)))
    return fail(BSA_ERR_INVALID_ARGUMENT, "device buffers must be 16-byte aligned");
  if (d.nkb > 2048) return fail(BSA_ERR_UNSUPPORTED, "nkb %d > 2048 for top-p selection", d.nkb);
  if (g->H > 4096) return fail(BSA_ERR_UNSUPPORTED, "H %d > 4096 for top-p selection", g->H);
  if ((int64_t)g->B * g->H * d.nqb > 0x7fffffffLL)
    return fail(BSA_ERR_UNSUPPORTED, "too many query blocks for one launch");
  const int64_t need = bsa::topp_workspace_bytes((int64_t)g->B * g->H, g->B, d.nqb, d.nkb);
  if (workspace_bytes < need)
    return fail(BSA_ERR_INVALID_ARGUMENT, "workspace of %lld bytes < %lld needed", (long long)workspace_bytes,
                (long long)need);
  bsa::TopPArgs a = {};
  a.scores = scores;
  a.vp = tp->value_aware ? v_pooled : nullptr;
  a.ws = workspace;
  a.entropy_out = head_entropy;
  a.mask = mask;
  a.cnt = kv_cnt;
  a.idx = kv_idx;
  a.B = g->B;
  a.H = g->H;
  a.BH = g->B * g->H;
  a.nqb = d.nqb;
  a.nkb = d.nkb;
  a.D = g->head_dim;
  a.vstride = (d.nkb + 3) / 4 * 4;
  a.npools = a.BH > 2 * g->B ? a.BH : 2 * g->B;
  a.domain = tp->domain;
  a.value_aware = tp->value_aware ? 1 : 0;
  a.top_p = tp->top_p;
  a.eps = tp->entropy_eps;
  a.frame0_first = tp->frame0_dense ? d.f0_first : -1;
  a.frame0_last = tp->frame0_dense ? d.f0_last : -1;
  a.text_last = tp->text_columns ? d.text_last : -1;
  hipError_t e = bsa::launch_topp(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BSA_ERR_HIP, "top-p launch: %s", hipGetErrorString(e));
  return ok();
}

bsa_status bsa_frame_scores(const float* scores, const bsa_geometry* g, int32_t window, double* alpha,
                            void* stream) {
  Derived d;
  bsa_status s = check_geometry(g, &d);
  if (s != BSA_OK) return s;
  if (!scores || !alpha) return fail(BSA_ERR_INVALID_ARGUMENT, "scores and alpha must not be NULL");
  if (!aligned16(scores) || !aligned16(alpha))
    return fail(BSA_ERR_INVALID_ARGUMENT, "device buffers must be 16-byte aligned");
  if (window < 1) return fail(BSA_ERR_INVALID_ARGUMENT, "window %d must be >= 1", window);
  if ((int64_t)g->latent_h * g->latent_w < 1 || g->frames < 1)
    return fail(BSA_ERR_INVALID_ARGUMENT, "frame scores need frames and latent_h * latent_w >= 1");
  if (g->frames > bsa::kMaxStructFrames)
    return fail(BSA_ERR_UNSUPPORTED, "frames %d > %d", g->frames, bsa::kMaxStructFrames);
  bsa::StructArgs a = {};
  a.scores = scores;
  a.alpha = alpha;
  a.S = d.S;
  a.text_len = g->text_len;
  a.tpf = (int64_t)g->latent_h * g->latent_w;
  a.frames = g->frames;
  a.BH = g->B * g->H;
  a.nqb = d.nqb;
  a.nkb = d.nkb;
  a.q_block = g->q_block;
  a.k_block = g->k_block;
  a.window = window;
  hipError_t e = bsa::launch_frame_scores(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BSA_ERR_HIP, "frame-score launch: %s", hipGetErrorString(e));
  return ok();
}

bsa_status bsa_classify_heads(const double* alpha, int32_t B, int32_t H, int32_t n_dummy, int32_t* classes) {
  if (!alpha || !classes) return fail(BSA_ERR_INVALID_ARGUMENT, "alpha and classes must not be NULL");
  if (B < 1 || H < 1) return fail(BSA_ERR_INVALID_ARGUMENT, "B=%d and H=%d must be >= 1", B, H);
  if (n_dummy < 0 || n_dummy > H) return fail(BSA_ERR_INVALID_ARGUMENT, "n_dummy %d must be in 0..H", n_dummy);
  for (int64_t t = 0; t < (int64_t)B * H * 3; ++t)
    if (!std::isfinite(alpha[t])) return fail(BSA_ERR_INVALID_ARGUMENT, "alpha[%lld] is not finite", (long long)t);
  std::vector<int32_t> order(H);
  for (int32_t b = 0; b < B; ++b) {
    const double* al = alpha + (int64_t)b * H * 3;
    auto lh = [&](int32_t h) { return std::max(al[h * 3 + 0], al[h * 3 + 1]); };
    for (int32_t h = 0; h < H; ++h) order[h] = h;
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return lh(x) < lh(y); });
    for (int32_t r = 0; r < H; ++r) {
      const int32_t h = order[r];
      classes[(int64_t)b * H + h] =
          r < n_dummy ? BSA_HEAD_DUMMY : (al[h * 3 + 0] > al[h * 3 + 1] ? BSA_HEAD_SINK : BSA_HEAD_NEIGHBOR);
    }
  }
  return ok();
}

bsa_status bsa_structured_lists(const int32_t* head_class, const bsa_geometry* g, const bsa_struct_params* sp,
                                uint8_t* mask, int32_t* kv_cnt, int32_t* kv_idx, void* stream) {
  Derived d;
  bsa_status s = check_geometry(g, &d);
  if (s != BSA_OK) return s;
  if (!sp) return fail(BSA_ERR_INVALID_ARGUMENT, "structure params are NULL");
  if (!head_class || !kv_cnt || !kv_idx)
    return fail(BSA_ERR_INVALID_ARGUMENT, "head_class, kv_cnt and kv_idx must not be NULL");
  if (!aligned16(head_class) || !aligned16(kv_cnt) || !aligned16(kv_idx) || (mask && !aligned16(mask)))
    return fail(BSA_ERR_INVALID_ARGUMENT, "device buffers must be 16-byte aligned");
  if (sp->window < 1) return fail(BSA_ERR_INVALID_ARGUMENT, "window %d must be >= 1", sp->window);
  if ((int64_t)g->latent_h * g->latent_w < 1 && g->frames > 0)
    return fail(BSA_ERR_INVALID_ARGUMENT, "latent_h * latent_w must be >= 1");
  if ((int64_t)g->B * g->H * d.nqb > 0x7fffffffLL)
    return fail(BSA_ERR_UNSUPPORTED, "too many query blocks for one launch");
  bsa::StructArgs a = {};
  a.classes = head_class;
  a.mask = mask;
  a.cnt = kv_cnt;
  a.idx = kv_idx;
  a.S = d.S;
  a.text_len = g->text_len;
  a.tpf = std::max<int64_t>(1, (int64_t)g->latent_h * g->latent_w);
  a.frames = g->frames;
  a.BH = g->B * g->H;
  a.nqb = d.nqb;
  a.nkb = d.nkb;
  a.q_block = g->q_block;
  a.k_block = g->k_block;
  a.window = sp->window;
  a.dummy_prev = sp->dummy_prev ? 1 : 0;
  a.block_causal = sp->block_causal ? 1 : 0;
  a.frame0_first = sp->frame0_dense ? d.f0_first : -1;
  a.frame0_last = sp->frame0_dense ? d.f0_last : -1;
  a.text_last = sp->text_columns ? d.text_last : -1;
  hipError_t e = bsa::launch_struct_lists(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BSA_ERR_HIP, "structured-list launch: %s", hipGetErrorString(e));
  return ok();
}

bsa_status bsa_forward(const void* q, const void* k, const void* v, int32_t dtype,
                       const bsa_geometry* g, const int32_t* kv_cnt, const int32_t* kv_idx,
                       const float* log_w, float softmax_scale, void* out, float* lse,
                       void* stream) {
  return bsa_forward_ex(q, k, v, dtype, g, kv_cnt, kv_idx, log_w, softmax_scale, out, lse, nullptr, stream);
}

}  // extern "C"

namespace {

// frame-0 query blocks of a derived geometry (the rows the forward runs first
// and may split)
int32_t dense_rows(const Derived& d) { return d.f0_first >= 0 ? d.f0_last - d.f0_first + 1 : 0; }

bsa_status forward_impl(const void* q, const void* k, const void* v, int32_t dtype, const bsa_geometry* g,
                        const int32_t* kv_cnt, const int32_t* kv_idx, const float* log_w, float softmax_scale,
                        void* out, float* lse, const bsa_forward_options* opt, int32_t split, void* workspace,
                        int64_t workspace_bytes, void* stream, bool static_ws = false) {
  const int32_t order = opt ? opt->launch_order : BSA_ORDER_FRAME_POSITION;
  if (order != BSA_ORDER_FRAME_POSITION && order != BSA_ORDER_FRAME_RUNS)
    return fail(BSA_ERR_INVALID_ARGUMENT, "unknown launch order %d", order);
  Derived d;
  bsa_status s = check_geometry(g, &d);
  if (s != BSA_OK) return s;
  if (dtype != BSA_DTYPE_BF16 && dtype != BSA_DTYPE_F32)
    return fail(BSA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (!q || !k || !v || !kv_cnt || !kv_idx || !out)
    return fail(BSA_ERR_INVALID_ARGUMENT, "q, k, v, kv_cnt, kv_idx and out must not be NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(kv_cnt) ||
      !aligned16(kv_idx) || (log_w && !aligned16(log_w)) || (lse && !aligned16(lse)))
    return fail(BSA_ERR_INVALID_ARGUMENT, "device buffers must be 16-byte aligned");
  if (!(std::isfinite(softmax_scale) && softmax_scale >= 0.0f))
    return fail(BSA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0");
  if (d.nkb > 8192) return fail(BSA_ERR_UNSUPPORTED, "nkb %d > 8192", d.nkb);
  if (g->seq_alloc * g->head_dim * (dtype == BSA_DTYPE_F32 ? 4 : 2) >= (1LL << 31))
    return fail(BSA_ERR_UNSUPPORTED, "one head of q/k/v exceeds 2 GiB");
  const int64_t units = (int64_t)g->B * g->H * d.nqb;
  if (units > 0x7fffffffLL) return fail(BSA_ERR_UNSUPPORTED, "too many query blocks for one launch");
  bsa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.cnt = kv_cnt;
  a.idx = kv_idx;
  a.logw = log_w;
  a.out = out;
  a.lse = lse;
  a.seq_alloc = g->seq_alloc;
  a.S = d.S;
  a.BH = g->B * g->H;
  a.nqb = d.nqb;
  a.nkb = d.nkb;
  a.q_block = g->q_block;
  a.k_block = g->k_block;
  const float scale = softmax_scale > 0.0f ? softmax_scale : (float)(1.0 / std::sqrt((double)g->head_dim));
  a.scale_log2 = scale * 1.4426950408889634f;
  a.dense_first = d.f0_first;
  a.dense_last = d.f0_last;
  const int64_t tpf = (int64_t)g->latent_h * g->latent_w;
  a.period = tpf > 0 ? (int32_t)std::max<int64_t>(1, (tpf + g->q_block / 2) / g->q_block) : 1;
  const int32_t nd = dense_rows(d);
  if (split < 1 || split > 16) return fail(BSA_ERR_INVALID_ARGUMENT, "dense_split %d must be in 1..16", split);
  if (nd == 0) split = 1;                        // no frame-0 rows: nothing to split
  if (split > 1 && static_ws) {
    // the library's own scratch: checked against its size, looked up last
    const int64_t need = bsa::split_ws_floats((int64_t)a.BH * nd * split, g->q_block, g->head_dim) * 4;
    if (need > bsa::kStaticScratchBytes)
      return fail(BSA_ERR_UNSUPPORTED, "the key split needs %lld bytes of scratch, more than the %lld the library "
                  "holds", (long long)need, (long long)bsa::kStaticScratchBytes);
    if ((int64_t)a.BH * nd * split > 0x7fffffffLL)
      return fail(BSA_ERR_UNSUPPORTED, "too many query blocks for one launch");
    float* ws = nullptr;
    const hipError_t e = bsa::static_scratch(&ws);
    if (e != hipSuccess) return fail(BSA_ERR_HIP, "device scratch lookup: %s", hipGetErrorString(e));
    workspace = ws;
    workspace_bytes = bsa::kStaticScratchBytes;
  }
  if (split > 1) {
    const int64_t need = bsa::split_ws_floats((int64_t)a.BH * nd * split, g->q_block, g->head_dim) * 4;
    if (!workspace || !aligned16(workspace))
      return fail(BSA_ERR_INVALID_ARGUMENT, "the key split needs a 16-byte aligned workspace");
    if (workspace_bytes < need)
      return fail(BSA_ERR_INVALID_ARGUMENT, "workspace of %lld bytes < %lld needed", (long long)workspace_bytes,
                  (long long)need);
  }
  if ((int64_t)a.BH * nd * split > 0x7fffffffLL)
    return fail(BSA_ERR_UNSUPPORTED, "too many query blocks for one launch");
  a.split = split;
  a.ws = split > 1 ? static_cast<float*>(workspace) : nullptr;
  a.n_dense = a.BH * nd * split;
  const int64_t n_other = (int64_t)a.BH * (d.nqb - nd);
  a.order = order;
  a.per_xcd = order == BSA_ORDER_FRAME_RUNS
                  ? (int32_t)((int64_t)a.BH * ((d.nqb - nd + bsa::kXcds - 1) / bsa::kXcds))
                  : (int32_t)((n_other + bsa::kXcds - 1) / bsa::kXcds);
  if (bsa::forward_grid(a) > 0x7fffffffLL) return fail(BSA_ERR_UNSUPPORTED, "too many query blocks for one launch");
  hipError_t e = bsa::launch_forward(a, dtype, g->head_dim, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BSA_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

bsa_status bsa_forward_ex(const void* q, const void* k, const void* v, int32_t dtype,
                          const bsa_geometry* g, const int32_t* kv_cnt, const int32_t* kv_idx,
                          const float* log_w, float softmax_scale, void* out, float* lse,
                          const bsa_forward_options* opt, void* stream) {
  return forward_impl(q, k, v, dtype, g, kv_cnt, kv_idx, log_w, softmax_scale, out, lse, opt, 1, nullptr, 0,
                      stream);
}

bsa_status bsa_forward_split_workspace_bytes(const bsa_geometry* g, int32_t dense_split, int64_t* bytes) {
  if (!bytes) return fail(BSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  Derived d;
  bsa_status s = check_geometry(g, &d);
  if (s != BSA_OK) return s;
  if (dense_split < 1 || dense_split > 16)
    return fail(BSA_ERR_INVALID_ARGUMENT, "dense_split %d must be in 1..16", dense_split);
  const int32_t nd = dense_rows(d);
  *bytes = (dense_split > 1 && nd > 0)
               ? bsa::split_ws_floats((int64_t)g->B * g->H * nd * dense_split, g->q_block, g->head_dim) * 4
               : 0;
  return ok();
}

bsa_status bsa_forward_split(const void* q, const void* k, const void* v, int32_t dtype,
                             const bsa_geometry* g, const int32_t* kv_cnt, const int32_t* kv_idx,
                             const float* log_w, float softmax_scale, void* out, float* lse,
                             const bsa_forward_options* opt, int32_t dense_split, void* workspace,
                             int64_t workspace_bytes, void* stream) {
  return forward_impl(q, k, v, dtype, g, kv_cnt, kv_idx, log_w, softmax_scale, out, lse, opt, dense_split,
                      workspace, workspace_bytes, stream);
}

static_assert(BSA_SPLIT_STATIC_MAX_BYTES == bsa::kStaticScratchBytes, "header and library scratch sizes differ");

bsa_status bsa_forward_split_static(const void* q, const void* k, const void* v, int32_t dtype,
                                    const bsa_geometry* g, const int32_t* kv_cnt, const int32_t* kv_idx,
                                    const float* log_w, float softmax_scale, void* out, float* lse,
                                    const bsa_forward_options* opt, int32_t dense_split, void* stream) {
  return forward_impl(q, k, v, dtype, g, kv_cnt, kv_idx, log_w, softmax_scale, out, lse, opt, dense_split, nullptr,
                      0, stream, true);
}

}  // extern "C"
