// C ABI of libspa.so: argument validation, workspace carving and kernel launches.
// Every check runs on the host before any HIP call, so invalid arguments never reach a
// kernel.
#include <cmath>
#include <climits>

#include "spa.h"
#include "spa_internal.h"

namespace {

using spa::Geometry;

constexpr int kMaxKeyBlocks = 2048;  // kMaxBlocks of the kernels

int check_dims(const spa_dims* d, Geometry* g) {
  if (!d) return SPA_E_NULL;
  if (d->B < 1 || d->H < 1 || d->N < 1) return SPA_E_SHAPE;
  if (d->d != 64 && d->d != 128) return SPA_E_UNSUPPORTED;
  if (d->blk_q != 64 && d->blk_q != 128) return SPA_E_UNSUPPORTED;
  if (d->blk_k != 64) return SPA_E_UNSUPPORTED;
  const long long total = (long long)d->B * d->H * d->N * d->d;
  if (total >= (1LL << 31) || (long long)d->B * d->H > 65535) return SPA_E_SHAPE;
  g->B = d->B;
  g->H = d->H;
  g->N = d->N;
  g->d = d->d;
  g->blk_q = d->blk_q;
  g->blk_k = d->blk_k;
  g->nqb = (d->N + d->blk_q - 1) / d->blk_q;
  g->nkb = (d->N + d->blk_k - 1) / d->blk_k;
  if (g->nkb > kMaxKeyBlocks) return SPA_E_UNSUPPORTED;
  return SPA_OK;
}

bool bad_frac(double x) { return !(x >= 0.0 && x <= 1.0); }  // also rejects NaN

float resolve_scale(double scale, int d) {
  return scale > 0.0 ? (float)scale : (float)(1.0 / std::sqrt((double)d));
}

int launch_status(hipError_t e) { return e == hipSuccess ? SPA_OK : SPA_E_LAUNCH; }

}  // namespace

extern "C" {

size_t spa_mask_workspace_bytes(const spa_dims* dims) {
  Geometry g;
  if (check_dims(dims, &g) != SPA_OK) return 0;
  return spa::mask_workspace_bytes(g);
}

int spa_build_mask(const spa_dims* dims, const void* q, const void* k, double k_frac, double p,
                   double pooled_scale, int32_t* kv_idx, int32_t* kv_cnt, int32_t* rule_len,
                   void* ws, size_t ws_bytes, void* stream) {
  return spa_build_mask_stages(dims, q, k, k_frac, p, pooled_scale, kv_idx, kv_cnt, rule_len, ws,
                               ws_bytes, SPA_MASK_ALL, stream);
}

int spa_build_mask_stages(const spa_dims* dims, const void* q, const void* k, double k_frac,
                          double p, double pooled_scale, int32_t* kv_idx, int32_t* kv_cnt,
                          int32_t* rule_len, void* ws, size_t ws_bytes, unsigned stages,
                          void* stream) {
  Geometry g;
  int rc = check_dims(dims, &g);
  if (rc != SPA_OK) return rc;
  if (!q || !k || !kv_idx || !kv_cnt || !ws) return SPA_E_NULL;
  if (bad_frac(k_frac) || bad_frac(p) || std::isnan(pooled_scale) || std::isinf(pooled_scale))
    return SPA_E_PARAM;
  if (ws_bytes < spa::mask_workspace_bytes(g)) return SPA_E_WORKSPACE;
  if (stages == 0u || (stages & ~(unsigned)SPA_MASK_ALL)) return SPA_E_PARAM;
  spa::MaskArgs a;
  a.g = g;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.pooled_scale = pooled_scale > 0.0 ? pooled_scale : 1.0 / std::sqrt((double)g.d);
  // Top-k length: ceil(k * Nkb) with a 1e-9 guard for decimal fractions, clamped to [1, Nkb]
  double lk = std::ceil(k_frac * (double)g.nkb - 1e-9);
  if (lk < 1.0) lk = 1.0;
  if (lk > (double)g.nkb) lk = (double)g.nkb;
  a.lk = (int)lk;
  a.p_all = p >= 1.0 ? 1 : 0;
  a.wp = a.p_all ? 0 : (uint64_t)std::llrint(p * 0x1p62);
  a.kv_idx = kv_idx;
  a.kv_cnt = kv_cnt;
  a.rule_len = rule_len;
  spa::mask_workspace_carve(g, ws, &a.qbar, &a.kbar_t);
  return launch_status(spa::launch_mask(a, stages, static_cast<hipStream_t>(stream)));
}

int spa_build_mask_noalloc(const spa_dims* dims, const void* q, const void* k, double k_frac,
                           double p, double pooled_scale, int32_t* kv_idx, int32_t* kv_cnt,
                           int32_t* rule_len, void* stream) {
  static_assert(spa::kNoallocScratchBytes == (size_t)SPA_NOALLOC_SCRATCH_BYTES,
                "header and library agree on the scratch size");
  Geometry g;
  int rc = check_dims(dims, &g);
  if (rc != SPA_OK) return rc;
  if (!q || !k || !kv_idx || !kv_cnt) return SPA_E_NULL;
  if (bad_frac(k_frac) || bad_frac(p) || std::isnan(pooled_scale) || std::isinf(pooled_scale))
    return SPA_E_PARAM;
  const size_t need = spa::mask_workspace_bytes(g);
  if (need > spa::kNoallocScratchBytes) return SPA_E_SCRATCH;
  void* ws = nullptr;
  if (spa::noalloc_scratch(static_cast<hipStream_t>(stream), &ws) != hipSuccess)
    return SPA_E_SCRATCH;
  return spa_build_mask_stages(dims, q, k, k_frac, p, pooled_scale, kv_idx, kv_cnt, rule_len, ws,
                               need, SPA_MASK_ALL, stream);
}

size_t spa_fwd_workspace_bytes(const spa_dims* dims) {
  Geometry g;
  if (check_dims(dims, &g) != SPA_OK) return 0;
  return spa::fwd_workspace_bytes(g);
}

int spa_sparse_attn_fwd(const spa_dims* dims, const void* q, const void* k, const void* v,
                        const int32_t* kv_idx, const int32_t* kv_cnt, double scale, void* o,
                        void* o_lo, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return spa_sparse_attn_fwd_stages(dims, q, k, v, kv_idx, kv_cnt, scale, o, o_lo, lse, ws,
                                    ws_bytes, SPA_FWD_ALL, stream);
}

int spa_sparse_attn_fwd_stages(const spa_dims* dims, const void* q, const void* k,
                               const void* v, const int32_t* kv_idx, const int32_t* kv_cnt,
                               double scale, void* o, void* o_lo, float* lse, void* ws,
                               size_t ws_bytes, unsigned stages, void* stream) {
  Geometry g;
  int rc = check_dims(dims, &g);
  if (rc != SPA_OK) return rc;
  if (stages == 0u || (stages & ~(unsigned)SPA_FWD_ALL)) return SPA_E_PARAM;
  if (!q || !k || !v || !kv_idx || !kv_cnt || !o || !lse) return SPA_E_NULL;
  if (o_lo && !ws) return SPA_E_NULL;
  if (std::isnan(scale) || std::isinf(scale)) return SPA_E_PARAM;
  if (o_lo && ws_bytes < spa::fwd_workspace_bytes(g)) return SPA_E_WORKSPACE;
  spa::FwdArgs a;
  a.v16 = nullptr;
  a.vflag = nullptr;
  if (o_lo) spa::fwd_workspace_carve(g, ws, &a);
  a.g = g;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.kv_idx = kv_idx;
  a.kv_cnt = kv_cnt;
  a.scale = resolve_scale(scale, g.d);
  a.o = static_cast<uint16_t*>(o);
  a.o_lo = static_cast<uint16_t*>(o_lo);
  a.lse = lse;
  return launch_status(spa::launch_fwd(a, stages, static_cast<hipStream_t>(stream)));
}

size_t spa_bwd_workspace_bytes(const spa_dims* dims) {
  Geometry g;
  if (check_dims(dims, &g) != SPA_OK) return 0;
  return spa::bwd_workspace_bytes(g);
}

int spa_sparse_attn_bwd(const spa_dims* dims, const void* q, const void* k, const void* v,
                        const void* o, const void* o_lo, const void* dout, const float* lse,
                        const int32_t* kv_idx, const int32_t* kv_cnt, double scale, void* dq,
                        void* dk, void* dv, int grad_dtype, void* ws, size_t ws_bytes,
                        void* stream) {
  return spa_sparse_attn_bwd_stages(dims, q, k, v, o, o_lo, dout, lse, kv_idx, kv_cnt, scale, dq,
                                    dk, dv, grad_dtype, ws, ws_bytes, SPA_BWD_ALL, stream);
}

int spa_sparse_attn_bwd_stages(const spa_dims* dims, const void* q, const void* k, const void* v,
                               const void* o, const void* o_lo, const void* dout,
                               const float* lse, const int32_t* kv_idx, const int32_t* kv_cnt,
                               double scale, void* dq, void* dk, void* dv, int grad_dtype,
                               void* ws, size_t ws_bytes, unsigned stages, void* stream) {
  Geometry g;
  int rc = check_dims(dims, &g);
  if (rc != SPA_OK) return rc;
  if (!q || !k || !v || !o || !dout || !lse || !kv_idx || !kv_cnt || !dq || !dk || !dv || !ws)
    return SPA_E_NULL;
  if (std::isnan(scale) || std::isinf(scale) || (grad_dtype != 0 && grad_dtype != 1))
    return SPA_E_PARAM;
  if (ws_bytes < spa::bwd_workspace_bytes(g)) return SPA_E_WORKSPACE;
  if (stages == 0u || (stages & ~(unsigned)SPA_BWD_ALL)) return SPA_E_PARAM;
  spa::BwdArgs a;
  a.g = g;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.o_lo = static_cast<const uint16_t*>(o_lo);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.kv_idx = kv_idx;
  a.kv_cnt = kv_cnt;
  a.scale = resolve_scale(scale, g.d);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.grad_bf16 = grad_dtype;
  spa::bwd_workspace_carve(g, ws, &a);
  return launch_status(spa::launch_bwd(a, stages, static_cast<hipStream_t>(stream)));
}

const char* spa_status_string(int status) {
  switch (status) {
    case SPA_OK: return "ok";
    case SPA_E_NULL: return "a required pointer is NULL";
    case SPA_E_SHAPE: return "invalid shape (B, H, N must be >= 1 and the tensor < 2^31 elements)";
    case SPA_E_PARAM: return "invalid parameter (k_frac and p in [0, 1]; finite scales; grad_dtype 0 or 1; known stage bits)";
    case SPA_E_UNSUPPORTED: return "unsupported configuration (d in {64,128}, blk_q in {64,128}, blk_k 64, Nkb <= 2048)";
    case SPA_E_WORKSPACE: return "workspace too small";
    case SPA_E_LAUNCH: return "kernel launch failed";
    case SPA_E_SCRATCH: return "the fixed device scratch is too small for this problem or not available on the stream's device";
    default: return "unknown status";
  }
}

int spa_version(void) { return 100; }

}  // extern "C"
