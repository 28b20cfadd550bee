// C-ABI entry points of libgrowpage: argument validation on the host, then kernel
// launches on the caller's stream.  Nothing here allocates or synchronises.
#include <math.h>

#include "gp_internal.h"

using namespace gp;

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

thread_local hipError_t g_last_hip_error = hipSuccess;

}  // namespace

void gp::note_hip_error(hipError_t e) { g_last_hip_error = e; }

namespace {

gp_status from_hip(hipError_t e) {
  if (e == hipSuccess) return GP_OK;
  g_last_hip_error = e;
  return GP_ERR_HIP;
}

gp_status check_params(const gp_params* p) {
  if (!p) return GP_ERR_INVALID;
  if (!(p->beta_s > 0.f && p->beta_s <= 1.f) || !(p->beta_l > 0.f && p->beta_l <= 1.f)) return GP_ERR_INVALID;
  if (!(p->top_p == p->top_p) || p->n_local < 0) return GP_ERR_INVALID;
  if (p->shrink != 0 && p->shrink != 1) return GP_ERR_INVALID;
  return GP_OK;
}

// Shapes and layout of the pools.  Returns GP_ERR_UNSUPPORTED for shapes the kernels
// do not implement and GP_ERR_INVALID for inconsistent or misaligned ones.
gp_status check_kv(const gp_kv* kv) {
  if (!kv || !kv->k || !kv->v) return GP_ERR_INVALID;
  if (kv->L <= 0 || kv->Hq <= 0 || kv->Hkv <= 0 || kv->d <= 0 || kv->P <= 0 || kv->num_pages <= 0)
    return GP_ERR_INVALID;
  if (kv->dtype != GP_F32 && kv->dtype != GP_BF16) return GP_ERR_INVALID;
  if (kv->stride_layer < 0 || kv->stride_page < 0 || kv->stride_head < 0 || kv->stride_tok < kv->d)
    return GP_ERR_INVALID;
  const int64_t esz = kv->dtype == GP_BF16 ? 2 : 4;
  if (!aligned(kv->k, 16) || !aligned(kv->v, 16)) return GP_ERR_INVALID;
  if ((kv->stride_layer * esz) % 16 || (kv->stride_page * esz) % 16 || (kv->stride_head * esz) % 16 ||
      (kv->stride_tok * esz) % 16)
    return GP_ERR_INVALID;
  if (kv->Hq % kv->Hkv != 0) return GP_ERR_UNSUPPORTED;
  const int32_t G = kv->Hq / kv->Hkv;
  if (G != 1 && G != 2 && G != kGroup) return GP_ERR_UNSUPPORTED;
  if (kv->d != 64 && kv->d != 128) return GP_ERR_UNSUPPORTED;
  if (kv->P % 8 != 0 || kv->P > 256) return GP_ERR_UNSUPPORTED;
  return GP_OK;
}

gp_status check_pages(const gp_pages* pg, bool need_pool) {
  if (!pg || !pg->page_table || !pg->n_alloc || !pg->fill) return GP_ERR_INVALID;
  if (pg->max_req <= 0 || pg->max_pages <= 0) return GP_ERR_INVALID;
  if (need_pool && (!pg->refcount || !pg->free_stack || !pg->free_top)) return GP_ERR_INVALID;
  return GP_OK;
}

Geo make_geo(const gp_kv* kv, const gp_pages* pg, const int32_t* req_ids, int32_t n_req) {
  Geo g;
  g.k = kv->k;
  g.v = kv->v;
  g.s_layer = kv->stride_layer;
  g.s_page = kv->stride_page;
  g.s_head = kv->stride_head;
  g.s_tok = kv->stride_tok;
  g.L = kv->L;
  g.Hq = kv->Hq;
  g.Hkv = kv->Hkv;
  g.G = kv->Hq / kv->Hkv;
  g.d = kv->d;
  g.P = kv->P;
  g.num_pages = kv->num_pages;
  g.dtype = kv->dtype;
  g.page_table = pg->page_table;
  g.max_pages = pg->max_pages;
  g.n_alloc = pg->n_alloc;
  g.fill = pg->fill;
  g.req_ids = req_ids;
  g.n_req = n_req;
  return g;
}

}  // namespace

extern "C" {

int32_t gp_abi_version(void) { return GP_ABI_VERSION; }

const char* gp_last_hip_error_string(void) { return hipGetErrorString(g_last_hip_error); }

const char* gp_status_string(int32_t status) {
  switch (status) {
    case GP_OK: return "GP_OK";
    case GP_ERR_INVALID: return "GP_ERR_INVALID: invalid argument";
    case GP_ERR_HIP: return "GP_ERR_HIP: HIP runtime or launch failure";
    case GP_ERR_SCRATCH: return "GP_ERR_SCRATCH: scratch buffer too small";
    case GP_ERR_UNSUPPORTED: return "GP_ERR_UNSUPPORTED: shape not implemented";
    default: return "unknown gp_status";
  }
}

gp_status gp_update_summaries(const void* q, int32_t q_dtype, int64_t q_stride_req,
                              int64_t q_stride_layer, int64_t q_stride_head,
                              const int32_t* req_ids, int32_t n_req, int32_t L, int32_t Hq,
                              int32_t d, float* sum_s, float* sum_l, const gp_params* params,
                              void* stream) {
  if (n_req < 0 || L <= 0 || Hq <= 0 || d <= 0 || d % 4) return GP_ERR_INVALID;
  if (gp_status s = check_params(params)) return s;
  if (n_req == 0) return GP_OK;
  if (!q || !req_ids || !sum_s || !sum_l) return GP_ERR_INVALID;
  if (q_dtype != GP_F32 && q_dtype != GP_BF16) return GP_ERR_INVALID;
  if (q_stride_req % 4 || q_stride_layer % 4 || q_stride_head % 4) return GP_ERR_INVALID;
  if (!aligned(q, q_dtype == GP_BF16 ? 8 : 16) || !aligned(sum_s, 16) || !aligned(sum_l, 16))
    return GP_ERR_INVALID;
  return from_hip(launch_ema(q, q_dtype, q_stride_req, q_stride_layer, q_stride_head, req_ids, n_req,
                             L, Hq, d, sum_s, sum_l, params->beta_s, params->beta_l,
                             (hipStream_t)stream));
}

size_t gp_scratch_bytes(const gp_kv* kv, int32_t n_req, int64_t max_total_tokens) {
  if (!kv || n_req < 0 || max_total_tokens < 0 || kv->L <= 0 || kv->Hkv <= 0 || kv->Hq <= 0 || kv->P <= 0)
    return 0;
  return scratch_layout(*kv, n_req, max_total_tokens).total;
}

gp_status gp_boundary_scan(const gp_kv* kv, const gp_pages* pages, const int32_t* req_ids,
                           int32_t n_req, const float* sum_s, const float* sum_l,
                           const float* rope_cos, const float* rope_sin, int32_t rope_max_pos,
                           const int32_t* pos, const gp_params* params, int32_t* ws_out,
                           float* stats_out, void* scratch, size_t scratch_bytes,
                           int64_t max_total_tokens, void* stream) {
  if (gp_status s = check_kv(kv)) return s;
  if (gp_status s = check_pages(pages, false)) return s;
  if (gp_status s = check_params(params)) return s;
  if (n_req < 0 || n_req > pages->max_req || max_total_tokens < 0) return GP_ERR_INVALID;
  if (n_req == 0) return GP_OK;
  if (!req_ids || !sum_s || !sum_l || !ws_out || !scratch) return GP_ERR_INVALID;
  if ((rope_cos == nullptr) != (rope_sin == nullptr)) return GP_ERR_INVALID;
  if (rope_cos && (!pos || rope_max_pos <= 0)) return GP_ERR_INVALID;
  if ((int64_t)pages->max_pages * kv->P > kMaxSlots) return GP_ERR_UNSUPPORTED;
  if (!aligned(scratch, 256)) return GP_ERR_INVALID;
  const ScratchLayout lay = scratch_layout(*kv, n_req, max_total_tokens);
  if (scratch_bytes < lay.total) return GP_ERR_SCRATCH;
  const Geo g = make_geo(kv, pages, req_ids, n_req);
  return from_hip(launch_scan(g, scratch_ptrs(scratch, lay), max_total_tokens, sum_s, sum_l, rope_cos,
                              rope_sin, rope_max_pos, pos, params->top_p, params->n_local,
                              params->shrink, ws_out, stats_out, (hipStream_t)stream));
}

gp_status gp_scan_logits(const gp_kv* kv, int32_t n_req, int64_t max_total_tokens, const void* scratch,
                         size_t scratch_bytes, int32_t entry, int32_t n, float* logits_out, void* stream) {
  if (!kv || kv->L <= 0 || kv->Hkv <= 0 || kv->Hq <= 0 || kv->P <= 0) return GP_ERR_INVALID;
  if (n_req <= 0 || entry < 0 || entry >= n_req || n < 0 || max_total_tokens < 0) return GP_ERR_INVALID;
  if (!scratch || !aligned(scratch, 256)) return GP_ERR_INVALID;
  if (n == 0) return GP_OK;
  if (!logits_out) return GP_ERR_INVALID;
  const ScratchLayout lay = scratch_layout(*kv, n_req, max_total_tokens);
  if (scratch_bytes < lay.total) return GP_ERR_SCRATCH;
  Geo g{};
  g.L = kv->L;
  g.Hkv = kv->Hkv;
  return from_hip(launch_copy_logits(g, scratch_ptrs(const_cast<void*>(scratch), lay), entry, n, logits_out,
                                     (hipStream_t)stream));
}

gp_status gp_decide(const int32_t* ws, const int32_t* req_ids, int32_t n_req, int32_t L,
                    int32_t Hq, int32_t P, const gp_params* params, const gp_pages* pages,
                    uint8_t* decision_out, int32_t* delta_out, int32_t* status_out,
                    int32_t* counters_out, void* stream) {
  if (gp_status s = check_pages(pages, true)) return s;
  if (gp_status s = check_params(params)) return s;
  if (params->shrink) return GP_ERR_INVALID;  // GrowPage's own rule never shrinks
  if (n_req < 0 || n_req > pages->max_req || L <= 0 || Hq <= 0 || P <= 0) return GP_ERR_INVALID;
  if (n_req == 0) return GP_OK;
  if (!ws || !req_ids || !decision_out || !delta_out || !status_out) return GP_ERR_INVALID;
  return from_hip(launch_decide(ws, req_ids, n_req, L, Hq, params->tau, *pages, P, GP_POLICY_GROWPAGE,
                                nullptr, 0.f, decision_out, delta_out, status_out, counters_out,
                                (hipStream_t)stream));
}

gp_status gp_decide_policy(const int32_t* ws, const int32_t* req_ids, int32_t n_req, int32_t L,
                           int32_t Hq, int32_t P, const gp_params* params, int32_t policy,
                           const float* rand_u, float grow_prob, const gp_pages* pages,
                           uint8_t* decision_out, int32_t* delta_out, int32_t* status_out,
                           int32_t* counters_out, void* stream) {
  if (gp_status s = check_pages(pages, true)) return s;
  if (gp_status s = check_params(params)) return s;
  if (policy < GP_POLICY_GROWPAGE || policy > GP_POLICY_SHRINK) return GP_ERR_INVALID;
  // the scan sized the keep-sets for the policy: (A-1)*P slots exactly under SHRINK
  if ((policy == GP_POLICY_SHRINK) != (params->shrink == 1)) return GP_ERR_INVALID;
  if (n_req < 0 || n_req > pages->max_req || L <= 0 || Hq <= 0 || P <= 0) return GP_ERR_INVALID;
  if (n_req == 0) return GP_OK;
  if (!ws || !req_ids || !decision_out || !delta_out || !status_out) return GP_ERR_INVALID;
  if (policy == GP_POLICY_RANDOM && !rand_u) return GP_ERR_INVALID;
  return from_hip(launch_decide(ws, req_ids, n_req, L, Hq, params->tau, *pages, P, policy, rand_u,
                                grow_prob, decision_out, delta_out, status_out, counters_out,
                                (hipStream_t)stream));
}

namespace {
gp_status compact_checks(const gp_kv* kv, const gp_pages* pages, int32_t n_req,
                         const gp_params* params, int64_t max_total_tokens) {
  if (gp_status s = check_kv(kv)) return s;
  if (gp_status s = check_pages(pages, true)) return s;
  if (params)
    if (gp_status s = check_params(params)) return s;
  if (n_req < 0 || n_req > pages->max_req || max_total_tokens < 0) return GP_ERR_INVALID;
  return GP_OK;
}
}  // namespace

gp_status gp_compact_prepare(const gp_kv* kv, const gp_pages* pages, const int32_t* req_ids,
                             const uint8_t* decision, int32_t n_req, const gp_params* params,
                             int32_t* evicted_out, int32_t* status_out, void* scratch,
                             size_t scratch_bytes, int64_t max_total_tokens, void* stream) {
  if (!params) return GP_ERR_INVALID;
  if (gp_status s = compact_checks(kv, pages, n_req, params, max_total_tokens)) return s;
  if (n_req == 0) return GP_OK;
  if (!req_ids || !decision || !status_out || !scratch) return GP_ERR_INVALID;
  if (!aligned(scratch, 256)) return GP_ERR_INVALID;
  const ScratchLayout lay = scratch_layout(*kv, n_req, max_total_tokens);
  if (scratch_bytes < lay.total) return GP_ERR_SCRATCH;
  const Geo g = make_geo(kv, pages, req_ids, n_req);
  return from_hip(launch_compact_prepare(g, *pages, scratch_ptrs(scratch, lay), decision,
                                         evicted_out, params->shrink ? 2 * kv->P : kv->P, status_out,
                                         (hipStream_t)stream));
}

gp_status gp_compact_move(const gp_kv* kv, const gp_pages* pages, const int32_t* req_ids,
                          int32_t n_req, int32_t* counters_out, void* scratch,
                          size_t scratch_bytes, int64_t max_total_tokens, void* stream) {
  if (gp_status s = compact_checks(kv, pages, n_req, nullptr, max_total_tokens)) return s;
  if (n_req == 0) return GP_OK;
  if (!req_ids || !scratch) return GP_ERR_INVALID;
  if (!aligned(scratch, 256)) return GP_ERR_INVALID;
  const ScratchLayout lay = scratch_layout(*kv, n_req, max_total_tokens);
  if (scratch_bytes < lay.total) return GP_ERR_SCRATCH;
  const Geo g = make_geo(kv, pages, req_ids, n_req);
  return from_hip(launch_compact_move(g, *pages, scratch_ptrs(scratch, lay), counters_out,
                                      (hipStream_t)stream));
}

gp_status gp_compact(const gp_kv* kv, const gp_pages* pages, const int32_t* req_ids,
                     const uint8_t* decision, int32_t n_req, const gp_params* params,
                     int32_t* evicted_out, int32_t* status_out, int32_t* counters_out,
                     void* scratch, size_t scratch_bytes, int64_t max_total_tokens,
                     void* stream) {
  if (gp_status s = gp_compact_prepare(kv, pages, req_ids, decision, n_req, params, evicted_out,
                                       status_out, scratch, scratch_bytes, max_total_tokens, stream))
    return s;
  return gp_compact_move(kv, pages, req_ids, n_req, counters_out, scratch, scratch_bytes,
                         max_total_tokens, stream);
}

gp_status gp_append_kv(const gp_kv* kv, const gp_pages* pages, const void* k_new,
                       const void* v_new, const int32_t* req_ids, int32_t n_req,
                       int32_t* status_out, void* stream) {
  if (gp_status s = check_kv(kv)) return s;
  if (gp_status s = check_pages(pages, false)) return s;
  if (n_req < 0 || n_req > pages->max_req) return GP_ERR_INVALID;
  if (n_req == 0) return GP_OK;
  if (!k_new || !v_new || !req_ids) return GP_ERR_INVALID;
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return GP_ERR_INVALID;
  const Geo g = make_geo(kv, pages, req_ids, n_req);
  return from_hip(launch_append(g, *pages, k_new, v_new, status_out, (hipStream_t)stream));
}

gp_status gp_decode_attention(const gp_kv* kv, const gp_pages* pages, const void* q, int32_t q_dtype,
                              int64_t q_stride_req, int64_t q_stride_layer, int64_t q_stride_head,
                              const int32_t* req_ids, int32_t n_req, const float* rope_cos,
                              const float* rope_sin, int32_t rope_max_pos, const int32_t* pos,
                              float* out, void* stream) {
  if (gp_status s = check_kv(kv)) return s;
  if (gp_status s = check_pages(pages, false)) return s;
  if (n_req < 0 || n_req > pages->max_req) return GP_ERR_INVALID;
  if (n_req == 0) return GP_OK;
  if (!q || !req_ids || !out) return GP_ERR_INVALID;
  if (q_dtype != GP_F32 && q_dtype != GP_BF16) return GP_ERR_INVALID;
  if ((rope_cos == nullptr) != (rope_sin == nullptr)) return GP_ERR_INVALID;
  if (rope_cos && (!pos || rope_max_pos <= 0)) return GP_ERR_INVALID;
  const Geo g = make_geo(kv, pages, req_ids, n_req);
  return from_hip(launch_decode_attention(g, q, q_dtype, q_stride_req, q_stride_layer, q_stride_head,
                                          rope_cos, rope_sin, rope_max_pos, pos, out,
                                          (hipStream_t)stream));
}

}  // extern "C"
