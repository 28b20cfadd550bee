// gp_boundary_step_static: one whole boundary batch (scan, decide, compaction) whose
// scratch is a buffer the library holds on each device, for callers that cannot allocate
// device memory.  The kernels are those of gp_boundary_scan, gp_decide_policy and
// gp_compact, given the buffer's device address as they are given the caller's scratch.
#include <mutex>

#include "gp_internal.h"

namespace gp {
namespace {

// The buffer itself: one copy per device, alive until the process ends.  In host code
// this name is a stand-in for the symbol, not a device address: the device address comes
// from hipGetSymbolAddress on that device (scratch_ptr below) and nothing else is used.
static __device__ __align__(256) unsigned char scratch[GP_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// Device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept.
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev]() {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace gp

using namespace gp;

extern "C" {

gp_status gp_boundary_step_static(const gp_kv* kv, const gp_pages* pages, const int32_t* req_ids,
                                  int32_t n_req, const float* sum_s, const float* sum_l,
                                  const float* rope_cos, const float* rope_sin, int32_t rope_max_pos,
                                  const int32_t* pos, const gp_params* params, int64_t max_total_tokens,
                                  int32_t* ws_out, float* stats_out, uint8_t* decision_out,
                                  int32_t* delta_out, int32_t* status_out, int32_t* evicted_out,
                                  int32_t* counters_out, void* stream) {
  if (!kv || !pages || !params || n_req < 0 || max_total_tokens < 0) return GP_ERR_INVALID;
  if (n_req == 0) return GP_OK;
  if (!decision_out || !delta_out || !status_out) return GP_ERR_INVALID;
  if (kv->L <= 0 || kv->Hkv <= 0 || kv->Hq <= 0 || kv->P <= 0) return GP_ERR_INVALID;
  // the batch must fit the library's buffer: checked before anything is launched
  const size_t need = gp_scratch_bytes(kv, n_req, max_total_tokens);
  if (need == 0 || need > (size_t)GP_STATIC_SCRATCH_BYTES) return GP_ERR_SCRATCH;
  void* buf = nullptr;
  hipError_t e = scratch_ptr(&buf);
  if (e != hipSuccess) {
    note_hip_error(e);
    return GP_ERR_HIP;
  }
  // The existing entry points, in order, with the buffer's device address as scratch; each
  // validates its own arguments before launching anything (the first one that fails
  // returns, and nothing after it runs).
  gp_status s = gp_boundary_scan(kv, pages, req_ids, n_req, sum_s, sum_l, rope_cos, rope_sin, rope_max_pos,
                                 pos, params, ws_out, stats_out, buf, need, max_total_tokens, stream);
  if (s != GP_OK) return s;
  s = gp_decide_policy(ws_out, req_ids, n_req, kv->L, kv->Hq, kv->P, params,
                       params->shrink ? GP_POLICY_SHRINK : GP_POLICY_GROWPAGE, nullptr, 0.f, pages,
                       decision_out, delta_out, status_out, counters_out, stream);
  if (s != GP_OK) return s;
  return gp_compact(kv, pages, req_ids, decision_out, n_req, params, evicted_out, status_out, counters_out,
                    buf, need, max_total_tokens, stream);
}

}  // extern "C"
