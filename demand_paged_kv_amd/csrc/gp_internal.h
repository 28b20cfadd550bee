// Internal declarations of libgrowpage: scratch layout, argument blocks and the
// launchers each kernel file provides.  Device code targets gfx950 (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "growpage.h"

namespace gp {

constexpr int kDists = 8;          // score rows per unit: 4 query-head slots x 2 summaries
constexpr int kGroup = 4;          // query-head slots per unit (the largest group supported)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int64_t kMaxSlots = 1 << 24;  // candidate slots per request (max_pages * P) the scan indexes
constexpr int kReqFields = 8;      // per-request int32 fields of the compaction plan
constexpr int kLogitAlign = 16;    // each unit's logit rows start on a 512-byte boundary

// Token rows a unit of n candidate slots takes in the logit scratch: n rounded up to a
// multiple of kLogitAlign, so that every 16-token store covers whole cache lines.
__host__ __device__ inline int64_t logit_rows(int64_t n) { return (n + kLogitAlign - 1) / kLogitAlign * kLogitAlign; }

// Query head (within its KV head's group of G = Hq / Hkv in {1, 2, 4}) that score row k of a
// unit scores: rows 2j, 2j+1 belong to head j; with G < 4 the rows of the missing heads
// repeat the last head's (equal logits: no change to any working set or to the max-of-rows
// importance), and only rows of real heads (row_real) are written out.
__host__ __device__ inline int row_head(int k, int G) { return min(k >> 1, G - 1); }
__host__ __device__ inline bool row_real(int k, int G) { return (k >> 1) < G; }

// Evicted slots per unit: at the boundary n = (A+1)P, so a compaction evicts P slots,
// or 2P when it shrinks the allocation by a page.
__host__ __device__ inline int ev_stride(int P) { return 2 * P; }

// Slots a compaction of a request with A allocation pages keeps.
__host__ __device__ inline int kept_slots(int A, int P, bool shrink) { return (shrink && A >= 2 ? A - 1 : A) * P; }

// ----------------------------------------------------------------------------- scratch
// One caller buffer, carved into 256-byte aligned regions.  The scan fills the
// request plan, logits and statistics; the compaction reads them.
struct ScratchLayout {
  size_t tok_off;   // int64 [n_req]  first logit row of each entry (multiple of 16)
  size_t n_tok;     // int32 [n_req]  candidate slots n (0 when over budget)
  size_t order;     // int32 [n_req]  entries by n descending (ties by index)
  size_t flags;     // int32 [n_req]  GP_REQ_OVERFLOW when over budget
  size_t stats;     // float [n_req][L][Hq][2][2]  max logit, sum exp
  size_t logits;    // float [rows][L][Hkv][8] (per unit: [logit_rows(n)][8], token-major)
  size_t ev;        // int32 [n_req][L][Hkv][2P] slots a compaction evicts, ascending
  size_t e_unit;    // int32 [n_req][L][Hkv]     first of them (n if none)
  size_t req;       // int32 [n_req][kReqFields]  first changed slot, copy-on-write plan
  size_t cow;       // int32 [cow_cap][2]  (old page, new page)
  size_t misc;      // int32 [16]  ncow, ...
  size_t bitmap;    // uint32 [num_pages/32 + 1]
  size_t total;
  int64_t cow_cap;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline ScratchLayout scratch_layout(const gp_kv& kv, int32_t n_req, int64_t max_tokens) {
  ScratchLayout s{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t nr = (size_t)(n_req > 0 ? n_req : 1);
  const size_t units = nr * kv.L * kv.Hkv;
  const size_t tok = (size_t)(max_tokens > 0 ? max_tokens : 1);
  s.tok_off = take(nr * sizeof(int64_t));
  s.n_tok = take(nr * sizeof(int32_t));
  s.order = take(nr * sizeof(int32_t));
  s.flags = take(nr * sizeof(int32_t));
  s.stats = take(nr * kv.L * kv.Hq * 4 * sizeof(float));
  // Padding adds fewer than kLogitAlign rows per entry.
  s.logits = take((tok + nr * (kLogitAlign - 1)) * kv.L * kv.Hkv * kDists * sizeof(float));
  s.ev = take(units * ev_stride(kv.P) * sizeof(int32_t));
  s.e_unit = take(units * sizeof(int32_t));
  s.req = take(nr * kReqFields * sizeof(int32_t));
  s.cow_cap = (int64_t)(tok / (kv.P > 0 ? kv.P : 1) + nr);
  s.cow = take((size_t)s.cow_cap * 2 * sizeof(int32_t));
  s.misc = take(16 * sizeof(int32_t));
  s.bitmap = take(((size_t)kv.num_pages / 32 + 1) * sizeof(uint32_t));
  s.total = off;
  return s;
}

// Pointers into the scratch buffer, passed to kernels by value.
struct ScratchPtrs {
  int64_t* tok_off;
  int32_t* n_tok;
  int32_t* order;
  int32_t* flags;
  float* stats;
  float* logits;
  int32_t* ev;
  int32_t* e_unit;
  int32_t* req;
  int32_t* cow;
  int32_t* misc;
  uint32_t* bitmap;
  int64_t cow_cap;
};

inline ScratchPtrs scratch_ptrs(void* base, const ScratchLayout& s) {
  char* b = (char*)base;
  ScratchPtrs p;
  p.tok_off = (int64_t*)(b + s.tok_off);
  p.n_tok = (int32_t*)(b + s.n_tok);
  p.order = (int32_t*)(b + s.order);
  p.flags = (int32_t*)(b + s.flags);
  p.stats = (float*)(b + s.stats);
  p.logits = (float*)(b + s.logits);
  p.ev = (int32_t*)(b + s.ev);
  p.e_unit = (int32_t*)(b + s.e_unit);
  p.req = (int32_t*)(b + s.req);
  p.cow = (int32_t*)(b + s.cow);
  p.misc = (int32_t*)(b + s.misc);
  p.bitmap = (uint32_t*)(b + s.bitmap);
  p.cow_cap = s.cow_cap;
  return p;
}

// Geometry shared by the scan, selection and compaction kernels.
struct Geo {
  const void* k;
  const void* v;
  int64_t s_layer, s_page, s_head, s_tok;
  int32_t L, Hq, Hkv, d, P, num_pages;
  int32_t G;          // query heads per KV head: 1, 2 or 4
  int32_t dtype;
  const int32_t* page_table;
  int32_t max_pages;
  const int32_t* n_alloc;
  const int32_t* fill;
  const int32_t* req_ids;
  int32_t n_req;
};

// The HIP error gp_last_hip_error_string() reports (kept per host thread).
void note_hip_error(hipError_t e);

// ----------------------------------------------------------------------------- launchers
hipError_t launch_ema(const void* q, int32_t q_dtype, int64_t sr, int64_t sl, int64_t sh,
                      const int32_t* req_ids, int32_t n_req, int32_t L, int32_t Hq, int32_t d,
                      float* sum_s, float* sum_l, float beta_s, float beta_l, hipStream_t st);

hipError_t launch_scan(const Geo& g, const ScratchPtrs& sp, int64_t max_tokens,
                       const float* sum_s, const float* sum_l, const float* rope_cos,
                       const float* rope_sin, int32_t rope_max_pos, const int32_t* pos,
                       float top_p, int32_t n_local, int32_t shrink, int32_t* ws_out,
                       float* stats_out, hipStream_t st);

hipError_t launch_copy_logits(const Geo& g, const ScratchPtrs& sp, int32_t entry, int32_t n, float* out,
                              hipStream_t st);

struct FinishArgs {
  Geo g;
  ScratchPtrs sp;
  float top_p;
  int32_t n_local;
  int32_t shrink;   // keep-sets of kept_slots(A, P, shrink) slots
  int32_t* ws_out;
  float* stats_out;
};
hipError_t launch_finish(const FinishArgs& a, hipStream_t st);

// Arguments of the scan's logit kernels.
struct ScanArgs {
  Geo g;
  ScratchPtrs sp;
  int64_t max_tokens;
  const float* sum_s;
  const float* sum_l;
  const float* rope_cos;
  const float* rope_sin;
  int32_t rope_max_pos;
  const int32_t* pos;
  float scale;
  int32_t* ws_out;
};
// bf16 keys in pages of a multiple of 16 tokens: logits and working sets in one kernel.
constexpr int kFusedPageMultiple = 16;
hipError_t launch_fused_scan(const ScanArgs& s, const FinishArgs& f, hipStream_t st);
// The same for batches of at most kSplitUnits units: each unit's steps in `parts` blocks,
// then finish_kernel.
constexpr int64_t kSplitUnits = 512;
hipError_t launch_split_scan(const ScanArgs& s, const FinishArgs& f, int parts, hipStream_t st);

hipError_t launch_decide(const int32_t* ws, const int32_t* req_ids, int32_t n_req, int32_t L,
                         int32_t Hq, int32_t tau, const gp_pages& pg, int32_t P, int32_t policy,
                         const float* rand_u, float grow_prob, uint8_t* decision, int32_t* delta,
                         int32_t* status, int32_t* counters, hipStream_t st);

hipError_t launch_compact_prepare(const Geo& g, const gp_pages& pg, const ScratchPtrs& sp,
                                  const uint8_t* decision, int32_t* evicted_out,
                                  int32_t evicted_stride, int32_t* status_out, hipStream_t st);
hipError_t launch_compact_move(const Geo& g, const gp_pages& pg, const ScratchPtrs& sp,
                               int32_t* counters_out, hipStream_t st);

hipError_t launch_append(const Geo& g, const gp_pages& pg, const void* k_new, const void* v_new,
                         int32_t* status_out, hipStream_t st);

hipError_t launch_decode_attention(const Geo& g, const void* q, int32_t q_dtype, int64_t sr, int64_t sl,
                                   int64_t sh, const float* rope_cos, const float* rope_sin,
                                   int32_t rope_max_pos, const int32_t* pos, float* out,
                                   hipStream_t st);

}  // namespace gp
