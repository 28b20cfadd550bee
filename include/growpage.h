/*
 * growpage.h -- C ABI of libgrowpage, the GrowPage capacity-boundary engine for
 * AMD Instinct MI355X (CDNA4, gfx950).
 *
 * What the engine computes (GrowPage review on evolve.pub, section "Summary", and the
 * paper's abstract): every request keeps two moving averages of its queries per query
 * head, one fast and one slow, taken before RoPE.  When the request's last KV
 * page fills (a capacity boundary), both summaries are scored against every retained
 * key, the Top-p attention working-set size of each summary's softmax is taken, and
 * the request either gets one more physical page (the recent working set is larger)
 * or is compacted in place inside its current allocation, keeping the slots with the
 * highest max-of-both importance.  Hyper-parameters of the paper's runs (same page,
 * FAQ "Is GrowPage's code available?"): beta_S 0.9, beta_L 0.999, Top-p 0.99,
 * tau 0, local retention quota 64, KV block 256.
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller unless a comment says
 *     "host".  The library keeps no state between calls and allocates no memory.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 *     Nothing is synchronised with the host; device-side outcomes (pool exhaustion,
 *     copy-on-write shortfall) are reported per request in `status_out`.
 *   - Lifetimes: the library keeps no reference to a buffer once a call returns, but the
 *     kernels it queued read and write every buffer passed (request ids, inputs, outputs,
 *     scratch, pools, page state) until they complete.  Each buffer must stay allocated,
 *     and must not be handed to other work, until the work queued on `stream` is done:
 *     order its release after that stream (an event recorded on it, or a stream-aware
 *     allocator told of the use, e.g. PyTorch's Tensor.record_stream).  Releasing a
 *     request-id array right after a call on a second stream lets an allocator reuse it
 *     while the kernels still index page tables with it.
 *   - Argument errors are detected on the host before any launch and return
 *     GP_ERR_INVALID (nothing is launched).  A failed launch returns GP_ERR_HIP.
 *     Shapes the kernels do not implement return GP_ERR_UNSUPPORTED.
 *   - `req_ids[b]` (b < n_req) names the request slot of batch entry b; all
 *     per-request state (summaries, page-table rows, n_alloc, fill) is indexed by slot,
 *     all outputs by batch entry.  Slots in one call must be distinct.
 *   - Device-resident state is trusted, not validated (checking it would need a copy to
 *     the host): slots req_ids[b] in [0, max_req); 0 <= n_alloc[r] < max_pages;
 *     0 <= fill[r] <= P; page ids in page_table[r][0 .. n_alloc[r]] in [0, num_pages);
 *     refcounts and the free stack consistent with the page tables; pos[b] >= 0.
 *     Values outside these ranges make the kernels read or write out of bounds.
 *
 * Paged KV model (the write-page model).  Request r owns n_alloc[r] = A allocation
 * pages page_table[r][0..A-1] plus one write page page_table[r][A] holding fill[r]
 * tokens.  Its candidate slots are n = A*P + fill, slot i living in page i / P at
 * offset i % P.  A boundary is fill == P.  Grow: the write page joins the allocation
 * (A+1) and a page popped from the free stack becomes the new write page (fill 0).
 * Compact: k = A*P slots are kept -- the last min(n_local, k) always, the others by
 * importance (max over the KV head's query heads and both summaries of the softmax
 * probability), an exact tie going to the more recent slot -- and are packed in slot
 * order into slots 0..k-1 of the same pages (stable, in place); fill becomes 0.
 * Pages are shared by all layers and heads.  A page whose refcount exceeds 1 at the
 * start of gp_compact and whose contents would change is first copied to a fresh page
 * (copy-on-write).  The free stack is free_stack[0 .. *free_top-1], top last.
 */
#ifndef GROWPAGE_H
#define GROWPAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GP_ABI_VERSION 2

typedef enum gp_status {
  GP_OK = 0,
  GP_ERR_INVALID = 1,      /* bad argument (NULL pointer, size, stride, alignment)    */
  GP_ERR_HIP = 2,          /* a HIP runtime call or kernel launch failed              */
  GP_ERR_SCRATCH = 3,      /* scratch buffer smaller than gp_scratch_bytes() asks for */
  GP_ERR_UNSUPPORTED = 4   /* shape not implemented (see each entry point)            */
} gp_status;

typedef enum gp_dtype { GP_F32 = 0, GP_BF16 = 1 } gp_dtype;

/* Per-request status bits written to status_out (device, int32). */
#define GP_REQ_GROW_DENIED 1      /* wanted to grow; free stack empty or page-table row full: compacted */
#define GP_REQ_DEFERRED 2         /* copy-on-write demand exceeded the free stack: left untouched      */
#define GP_REQ_NOT_AT_BOUNDARY 4  /* fill != P: no decision applied, left untouched                    */
#define GP_REQ_OVERFLOW 8         /* sum of candidate slots exceeded max_total_tokens: not scanned     */

/* Decisions written to decision_out (device, uint8). */
#define GP_DECISION_COMPACT 0
#define GP_DECISION_GROW 1
#define GP_DECISION_SHRINK 2   /* compacted into one allocation page fewer (GP_POLICY_SHRINK) */

/* Counters written to counters_out (device, int32[GP_NUM_COUNTERS]).  gp_decide
 * writes GROWS and GROW_DENIED; gp_compact writes the others. */
enum {
  GP_CNT_GROWS = 0,
  GP_CNT_COMPACTS = 1,       /* requests compacted (not deferred)                   */
  GP_CNT_GROW_DENIED = 2,
  GP_CNT_DEFERRED = 3,
  GP_CNT_COW_PAGES = 4,      /* pages copied on write                               */
  GP_CNT_FREED_PAGES = 5,    /* pages whose refcount reached 0 and were pushed      */
  GP_CNT_MOVED_ROWS = 6,     /* sum over compacted (layer, KV head) of rows moved   */
  GP_CNT_COPIED_ROWS = 7,    /* rows (per layer and KV head) copied by copy-on-write */
  GP_CNT_SHRINKS = 8,        /* requests that released an allocation page (SHRINK)   */
  GP_NUM_COUNTERS = 9
};

/* Engine parameters (host struct, passed by pointer, read during the call only). */
typedef struct gp_params {
  float beta_s;     /* short-timescale smoothing factor, (0, 1]                        */
  float beta_l;     /* long-timescale smoothing factor, (0, 1]                         */
  float top_p;      /* working-set mass threshold; >= 1 means "all n slots"            */
  int32_t tau;      /* demand threshold: grow iff sum(W_S - W_L) > tau                 */
  int32_t n_local;  /* most recent slots always kept by a compaction (>= 0)            */
  int32_t shrink;   /* 0, or 1 for the SHRINK policy: a compaction of a request holding
                       A >= 2 allocation pages keeps (A-1)*P slots instead of A*P; must
                       match the policy given to gp_decide_policy                      */
} gp_params;

/* Paged K/V pools (host struct).  Element (layer l, page p, KV head g, slot s, i) of
 * K lives at k + l*stride_layer + p*stride_page + g*stride_head + s*stride_tok + i
 * (strides in elements, the d elements of a row contiguous); V likewise.  Rows must
 * be 16-byte aligned.  Supported: Hq == G*Hkv with G in {1, 2, 4}, d in {64, 128}, P a multiple of 8. */
typedef struct gp_kv {
  int32_t L, Hq, Hkv, d, P, num_pages;
  int32_t dtype;                 /* gp_dtype of K and V */
  void* k;                       /* device */
  void* v;                       /* device */
  int64_t stride_layer, stride_page, stride_head, stride_tok;
} gp_kv;

/* Page state (host struct of device pointers; all int32). */
typedef struct gp_pages {
  int32_t* page_table;  /* [max_req][max_pages] */
  int32_t max_req;
  int32_t max_pages;
  int32_t* n_alloc;     /* [max_req] allocation pages A            */
  int32_t* fill;        /* [max_req] tokens in the write page      */
  int32_t* refcount;    /* [num_pages]                              */
  int32_t* free_stack;  /* [num_pages]                              */
  int32_t* free_top;    /* [1]                                      */
} gp_pages;

/* Version of this ABI (GP_ABI_VERSION). */
int32_t gp_abi_version(void);

/* Human-readable name of a gp_status value (static string). */
const char* gp_status_string(int32_t status);

/* Text of the HIP error behind the calling thread's most recent GP_ERR_HIP (static
 * string from the HIP runtime; "no error" if there was none). */
const char* gp_last_hip_error_string(void);

/* Summary update, for every batch entry b, layer l, query head h and element i:
 *   S <- beta_s*S + (1-beta_s)*q,   L <- beta_l*L + (1-beta_l)*q
 * in float32 with each product and the sum rounded separately and (1-beta) formed in
 * float32 (GrowPage review, "Summary": moving averages of the queries before RoPE).
 * q: [n_req] x [L] x [Hq] x [d] of q_dtype at element strides q_stride_req,
 *    q_stride_layer, q_stride_head (d contiguous, 8-byte aligned rows).
 * sum_s, sum_l: [max_req][L][Hq][d] float32, updated in place at row req_ids[b].
 * Errors: GP_ERR_INVALID for NULL pointers, n_req < 0, d % 4 != 0. */
gp_status gp_update_summaries(const void* q, int32_t q_dtype, int64_t q_stride_req,
                              int64_t q_stride_layer, int64_t q_stride_head,
                              const int32_t* req_ids, int32_t n_req, int32_t L, int32_t Hq,
                              int32_t d, float* sum_s, float* sum_l, const gp_params* params,
                              void* stream);

/* Bytes of scratch that gp_boundary_scan and gp_compact need for a batch of n_req
 * requests whose candidate slots sum to at most max_total_tokens. */
size_t gp_scratch_bytes(const gp_kv* kv, int32_t n_req, int64_t max_total_tokens);

/* Boundary scan (GrowPage review, "Summary": one Top-p working-set size per summary).  For each batch entry b (slot r = req_ids[b]), layer l and query head h,
 * both summaries are rotated to position pos[r] (pos: [max_req] int32 by slot; positions
 * outside the table are clamped to it) with rotate-half pairs (i, i+d/2) and the caller's
 * table rope_cos/rope_sin [rope_max_pos][d/2] float32 (both NULL = no rotation), scored
 * against all n = n_alloc*P + fill keys of the request (scale 1/sqrt(d)), and
 *   ws_out[b][l][h][s] = smallest m whose m largest softmax probabilities sum >= top_p
 * (s = 0 short, 1 long; top_p >= 1 gives n).  It also selects each (layer, KV head)'s
 * evicted slots for a compaction into k = A*P slots (A = n_alloc; k = (A-1)*P when
 * params->shrink and A >= 2).  stats_out (optional, may be NULL):
 * [n_req][L][Hq][2][2] float32 = (max logit, sum exp(logit - max)); an entry with no
 * candidate slots (n = 0) gets working sets 0, max -INFINITY and sum 0.  The logits and
 * statistics are also kept in `scratch` for gp_compact, so the same scratch must be
 * passed to gp_compact unchanged.  The page state is only read.
 * Errors: GP_ERR_INVALID (NULL/shape), GP_ERR_SCRATCH (scratch too small),
 * GP_ERR_UNSUPPORTED (Hq / Hkv not 1, 2 or 4, d not 64/128, P % 8 != 0, max_pages * P > 2^24). */
gp_status gp_boundary_scan(const gp_kv* kv, const gp_pages* pages, const int32_t* req_ids,
                           int32_t n_req, const float* sum_s, const float* sum_l,
                           const float* rope_cos, const float* rope_sin, int32_t rope_max_pos,
                           const int32_t* pos, const gp_params* params, int32_t* ws_out,
                           float* stats_out, void* scratch, size_t scratch_bytes,
                           int64_t max_total_tokens, void* stream);

/* The logits behind the last gp_boundary_scan's working sets (GrowPage review, "Summary":
 * each summary is scored against every retained key), for inspection and parity checks:
 * copies batch entry `entry`'s scores from `scratch` (the scan's, unchanged since; n_req
 * and max_total_tokens as passed to it) to logits_out [L][Hkv][n][8] float32, row
 * 2*j + s being query head g*G + min(j, G-1) of KV head g (G = Hq/Hkv: with G < 4 the
 * rows of j >= G repeat head G-1) under summary s (0 short, 1 long),
 * scaled by 1/sqrt(d) and rotated as the scan did.  n: the entry's candidate slots
 * n_alloc*P + fill; slots the scan did not score (t >= its count, or an entry flagged
 * GP_REQ_OVERFLOW) read NaN.  gp_compact leaves the scores in place.
 * Errors: GP_ERR_INVALID (NULL, entry outside [0, n_req), n < 0), GP_ERR_SCRATCH. */
gp_status gp_scan_logits(const gp_kv* kv, int32_t n_req, int64_t max_total_tokens, const void* scratch,
                         size_t scratch_bytes, int32_t entry, int32_t n, float* logits_out, void* stream);

/* Decision and grow (GrowPage review, "Summary": one more page when the fast summary's
 * working set is the larger; FAQ: tau).  delta_out[b] = sum over l, h of
 * (ws[b][l][h][0] - ws[b][l][h][1]); decision GROW iff delta > tau.  Grows pop the free
 * stack in batch order; with the stack empty (or page_table row full) the request is
 * compacted instead and flagged GP_REQ_GROW_DENIED.  Requests with fill != P are
 * flagged GP_REQ_NOT_AT_BOUNDARY and left alone.  Updates page_table, n_alloc, fill,
 * refcount (1 for popped pages) and free_top.  ws: [n_req][L][Hq][2] as written by
 * gp_boundary_scan; P: page size (tokens).  decision_out [n_req] uint8,
 * delta_out [n_req] int32, status_out [n_req] int32 (overwritten), counters_out
 * (optional) int32[GP_NUM_COUNTERS]. */
gp_status gp_decide(const int32_t* ws, const int32_t* req_ids, int32_t n_req, int32_t L,
                    int32_t Hq, int32_t P, const gp_params* params, const gp_pages* pages,
                    uint8_t* decision_out, int32_t* delta_out, int32_t* status_out,
                    int32_t* counters_out, void* stream);

/* Decision policies the pages compare against GrowPage's own rule (GrowPage review,
 * "Strengths", item "Frequency-matched causal ablations", Tables 8-9; FAQ "How does
 * GrowPage differ from Zipage?" for the fixed budget). */
typedef enum {
  GP_POLICY_GROWPAGE = 0,        /* grow iff delta > tau (gp_decide)                         */
  GP_POLICY_RANDOM = 1,          /* grow iff rand_u[b] < grow_prob (random timing, matched frequency) */
  GP_POLICY_INVERSE = 2,         /* grow iff -delta > tau (signal direction reversed)        */
  GP_POLICY_ALWAYS_COMPACT = 3,  /* never grow (fixed per-request budget)                    */
  GP_POLICY_SHRINK = 4           /* grow iff delta > tau; otherwise (also after a denied grow)
                                    a request holding A >= 2 allocation pages is decided
                                    SHRINK: compacted into (A-1)*P slots, its reference to
                                    allocation page A-1 dropped and its write page moved to
                                    page_table[r][A-1] (irreversible shrinking); requires
                                    params->shrink == 1                                        */
} gp_policy;

/* gp_decide under a decision policy; everything but the grow/compact choice is as in
 * gp_decide (delta_out is always the signal).  rand_u: device float32 [n_req] uniform
 * draws in [0, 1), required for GP_POLICY_RANDOM and ignored otherwise; grow_prob: the
 * grow probability of GP_POLICY_RANDOM.  Errors: GP_ERR_INVALID for an unknown policy,
 * a missing rand_u, params->shrink not 1 exactly for GP_POLICY_SHRINK, or the gp_decide
 * conditions (gp_decide itself requires params->shrink == 0). */
gp_status gp_decide_policy(const int32_t* ws, const int32_t* req_ids, int32_t n_req, int32_t L,
                           int32_t Hq, int32_t P, const gp_params* params, int32_t policy,
                           const float* rand_u, float grow_prob, const gp_pages* pages,
                           uint8_t* decision_out, int32_t* delta_out, int32_t* status_out,
                           int32_t* counters_out, void* stream);

/* Compaction (GrowPage review, "Summary": pack the kept slots into the request's current
 * pages, ranked by the larger of the two importances; abstract: prefix sharing survives).
 * For every batch entry with decision COMPACT or SHRINK and fill == P: takes the n - k
 * evicted slots of each (layer, KV head) (k = A*P, or (A-1)*P for SHRINK, whose
 * allocation page A-1 then loses this reference and whose write page moves to
 * page_table[r][A-1], n_alloc = A-1), copies-on-write the pages that would change and are
 * shared (snapshot refcount > 1; fresh pages popped after gp_decide's grows, in batch
 * order and ascending page index), moves K and V rows in place, sets fill to 0,
 * decrements the refcounts of the replaced pages and pushes the pages that reach 0 in
 * ascending id order.  A request whose copy-on-write demand exceeds the free stack is
 * left untouched and flagged GP_REQ_DEFERRED (status_out is OR-ed, keep gp_decide's
 * bits).  evicted_out (optional): [n_req][L][Hkv][E] int32 with E = P (2P when
 * params->shrink), ascending evicted slots, -1 padded, for compacting entries.
 * params->shrink must be the value the scan used.  Needs the scratch of the preceding
 * gp_boundary_scan of the same batch, and gp_decide's decision_out. */
gp_status gp_compact(const gp_kv* kv, const gp_pages* pages, const int32_t* req_ids,
                     const uint8_t* decision, int32_t n_req, const gp_params* params,
                     int32_t* evicted_out, int32_t* status_out, int32_t* counters_out,
                     void* scratch, size_t scratch_bytes, int64_t max_total_tokens,
                     void* stream);

/* The two halves of gp_compact, in this order, with the same arguments; gp_compact is
 * exactly prepare followed by move.  prepare: keep-set selection, copy-on-write planning
 * and page copies, page-table rewrite (writes evicted_out and GP_REQ_DEFERRED).  move:
 * the in-place K/V row moves, refcount decrements, free-stack pushes, fill reset and
 * counters.  Exposed so that a caller can time or overlap the row moves on their own. */
gp_status gp_compact_prepare(const gp_kv* kv, const gp_pages* pages, const int32_t* req_ids,
                             const uint8_t* decision, int32_t n_req, const gp_params* params,
                             int32_t* evicted_out, int32_t* status_out, void* scratch,
                             size_t scratch_bytes, int64_t max_total_tokens, void* stream);
gp_status gp_compact_move(const gp_kv* kv, const gp_pages* pages, const int32_t* req_ids,
                          int32_t n_req, int32_t* counters_out, void* scratch,
                          size_t scratch_bytes, int64_t max_total_tokens, void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation: one boundary batch, exactly
 * gp_boundary_scan, then gp_decide_policy (GP_POLICY_SHRINK when params->shrink is 1,
 * else GP_POLICY_GROWPAGE), then gp_compact, with the same arguments, outputs and errors,
 * but no caller scratch: the scratch is a buffer of GP_STATIC_SCRATCH_BYTES that the
 * library holds on each device until the process ends.  Nothing is allocated: the
 * buffer's device address is looked up once per device (on the first call with that
 * device current) and kept.  Runs on the current device; `stream` must belong to it.
 * A batch whose gp_scratch_bytes(kv, n_req, max_total_tokens) exceeds
 * GP_STATIC_SCRATCH_BYTES returns GP_ERR_SCRATCH before anything is launched (64 MiB:
 * for example 16 requests of up to 8192 tokens on one layer of the 8B shape, or about
 * 7,000 tokens across all 32 layers).  The buffer keeps the last call's contents; every
 * region a call reads is written by that call first, so nothing needs clearing.  Calls
 * on one device share the buffer: two calls that can run at the same time on one device
 * (different streams or host threads without ordering) race and corrupt each other's
 * results; order them (one stream, or events).  evicted_out and counters_out may be NULL
 * as in gp_compact; decision_out, delta_out and status_out are required. */
#define GP_STATIC_SCRATCH_BYTES (64 << 20)
gp_status gp_boundary_step_static(const gp_kv* kv, const gp_pages* pages, const int32_t* req_ids,
                                  int32_t n_req, const float* sum_s, const float* sum_l,
                                  const float* rope_cos, const float* rope_sin, int32_t rope_max_pos,
                                  const int32_t* pos, const gp_params* params, int64_t max_total_tokens,
                                  int32_t* ws_out, float* stats_out, uint8_t* decision_out,
                                  int32_t* delta_out, int32_t* status_out, int32_t* evicted_out,
                                  int32_t* counters_out, void* stream);

/* Deployment helper (not part of the boundary path): physically contiguous device memory
 * for the K/V pools, with the signatures of a PyTorch pluggable allocator
 * (torch.cuda.memory.CUDAPluggableAllocator).  The compaction's row moves address pool
 * pages at random, and their speed depends on the physical pages behind the pools
 * (contiguity did not reliably change it in measurements).  Returns
 * NULL when the device cannot supply `size` contiguous bytes; the caller then allocates
 * ordinary memory.  The stream argument is unused. */
void* gp_contiguous_malloc(int64_t size, int32_t device, void* stream);
void gp_contiguous_free(void* ptr, int64_t size, int32_t device, void* stream);

/* Decode-loop helper: append one token per batch entry.  k_new, v_new:
 * [n_req][L][Hkv][d] of kv->dtype (contiguous).  Writes slot fill[r] of the write page
 * page_table[r][n_alloc[r]] and increments fill[r]; entries already at fill == P are
 * skipped and flagged GP_REQ_OVERFLOW in status_out (optional, OR-ed). */
gp_status gp_append_kv(const gp_kv* kv, const gp_pages* pages, const void* k_new,
                       const void* v_new, const int32_t* req_ids, int32_t n_req,
                       int32_t* status_out, void* stream);

/* Decode attention over the paged cache -- the consumer of the pages the engine rewrites
 * (GrowPage review, abstract and FAQ "How does GrowPage differ from Zipage?": the engine
 * works inside PagedAttention serving).  For batch entry b (request slot r =
 * req_ids[b]), layer l and query head h: out[b][l][h][:] = sum_i a_i v_i over the
 * request's n = n_alloc[r]*P + fill[r] slots, a = softmax(qr . k_i / sqrt(d)), where qr
 * is q[b][l][h] rotated to pos[r] (rotate-half pairs i, i + d/2, caller's table as in
 * gp_boundary_scan: both tables or neither, neither = identity; with tables, pos is
 * required, else GP_ERR_INVALID).  q: element strides like
 * gp_update_summaries, bf16 or float32; out: [n_req][L][Hq][d] float32 (zeros for n ==
 * 0).  Reads the pool only. */
gp_status gp_decode_attention(const gp_kv* kv, const gp_pages* pages, const void* q, int32_t q_dtype,
                              int64_t q_stride_req, int64_t q_stride_layer, int64_t q_stride_head,
                              const int32_t* req_ids, int32_t n_req, const float* rope_cos,
                              const float* rope_sin, int32_t rope_max_pos, const int32_t* pos,
                              float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GROWPAGE_H */
