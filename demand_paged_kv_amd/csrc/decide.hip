// Boundary decision and grow (GrowPage review on evolve.pub, "Summary": the request gets
// one more physical page when the fast summary's working set is the larger one, and is
// compacted otherwise; FAQ "Is GrowPage's code available?": threshold tau 0).
//
// delta_b = sum over layers and query heads of (W_short - W_long); grow iff delta > tau
// (or, for the ablation policies the pages compare: iff -delta > tau, iff a uniform draw
// falls below a grow probability, or never).  Under SHRINK a request at its boundary
// that does not grow and holds two or more allocation pages is decided SHRINK (the
// compaction then keeps one page fewer).
// Grows pop the device free stack in batch order: the eligible entries are ranked by a
// block prefix sum and the first `free_top` of them receive free_stack[top-1-rank], so
// page ids are deterministic without atomics.  One 1024-thread block: the batch is
// small and the work is latency-bound integer bookkeeping.
#include "device_util.h"
#include "gp_internal.h"

namespace gp {
namespace {

struct DecideArgs {
  const int32_t* ws;
  const int32_t* req_ids;
  int32_t n_req, L, Hq, tau, P, policy;
  const float* rand_u;
  float grow_prob;
  gp_pages pg;
  uint8_t* decision;
  int32_t* delta;
  int32_t* status;
  int32_t* counters;
};

__global__ __launch_bounds__(1024) void decide_kernel(DecideArgs a) {
  __shared__ int tmp[16];
  __shared__ int s_carry, s_top0, s_denied;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int per = a.L * a.Hq;

  // Delta per entry, one wave per entry (coalesced reads of the working sets).
  for (int b = wave; b < a.n_req; b += 16) {
    const int32_t* w = a.ws + (int64_t)b * per * 2;
    long long acc = 0;
    for (int i = lane; i < per; i += 64) acc += (long long)w[2 * i] - w[2 * i + 1];
    acc = wave_sum_i64(acc);
    if (lane == 0) {
      const long long c = acc > INT32_MAX ? INT32_MAX : (acc < INT32_MIN ? INT32_MIN : acc);
      a.delta[b] = (int32_t)c;
    }
  }
  if (tid == 0) {
    s_carry = 0;
    s_top0 = *a.pg.free_top;
    s_denied = 0;
  }
  __syncthreads();
  const int top0 = s_top0;
  for (int base = 0; base < a.n_req; base += 1024) {
    const int b = base + tid;
    int eligible = 0, want = 0, st = 0, r = 0, A = 0;
    bool over = false, at = false;
    if (b < a.n_req) {
      r = a.req_ids[b];
      A = a.pg.n_alloc[r];
      over = a.ws[(int64_t)b * per * 2] < 0;
      at = a.pg.fill[r] == a.P;
      if (over) st |= GP_REQ_OVERFLOW;
      if (!at) st |= GP_REQ_NOT_AT_BOUNDARY;
      const int d = a.delta[b];
      bool grow = d > a.tau;
      if (a.policy == GP_POLICY_INVERSE) grow = -(long long)d > a.tau;
      else if (a.policy == GP_POLICY_RANDOM) grow = a.rand_u[b] < a.grow_prob;
      else if (a.policy == GP_POLICY_ALWAYS_COMPACT) grow = false;
      want = (!over && at && grow) ? 1 : 0;
      eligible = (want && A + 2 <= a.pg.max_pages) ? 1 : 0;
    }
    int total = 0;
    const int rk = s_carry + block_exscan_1024(eligible, tmp, &total);
    if (b < a.n_req) {
      const bool granted = eligible && rk < top0;
      if (want && !granted) {
        st |= GP_REQ_GROW_DENIED;
        atomicAdd(&s_denied, 1);
      }
      if (granted) {
        const int page = a.pg.free_stack[top0 - 1 - rk];
        a.pg.page_table[(int64_t)r * a.pg.max_pages + A + 1] = page;
        a.pg.refcount[page] = 1;
        a.pg.n_alloc[r] = A + 1;
        a.pg.fill[r] = 0;
      }
      uint8_t dec = granted ? GP_DECISION_GROW : GP_DECISION_COMPACT;
      if (!granted && a.policy == GP_POLICY_SHRINK && !over && at && A >= 2) dec = GP_DECISION_SHRINK;
      a.decision[b] = dec;
      a.status[b] = st;
    }
    __syncthreads();
    if (tid == 0) s_carry += total;
    __syncthreads();
  }
  if (tid == 0) {
    const int grows = min(s_carry, top0);
    *a.pg.free_top = top0 - grows;
    if (a.counters) {
      a.counters[GP_CNT_GROWS] = grows;
      a.counters[GP_CNT_GROW_DENIED] = s_denied;
    }
  }
}

}  // namespace

hipError_t launch_decide(const int32_t* ws, const int32_t* req_ids, int32_t n_req, int32_t L,
                         int32_t Hq, int32_t tau, const gp_pages& pg, int32_t P, int32_t policy,
                         const float* rand_u, float grow_prob, uint8_t* decision, int32_t* delta,
                         int32_t* status, int32_t* counters, hipStream_t st) {
  DecideArgs a{ws, req_ids, n_req, L, Hq, tau, P, policy, rand_u, grow_prob, pg, decision, delta, status,
               counters};
  hipLaunchKernelGGL(decide_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

}  // namespace gp
