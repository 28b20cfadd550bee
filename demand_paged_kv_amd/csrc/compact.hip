// Compaction inside the pages a request already holds (GrowPage review on evolve.pub,
// "Summary": a request that does not grow packs its older cache entries into its current
// pages, slots ranked by the larger of the two summaries' importance; FAQ "Is GrowPage's
// code available?": 64 recent tokens always kept; abstract: the method works on
// PagedAttention's pages, so prefix sharing survives, here through copy-on-write).
//
// Launch sequence for one batch (all on the caller's stream, no host round trip):
//   (the keep-sets -- the n-k least important candidate slots of each (entry, layer,
//    KV head) unit, ties to the older slot -- come from the scan's finish kernel)
//   publish_kernel   copy the keep-sets of compacting entries to the caller (optional).
//   req_kernel       per entry: kept slots k (A*P, or (A-1)*P for a SHRINK decision),
//                    first changed slot e (min over units), copy-on-write demand =
//                    shared pages (refcount > 1) at index in [e / P, k / P).
//   cowplan_kernel   1 block: greedy in batch order -- an entry whose demand fits the
//                    free stack reserves its pops, otherwise it is deferred.
//   cowassign_kernel per entry: assign popped pages in ascending page index, rewrite the
//                    page table, record (old, new).
//   cowcopy_kernel   copy every (old page, layer, KV head) block of K and V to the new page.
//   gather_kernel    per unit and tensor (K and V blocks of a unit adjacent): in-place stable
//                    compaction, slot j <- slot kept[j] for j in [e, k), 128 destination
//                    rows per step, all reads of a step before its writes (destinations
//                    never exceed sources).
//   finalize_kernel  1 block: refcount decrements of replaced pages and of the page each
//                    SHRINK entry releases (its last allocation page, whose table slot
//                    its write page takes), push the pages that reached zero in
//                    ascending id order, empty the write pages, counters.
#include "device_util.h"
#include "gp_internal.h"

namespace gp {
namespace {

enum { RQ_E = 0, RQ_NEED = 1, RQ_BASE = 2, RQ_STATE = 3, RQ_TOP = 4, RQ_K = 5, RQ_SHRINK = 6, RQ_N = kReqFields };
enum { ST_NONE = 0, ST_PENDING = 1, ST_GO = 2, ST_DEFERRED = 3 };

struct CompactArgs {
  Geo g;
  gp_pages pg;
  ScratchPtrs sp;
  const uint8_t* decision;
  int32_t ev_out_stride;  // evicted_out row length (P, or 2P under SHRINK)
  int32_t* evicted_out;
  int32_t* status_out;
  int32_t* counters_out;
};

__device__ __forceinline__ void unit_of_block(const Geo& g, const ScratchPtrs& sp, int blk, int& b,
                                              int& l, int& kvh) {
  const int upr = g.L * g.Hkv;
  const int rank = blk / upr;
  const int rem = blk - rank * upr;
  l = rem / g.Hkv;
  kvh = rem - l * g.Hkv;
  b = sp.order[rank];
}

__device__ __forceinline__ bool is_compacting(const CompactArgs& a, int b, int r) {
  const uint8_t d = a.decision[b];
  return a.sp.flags[b] == 0 && (d == GP_DECISION_COMPACT || d == GP_DECISION_SHRINK) && a.g.fill[r] == a.g.P;
}

// ----------------------------------------------------------------------------- keep-set
// The keep-sets themselves are selected by the scan's finish kernel; here they are only
// published to the caller for the entries that compact.
__global__ __launch_bounds__(64) void publish_kernel(CompactArgs a) {
  const Geo& g = a.g;
  const int64_t u = blockIdx.x;
  const int upr = g.L * g.Hkv;
  const int b = (int)(u / upr);
  const int r = g.req_ids[b];
  const int P = g.P;
  const bool comp = is_compacting(a, b, r);
  const int E = comp ? a.sp.n_tok[b] - kept_slots(g.n_alloc[r], P, a.decision[b] == GP_DECISION_SHRINK) : 0;
  const int S = a.ev_out_stride;
  for (int i = threadIdx.x; i < S; i += 64)
    a.evicted_out[u * S + i] = i < E ? a.sp.ev[u * ev_stride(P) + i] : -1;
}

// ----------------------------------------------------------------------------- per entry
__global__ __launch_bounds__(256) void req_kernel(CompactArgs a) {
  const Geo& g = a.g;
  __shared__ int red[4];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int r = g.req_ids[b];
  int32_t* rq = a.sp.req + (int64_t)b * RQ_N;
  if (!is_compacting(a, b, r)) {
    if (tid < RQ_N) rq[tid] = 0;
    return;
  }
  const int upr = g.L * g.Hkv;
  int e = 0x7fffffff;
  for (int i = tid; i < upr; i += 256) e = min(e, a.sp.e_unit[(int64_t)b * upr + i]);
  e = wave_min_int(e);
  if ((tid & 63) == 0) red[tid >> 6] = e;
  __syncthreads();
  e = min(min(red[0], red[1]), min(red[2], red[3]));
  __syncthreads();
  const bool shrink = a.decision[b] == GP_DECISION_SHRINK;
  const int k = kept_slots(g.n_alloc[r], g.P, shrink);
  const int32_t* pt = g.page_table + (int64_t)r * g.max_pages;
  int c = 0;
  for (int j = e / g.P + tid; j < k / g.P; j += 256) c += a.pg.refcount[pt[j]] > 1 ? 1 : 0;
  c = wave_sum_int(c);
  if ((tid & 63) == 0) red[tid >> 6] = c;
  __syncthreads();
  if (tid == 0) {
    rq[RQ_E] = e;
    rq[RQ_NEED] = red[0] + red[1] + red[2] + red[3];
    rq[RQ_BASE] = 0;
    rq[RQ_STATE] = ST_PENDING;
    rq[RQ_TOP] = 0;
    rq[RQ_K] = k;
    rq[RQ_SHRINK] = shrink ? 1 : 0;
  }
}

// ----------------------------------------------------------------------------- plan
constexpr int kPlanChunk = 2048;

__global__ __launch_bounds__(1024) void cowplan_kernel(CompactArgs a) {
  __shared__ int c_need[kPlanChunk], c_state[kPlanChunk], c_base[kPlanChunk], c_top[kPlanChunk];
  __shared__ int s_top, s_cum;
  const int tid = threadIdx.x;
  const int n_req = a.g.n_req;
  if (tid == 0) {
    s_top = *a.pg.free_top;
    s_cum = 0;
  }
  __syncthreads();
  for (int base = 0; base < n_req; base += kPlanChunk) {
    const int cnt = min(kPlanChunk, n_req - base);
    for (int i = tid; i < cnt; i += 1024) {
      const int32_t* rq = a.sp.req + (int64_t)(base + i) * RQ_N;
      c_need[i] = rq[RQ_NEED];
      c_state[i] = rq[RQ_STATE];
    }
    __syncthreads();
    if (tid == 0) {
      int top = s_top, cum = s_cum;
      for (int i = 0; i < cnt; ++i) {
        if (c_state[i] != ST_PENDING) continue;
        if (c_need[i] <= top) {
          c_top[i] = top;
          c_base[i] = cum;
          top -= c_need[i];
          cum += c_need[i];
          c_state[i] = ST_GO;
        } else {
          c_state[i] = ST_DEFERRED;
        }
      }
      s_top = top;
      s_cum = cum;
    }
    __syncthreads();
    for (int i = tid; i < cnt; i += 1024) {
      int32_t* rq = a.sp.req + (int64_t)(base + i) * RQ_N;
      rq[RQ_STATE] = c_state[i];
      if (c_state[i] == ST_GO) {
        rq[RQ_BASE] = c_base[i];
        rq[RQ_TOP] = c_top[i];
      }
      if (c_state[i] == ST_DEFERRED) a.status_out[base + i] |= GP_REQ_DEFERRED;
    }
    __syncthreads();
  }
  if (tid == 0) {
    *a.pg.free_top = s_top;
    a.sp.misc[0] = s_cum;
  }
}

__global__ __launch_bounds__(256) void cowassign_kernel(CompactArgs a) {
  const Geo& g = a.g;
  __shared__ int tmp[4];
  __shared__ int s_carry;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int32_t* rq = a.sp.req + (int64_t)b * RQ_N;
  if (rq[RQ_STATE] != ST_GO || rq[RQ_NEED] == 0) return;
  const int r = g.req_ids[b];
  const int kp = rq[RQ_K] / g.P;  // allocation pages the compaction writes
  const int j0 = rq[RQ_E] / g.P;
  const int cbase = rq[RQ_BASE];
  const int ptop = rq[RQ_TOP];
  int32_t* pt = a.pg.page_table + (int64_t)r * g.max_pages;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int jb = j0; jb < kp; jb += 256) {
    const int j = jb + tid;
    int old = -1;
    int flag = 0;
    if (j < kp) {
      old = pt[j];
      flag = a.pg.refcount[old] > 1 ? 1 : 0;
    }
    int total = 0;
    const int idx = s_carry + block_exscan_256(flag, tmp, &total);
    if (flag) {
      const int fresh = a.pg.free_stack[ptop - 1 - idx];
      a.sp.cow[(int64_t)(cbase + idx) * 2] = old;
      a.sp.cow[(int64_t)(cbase + idx) * 2 + 1] = fresh;
      pt[j] = fresh;
      a.pg.refcount[fresh] = 1;
    }
    __syncthreads();
    if (tid == 0) s_carry += total;
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void cowcopy_kernel(CompactArgs a) {
  const Geo& g = a.g;
  const int tid = threadIdx.x;
  const int ncow = a.sp.misc[0];
  const int per = g.L * g.Hkv * 2;
  const long long items = (long long)ncow * per;
  const int esz = g.dtype == GP_BF16 ? 2 : 4;
  const int cpr = g.d * esz / 16;  // 16-byte chunks per row
  const int rpp = 256 / cpr;       // rows per pass
  for (long long it = blockIdx.x; it < items; it += gridDim.x) {
    const int e = (int)(it / per);
    const int rem = (int)(it - (long long)e * per);
    const int which = rem & 1;
    const int lg = rem >> 1;
    const int l = lg / g.Hkv;
    const int kvh = lg - l * g.Hkv;
    const int old = a.sp.cow[(int64_t)e * 2];
    const int fresh = a.sp.cow[(int64_t)e * 2 + 1];
    char* base = reinterpret_cast<char*>(const_cast<void*>(which ? g.v : g.k));
    const int64_t hoff = (int64_t)l * g.s_layer + (int64_t)kvh * g.s_head;
    const char* src = base + (hoff + (int64_t)old * g.s_page) * esz;
    char* dst = base + (hoff + (int64_t)fresh * g.s_page) * esz;
    const int c = tid % cpr;
    for (int row = tid / cpr; row < g.P; row += rpp) {
      const int64_t ro = (int64_t)row * g.s_tok * esz + (int64_t)c * 16;
      *reinterpret_cast<uint4*>(dst + ro) = *reinterpret_cast<const uint4*>(src + ro);
    }
  }
}

// ----------------------------------------------------------------------------- gather
typedef unsigned v4u __attribute__((ext_vector_type(4)));
constexpr int kPtLds = 2048;  // page-table entries of one request cached in LDS
constexpr int kResidentGatherBlocks = 256 * 8;  // 256 CUs x 8 blocks of 4 waves

// Destination slot j receives source slot j + s(j) with s(j) = #{m : ev[m] - m <= j}
// (ev ascending): the m-th evicted slot shifts every destination from ev[m] - m on.
__device__ __forceinline__ int shift_of(const int* thr, int E, int j) {
  int lo = 0, hi = E;  // first m with thr[m] > j
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (thr[mid] <= j) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// One block moves the rows of one tensor (K or V) of one unit; a unit's K and V blocks
// are adjacent in the grid, so both pools are walked together (on physically contiguous
// pools this measured 7.4 ms against 8.3 ms for all K blocks before all V blocks on the
// 32-layer sweep; on scattered pools the two orders tie).  A step moves 128 destination
// rows per 256 threads; in each of its load/store instructions the block's THREADS
// threads cover THREADS/CPR whole rows contiguously (lane t takes 16-byte piece t % CPR
// of a row), so every store writes complete cache lines.
//
// Two forms of a step.  By default the page ids are read through a pointer that may
// point at LDS or at the global table, so each of a step's loads waits for the one
// before it; with many blocks per CU that costs nothing (their loads overlap) and it
// measured 1% faster on the 32-layer sweep.  HOIST reads the ids as LDS (or global) and
// issues all of a step's loads together, which is what counts when the grid is too
// small to fill the chip and each block's walk through its unit is a latency chain.
// A grid of at most one block per CU takes blocks of 1024 threads (THREADS), which move
// 512 rows per step: a quarter of the steps in each block's chain.
template <int CPR, bool HOIST, int THREADS = 256>  // 16-byte pieces per row; all of a step's loads in flight
__global__ __launch_bounds__(THREADS) void gather_kernel(CompactArgs a) {
  const Geo& g = a.g;
  constexpr int ROWS = 128 * THREADS / 256;  // destination rows per step
  constexpr int RPI = THREADS / CPR;         // rows per instruction
  constexpr int NI = ROWS / RPI;       // instructions per step
  __shared__ int s_thr[2 * 256];  // E <= 2P <= 512
  __shared__ int s_pt[kPtLds];
  const int tid = threadIdx.x;
  const int which = blockIdx.x & 1;
  int b, l, kvh;
  unit_of_block(g, a.sp, blockIdx.x >> 1, b, l, kvh);
  const int32_t* rq = a.sp.req + (int64_t)b * RQ_N;
  if (rq[RQ_STATE] != ST_GO) return;
  const int r = g.req_ids[b];
  const int P = g.P;
  const int n = a.sp.n_tok[b];
  const int A = g.n_alloc[r];
  const int k = rq[RQ_K];
  const int E = n - k;
  const int64_t u = ((int64_t)b * g.L + l) * g.Hkv + kvh;
  const int e = a.sp.e_unit[u];
  if (e >= k) return;
  const int32_t* ptg = a.pg.page_table + (int64_t)r * g.max_pages;
  const bool pt_lds = A + 1 <= kPtLds;
  for (int i = tid; i < E; i += THREADS) s_thr[i] = a.sp.ev[u * ev_stride(P) + i] - i;
  if (pt_lds)
    for (int i = tid; i <= A; i += THREADS) s_pt[i] = ptg[i];
  __syncthreads();
  const int esz = g.dtype == GP_BF16 ? 2 : 4;
  const int64_t hoff = ((int64_t)l * g.s_layer + (int64_t)kvh * g.s_head) * esz;
  char* base = reinterpret_cast<char*>(const_cast<void*>(which ? g.v : g.k)) + hoff;
  const int piece = (tid % CPR) * 16;
  const int rr = tid / CPR;
  const int64_t spage = g.s_page * esz, stok = g.s_tok * esz;
  if constexpr (HOIST) {
    auto run = [&](auto pt) {
      for (int j0 = e; j0 < k; j0 += ROWS) {
        int64_t srco[NI], dsto[NI];
        bool act[NI];
#pragma unroll
        for (int q = 0; q < NI; ++q) {
          const int jj = j0 + q * RPI + rr;
          act[q] = jj < k;
          const int jc = act[q] ? jj : k - 1;  // inactive lanes re-read a valid row, store nothing
          const int src = jc + shift_of(s_thr, E, jc);
          srco[q] = (int64_t)pt[src / P] * spage + (int64_t)(src % P) * stok + piece;
          dsto[q] = (int64_t)pt[jc / P] * spage + (int64_t)(jc % P) * stok + piece;
        }
        v4u val[NI];
#pragma unroll
        for (int q = 0; q < NI; ++q)
          val[q] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(base + srco[q]));
        __syncthreads();  // every read of this step lands before any write of it
#pragma unroll
        for (int q = 0; q < NI; ++q)
          if (act[q]) __builtin_nontemporal_store(val[q], reinterpret_cast<v4u*>(base + dsto[q]));
      }
    };
    typedef const __attribute__((address_space(3))) int* lds_ids;
    typedef const __attribute__((address_space(1))) int* global_ids;
    if (pt_lds) run((lds_ids)s_pt);
    else run((global_ids)ptg);
    return;
  }
  const int* pt = pt_lds ? s_pt : ptg;
  for (int j0 = e; j0 < k; j0 += ROWS) {
    v4u val[NI];
    int64_t dsto[NI];
    bool act[NI];
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int jj = j0 + q * RPI + rr;
      act[q] = jj < k;
      const int jc = act[q] ? jj : k - 1;  // inactive lanes re-read a valid row, store nothing
      const int src = jc + shift_of(s_thr, E, jc);
      const int64_t srco = (int64_t)pt[src / P] * spage + (int64_t)(src % P) * stok + piece;
      dsto[q] = (int64_t)pt[jc / P] * spage + (int64_t)(jc % P) * stok + piece;
      val[q] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(base + srco));
    }
    __syncthreads();  // every read of this step lands before any write of it
#pragma unroll
    for (int q = 0; q < NI; ++q)
      if (act[q]) __builtin_nontemporal_store(val[q], reinterpret_cast<v4u*>(base + dsto[q]));
  }
}

// ----------------------------------------------------------------------------- finalize
__global__ __launch_bounds__(1024) void finalize_kernel(CompactArgs a) {
  const Geo& g = a.g;
  __shared__ int tmp[16];
  __shared__ int s_carry;
  __shared__ unsigned long long s_moved;
  __shared__ int s_comp, s_def, s_shrink;
  const int tid = threadIdx.x;
  const int ncow = a.sp.misc[0];
  const int words = g.num_pages / 32 + 1;
  for (int w = tid; w < words; w += 1024) a.sp.bitmap[w] = 0u;
  if (tid == 0) {
    s_carry = 0;
    s_moved = 0;
    s_comp = 0;
    s_def = 0;
    s_shrink = 0;
  }
  __syncthreads();
  for (int e = tid; e < ncow; e += 1024) {
    const int old = a.sp.cow[(int64_t)e * 2];
    if (atomicSub(&a.pg.refcount[old], 1) == 1) atomicOr(&a.sp.bitmap[old >> 5], 1u << (old & 31));
  }
  // SHRINK entries release their last allocation page (outside the copy-on-write range,
  // so still the original page) and move their write page into its table slot.
  for (int b = tid; b < g.n_req; b += 1024) {
    const int32_t* rq = a.sp.req + (int64_t)b * RQ_N;
    if (rq[RQ_STATE] != ST_GO || !rq[RQ_SHRINK]) continue;
    const int r = g.req_ids[b];
    const int A = a.pg.n_alloc[r];
    int32_t* pt = a.pg.page_table + (int64_t)r * g.max_pages;
    const int old = pt[A - 1];
    if (atomicSub(&a.pg.refcount[old], 1) == 1) atomicOr(&a.sp.bitmap[old >> 5], 1u << (old & 31));
    pt[A - 1] = pt[A];
    a.pg.n_alloc[r] = A - 1;
    atomicAdd(&s_shrink, 1);
  }
  __threadfence();
  __syncthreads();
  const int top = *a.pg.free_top;
  for (int wb = 0; wb < words; wb += 1024) {
    const int w = wb + tid;
    const uint32_t bits = w < words ? a.sp.bitmap[w] : 0u;
    int total = 0;
    int pos = s_carry + block_exscan_1024(__popc(bits), tmp, &total);
    for (int bit = 0; bit < 32; ++bit)
      if (bits & (1u << bit)) a.pg.free_stack[top + pos++] = w * 32 + bit;
    __syncthreads();
    if (tid == 0) s_carry += total;
    __syncthreads();
  }
  // Empty the write pages of compacted entries; counters.
  for (int b = tid; b < g.n_req; b += 1024) {
    const int st = a.sp.req[(int64_t)b * RQ_N + RQ_STATE];
    if (st == ST_GO) {
      a.pg.fill[g.req_ids[b]] = 0;
      atomicAdd(&s_comp, 1);
    } else if (st == ST_DEFERRED) {
      atomicAdd(&s_def, 1);
    }
  }
  const int upr = g.L * g.Hkv;
  unsigned long long moved = 0;
  for (long long uu = tid; uu < (long long)g.n_req * upr; uu += 1024) {
    const int b = (int)(uu / upr);
    if (a.sp.req[(int64_t)b * RQ_N + RQ_STATE] != ST_GO) continue;
    const int k = a.sp.req[(int64_t)b * RQ_N + RQ_K];
    const int e = a.sp.e_unit[uu];
    if (e < k) moved += (unsigned long long)(k - e);
  }
  atomicAdd(&s_moved, moved);
  __syncthreads();
  if (tid == 0) {
    *a.pg.free_top = top + s_carry;
    if (a.counters_out) {
      a.counters_out[GP_CNT_COMPACTS] = s_comp;
      a.counters_out[GP_CNT_DEFERRED] = s_def;
      a.counters_out[GP_CNT_COW_PAGES] = ncow;
      a.counters_out[GP_CNT_FREED_PAGES] = s_carry;
      a.counters_out[GP_CNT_MOVED_ROWS] = (int32_t)min(s_moved, (unsigned long long)INT32_MAX);
      a.counters_out[GP_CNT_COPIED_ROWS] = (int32_t)min((long long)ncow * upr * g.P, (long long)INT32_MAX);
      a.counters_out[GP_CNT_SHRINKS] = s_shrink;
    }
  }
}

// ----------------------------------------------------------------------------- append
__global__ __launch_bounds__(256) void append_write_kernel(Geo g, gp_pages pg, const void* k_new,
                                                           const void* v_new) {
  const int b = blockIdx.x / g.L;
  const int l = blockIdx.x - b * g.L;
  const int r = g.req_ids[b];
  const int f = pg.fill[r];
  if (f >= g.P) return;
  const int page = pg.page_table[(int64_t)r * pg.max_pages + pg.n_alloc[r]];
  const int esz = g.dtype == GP_BF16 ? 2 : 4;
  const int cpr = g.d * esz / 16;
  const int items = g.Hkv * cpr * 2;
  for (int it = threadIdx.x; it < items; it += 256) {
    const int which = it / (g.Hkv * cpr);
    const int rem = it - which * g.Hkv * cpr;
    const int kvh = rem / cpr;
    const int c = rem - kvh * cpr;
    const char* src = reinterpret_cast<const char*>(which ? v_new : k_new) +
                      ((((int64_t)b * g.L + l) * g.Hkv + kvh) * g.d) * esz + c * 16;
    char* dst = reinterpret_cast<char*>(const_cast<void*>(which ? g.v : g.k)) +
                ((int64_t)l * g.s_layer + (int64_t)page * g.s_page + (int64_t)kvh * g.s_head +
                 (int64_t)f * g.s_tok) * esz + c * 16;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
}

__global__ __launch_bounds__(256) void append_bump_kernel(Geo g, gp_pages pg, int32_t* status) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= g.n_req) return;
  const int r = g.req_ids[b];
  if (pg.fill[r] < g.P) {
    pg.fill[r] += 1;
  } else if (status) {
    status[b] |= GP_REQ_OVERFLOW;
  }
}

}  // namespace

hipError_t launch_compact_prepare(const Geo& g, const gp_pages& pg, const ScratchPtrs& sp,
                                  const uint8_t* decision, int32_t* evicted_out,
                                  int32_t evicted_stride, int32_t* status_out, hipStream_t st) {
  CompactArgs a{g, pg, sp, decision, evicted_stride, evicted_out, status_out, nullptr};
  const unsigned units = (unsigned)((int64_t)g.n_req * g.L * g.Hkv);
  if (evicted_out) hipLaunchKernelGGL(publish_kernel, dim3(units), dim3(64), 0, st, a);
  hipLaunchKernelGGL(req_kernel, dim3((unsigned)g.n_req), dim3(256), 0, st, a);
  hipLaunchKernelGGL(cowplan_kernel, dim3(1), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(cowassign_kernel, dim3((unsigned)g.n_req), dim3(256), 0, st, a);
  hipLaunchKernelGGL(cowcopy_kernel, dim3(2048), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_compact_move(const Geo& g, const gp_pages& pg, const ScratchPtrs& sp,
                               int32_t* counters_out, hipStream_t st) {
  CompactArgs a{g, pg, sp, nullptr, 0, nullptr, nullptr, counters_out};
  const unsigned units = (unsigned)((int64_t)g.n_req * g.L * g.Hkv);
  const int esz = g.dtype == GP_BF16 ? 2 : 4;
  const int cpr = g.d * esz / 16;  // 16-byte pieces per row: 8, 16 or 32
  const dim3 grid(2 * units);      // K and V block of each unit, adjacent
  // A grid that fits in one round of resident blocks (8 per CU) is latency-bound: take
  // the form with all of a step's loads in flight; with at most one block per CU, in
  // blocks of 1024 threads (rows of up to 256 bytes: wider rows would not fit the
  // registers of 16 waves per CU).
  const bool small = 2 * (int64_t)units <= kResidentGatherBlocks;
  const bool tiny = 2 * (int64_t)units <= kResidentGatherBlocks / 8 && cpr <= 16;
  if (tiny) {
    if (cpr == 8) hipLaunchKernelGGL((gather_kernel<8, true, 1024>), grid, dim3(1024), 0, st, a);
    else hipLaunchKernelGGL((gather_kernel<16, true, 1024>), grid, dim3(1024), 0, st, a);
  } else if (cpr == 8) {
    if (small) hipLaunchKernelGGL((gather_kernel<8, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((gather_kernel<8, false>), grid, dim3(256), 0, st, a);
  } else if (cpr == 16) {
    if (small) hipLaunchKernelGGL((gather_kernel<16, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((gather_kernel<16, false>), grid, dim3(256), 0, st, a);
  } else {
    if (small) hipLaunchKernelGGL((gather_kernel<32, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((gather_kernel<32, false>), grid, dim3(256), 0, st, a);
  }
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_append(const Geo& g, const gp_pages& pg, const void* k_new, const void* v_new,
                         int32_t* status_out, hipStream_t st) {
  hipLaunchKernelGGL(append_write_kernel, dim3((unsigned)(g.n_req * g.L)), dim3(256), 0, st, g, pg,
                     k_new, v_new);
  hipLaunchKernelGGL(append_bump_kernel, dim3((unsigned)((g.n_req + 255) / 256)), dim3(256), 0, st,
                     g, pg, status_out);
  return hipGetLastError();
}

}  // namespace gp
