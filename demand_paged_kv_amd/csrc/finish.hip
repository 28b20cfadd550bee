// Working sets and keep-sets of one boundary batch, from the logits the scan wrote.
// (GrowPage review on evolve.pub, "Summary": a Top-p working-set size per summary; a
// compaction keeps the slots ranked highest by the larger of the two importances;
// FAQ "Is GrowPage's code available?": local retention quota.)
//
// One 256-thread block per (entry, layer, KV head) unit, two reads of the unit's logits
// ([n][8] float32, token-major, with each row's max M), which either the same block has
// just computed (fused_scan_kernel, at the end of this file) or logit_kernel wrote:
//
//   read 1  x = M - l >= 0 for every element of the 8 rows.  Each element adds its
//           softmax mass exp(-x) (2^-40 fixed point, one 64-bit LDS atomic) to one of
//           255 bins of width 1/16, or to bin 255 (the tail) when x >= 255/16.
//           Integer sums make the normaliser Z exact and order-independent.  Walking
//           the bins from x = 0 (largest probabilities) gives the bin b* where the mass
//           reaches T = ceil(top_p * Z).
//   read 2  per row: elements above b* are counted in registers, the elements of b* are
//           appended to an LDS buffer (its size is bounded from the bin's mass: every
//           element of bin b carries at least the mass of x = (b+1)/16); in the same
//           pass the slot importance max_k exp(l_k - M_k) / Z_k feeds a threshold
//           buffer that keeps the n - k least important candidate slots (ties: older
//           slot first; importance ranked in the log domain, float64) -- the slots a
//           compaction evicts; whenever the buffer fills, a
//           radix select keeps its n - k smallest keys and lowers the threshold.
//   refine  per row, an exact radix select over the b* elements only, weighted by the
//           same fixed-point masses, in digits of 8 bits from the highest key bit in
//           which they differ: W = (elements above b*) + (elements of b* needed to reach T).
//           Rows whose b* elements did not fit the buffer (or whose crossing lies in the
//           tail, which only a near-tie allows) are refined by the whole block from
//           the logits in global memory, filtered to b*.
// All decisions are exact for the float32 logits the scan produced.
#include <algorithm>

#include "device_util.h"
#include "gp_internal.h"
#include "logit_mfma.h"

namespace gp {
namespace {

typedef unsigned long long u64;

constexpr int kXBins = 255;          // bins of width 1/16 covering x in [0, 255/16); 255 = tail
constexpr float kBinsPerNat = 16.0f;
// Crossing-bin elements held in LDS (all 8 rows): sized with the keep buffer so that a
// block stays within 40 KB of LDS and four blocks (16 waves) share a CU.
constexpr int cand_cap(int kcap) { return kcap == 512 ? 4864 : 3840; }
// Threshold buffer of keep-set candidates: 512 keys for pages of up to 64 slots, 1024
// above.  A unit evicts E <= 2P slots (2P when it shrinks by a page), and E + 256 <= the
// capacity, so that after a compaction down to the E smallest keys at least one more
// round of 256 new keys fits before the next one.
constexpr int keep_cap(int P) { return P <= 64 ? 512 : 1024; }
static_assert(2 * 64 + 256 <= 512 && 2 * 256 + 256 <= 1024, "keep buffer too small for 2P evictions");

enum { MODE_DONE = 0, MODE_LDS = 1, MODE_GLOBAL = 2 };

__device__ __forceinline__ int x_bin(float xv) {
  const float f = xv * kBinsPerNat;
  return f < (float)kXBins ? (int)f : kXBins;
}

__device__ __forceinline__ u64 wave_exscan_u64(u64 v, u64* total) {
  const u64 x = wave_incl_sum_u64(v);
  *total = lane_u64(x, 63);
  return x - v;
}

__device__ __forceinline__ uint32_t wave_exscan_u32(uint32_t v) { return wave_incl_sum_u32(v) - v; }

// Walk 256 bins (lane l owns 4 consecutive bins in walk order; DESC walks bin 255 first)
// accumulating mass from (base_mass, base_cnt); return the first bin where the mass
// reaches T together with the mass and count strictly before it.  cnt may be null
// (counts then stay at base_cnt).
template <bool DESC>
__device__ __forceinline__ bool wave_find_crossing(const uint32_t* cnt, const u64* ms, u64 base_mass,
                                                   uint32_t base_cnt, u64 T, int lane, int* chosen,
                                                   u64* mass_before, uint32_t* cnt_before) {
  u64 m4[4];
  uint32_t c4[4];
  u64 ls = 0;
  uint32_t lc = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int bin = DESC ? 255 - (4 * lane + q) : 4 * lane + q;
    m4[q] = ms[bin];
    c4[q] = cnt ? cnt[bin] : 0u;
    ls += m4[q];
    lc += c4[q];
  }
  u64 tot = 0;
  u64 acc = base_mass + wave_exscan_u64(ls, &tot);
  uint32_t ac = base_cnt + wave_exscan_u32(lc);
  int my = -1;
  u64 my_m = 0;
  uint32_t my_c = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (my < 0) {
      if (m4[q] > 0 && acc + m4[q] >= T) {
        my = DESC ? 255 - (4 * lane + q) : 4 * lane + q;
        my_m = acc;
        my_c = ac;
      } else {
        acc += m4[q];
        ac += c4[q];
      }
    }
  }
  const u64 bal = __ballot(my >= 0);
  if (bal == 0) return false;
  const int f = __builtin_ctzll(bal);
  *chosen = (int)lane_u32((uint32_t)my, f);
  *mass_before = lane_u64(my_m, f);
  *cnt_before = lane_u32(my_c, f);
  return true;
}

// W from the final key: (above) + elements of value vstar needed to reach T.
__device__ __forceinline__ int finish_w(uint32_t prefix, float M, u64 T, u64 acc_mass, uint32_t acc_cnt,
                                        int n) {
  const float vstar = ord_key_inv(prefix);
  const u64 q = fixed_mass(vstar - M);
  const u64 need = T > acc_mass ? T - acc_mass : 0;
  const u64 jn = q ? (need + q - 1) / q : 1ull;
  return (int)min((u64)n, (u64)acc_cnt + max(jn, 1ull));
}

// Keep-set key of slot i with negative log-importance v >= 0: bits 62..24 hold the top 39
// bits of v's float64 pattern complemented (a less important slot has a smaller key; the
// sign bit, always 0, is dropped, so every key stays below the buffer's initial
// threshold of all ones), the low 24 bits the slot, so that equal importance evicts the
// older slot first.  Relative resolution 2^-27; slots stay below 2^24 (max_pages * P is
// checked on the host).
constexpr u64 kSlotMask = (1ull << 24) - 1ull;
__device__ __forceinline__ u64 imp_key(double v, int i) {
  const u64 vb = (u64)__double_as_longlong(v);
  return (((~vb) << 1) >> 25 << 24) | (u64)(uint32_t)i;
}

// Exact weighted radix select by one wave over the m LDS elements of one row (keys
// descending), synchronised within the wave only.  (acc_cnt, acc_mass) hold the
// elements above the range.  Radix digits start at the highest differing key bit.
__device__ int wave_refine_lds(const float* src, int m, float M, u64 T, u64 acc_mass, uint32_t acc_cnt,
                               uint32_t* hcnt, u64* hms, int lane, int n) {
  uint32_t kmin = 0xffffffffu, kmax = 0;
  for (int c = lane; c < m; c += 64) {
    const uint32_t key = ord_key(src[c]);
    kmin = min(kmin, key);
    kmax = max(kmax, key);
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (kmin == kmax) return finish_w(kmin, M, T, acc_mass, acc_cnt, n);
  const int hb = 31 - __builtin_clz(kmin ^ kmax);     // highest differing bit
  uint32_t mask = hb >= 31 ? 0u : ~((2u << hb) - 1u);  // bits above hb: common to all
  uint32_t prefix = kmin & mask;
  // digits of up to 8 bits from the highest differing bit down
  for (int top = hb + 1; top > 0;) {
    const int w = min(8, top);
    const int shift = top - w;
    const uint32_t dmask = (1u << w) - 1u;
    top = shift;
    for (int q = lane; q < 256; q += 64) {
      hcnt[q] = 0;
      hms[q] = 0;
    }
    wave_lds_sync();
    for (int c = lane; c < m; c += 64) {
      const float v = src[c];
      const uint32_t key = ord_key(v);
      if ((key & mask) == prefix) {
        const uint32_t bin = (key >> shift) & dmask;
        atomicAdd(&hcnt[bin], 1u);
        atomicAdd(&hms[bin], (u64)fixed_mass(v - M));
      }
    }
    wave_lds_sync();
    int chosen = 0;
    u64 mb = acc_mass;
    uint32_t cb = acc_cnt;
    if (wave_find_crossing<true>(hcnt, hms, acc_mass, acc_cnt, T, lane, &chosen, &mb, &cb)) {
      acc_mass = mb;
      acc_cnt = cb;
      prefix |= (uint32_t)chosen << shift;
    }
    mask |= dmask << shift;
    wave_lds_sync();
  }
  return finish_w(prefix, M, T, acc_mass, acc_cnt, n);
}

// The same select by the whole block over the elements of one row in global memory whose
// bin is `bstar` (token-major logits, stride 8).  Block-uniform control flow.
__device__ int block_refine_global(const float* row, int n, int bstar, float M, u64 T, u64 acc_mass,
                                   uint32_t acc_cnt, uint32_t* hcnt, u64* hms, uint32_t* red, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  uint32_t kmin = 0xffffffffu, kmax = 0;
  for (int i = tid; i < n; i += 256) {
    const float v = row[(int64_t)i * kDists];
    if (x_bin(M - v) == bstar) {
      const uint32_t key = ord_key(v);
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    }
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    red[wave] = kmin;
    red[4 + wave] = kmax;
  }
  __syncthreads();
  kmin = min(min(red[0], red[1]), min(red[2], red[3]));
  kmax = max(max(red[4], red[5]), max(red[6], red[7]));
  __syncthreads();
  if (kmin == kmax) return finish_w(kmin, M, T, acc_mass, acc_cnt, n);
  const int hb = 31 - __builtin_clz(kmin ^ kmax);
  uint32_t mask = hb >= 31 ? 0u : ~((2u << hb) - 1u);
  uint32_t prefix = kmin & mask;
  for (int top = hb + 1; top > 0;) {
    const int w = min(8, top);
    const int shift = top - w;
    const uint32_t dmask = (1u << w) - 1u;
    top = shift;
    hcnt[tid] = 0;
    hms[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
      const float v = row[(int64_t)i * kDists];
      const uint32_t key = ord_key(v);
      if (x_bin(M - v) == bstar && (key & mask) == prefix) {
        const uint32_t bin = (key >> shift) & dmask;
        atomicAdd(&hcnt[bin], 1u);
        atomicAdd(&hms[bin], (u64)fixed_mass(v - M));
      }
    }
    __syncthreads();
    if (wave == 0) {
      int chosen = 0;
      u64 mb = acc_mass;
      uint32_t cb = acc_cnt;
      const bool ok = wave_find_crossing<true>(hcnt, hms, acc_mass, acc_cnt, T, lane, &chosen, &mb, &cb);
      if (lane == 0) {
        red[0] = ok ? 1u : 0u;
        red[1] = (uint32_t)chosen;
        red[2] = cb;
        red[3] = (uint32_t)(mb & 0xffffffffu);
        red[4] = (uint32_t)(mb >> 32);
      }
    }
    __syncthreads();
    if (red[0]) {
      prefix |= red[1] << shift;
      acc_cnt = red[2];
      acc_mass = ((u64)red[4] << 32) | red[3];
    }
    mask |= dmask << shift;
    __syncthreads();
  }
  return finish_w(prefix, M, T, acc_mass, acc_cnt, n);
}

// Bits of a 64-bit key above bit position top - 1 (top in 0..64).
__device__ __forceinline__ u64 mask_above(int top) { return top >= 64 ? 0ull : ~((1ull << top) - 1ull); }

// The kth smallest (1-based) of cnt distinct keys in LDS, by a block-wide radix select:
// 8-bit digits from the highest bit in which the keys differ, each pass histogramming
// the keys that match the digits chosen so far; it stops as soon as the chosen digit's
// bucket holds one key.  hist: 256 LDS counters; sx: 8 LDS scratch words.
// Block-uniform control flow.
__device__ u64 block_kth_smallest(const u64* keys, int cnt, int kth, uint32_t* hist, u64* sx, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  u64 kmin = ~0ull, kmax = 0;
  for (int i = tid; i < cnt; i += 256) {
    kmin = min(kmin, keys[i]);
    kmax = max(kmax, keys[i]);
  }
  kmin = wave_min_u64(kmin);
  kmax = wave_max_u64(kmax);
  if (lane == 0) {
    sx[wave] = kmin;
    sx[4 + wave] = kmax;
  }
  __syncthreads();
  kmin = min(min(sx[0], sx[1]), min(sx[2], sx[3]));
  kmax = max(max(sx[4], sx[5]), max(sx[6], sx[7]));
  __syncthreads();
  if (kmin == kmax) return kmin;
  const int hb = 63 - __builtin_clzll(kmin ^ kmax);
  u64 prefix = kmin & mask_above(hb + 1);
  int need = kth;
  for (int top = hb + 1; top > 0;) {
    const int w = min(8, top);
    const int shift = top - w;
    const uint32_t dmask = (1u << w) - 1u;
    const u64 hmask = mask_above(top);
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < cnt; i += 256) {
      const u64 key = keys[i];
      if (((key ^ prefix) & hmask) == 0) atomicAdd(&hist[(uint32_t)(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (wave == 0) {  // ascending walk: the first digit whose cumulative count reaches need
      uint32_t c4[4], ls = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c4[q] = hist[4 * lane + q];
        ls += c4[q];
      }
      uint32_t acc = wave_incl_sum_u32(ls) - ls;
      int my = -1;
      uint32_t before = 0, inbin = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (my < 0) {
          if (acc + c4[q] >= (uint32_t)need) {
            my = 4 * lane + q;
            before = acc;
            inbin = c4[q];
          } else {
            acc += c4[q];
          }
        }
      }
      const u64 bal = __ballot(my >= 0);
      const int f = bal ? __builtin_ctzll(bal) : 0;
      if (lane == 0) {
        sx[0] = lane_u32((uint32_t)my, f);
        sx[1] = lane_u32(before, f);
        sx[2] = lane_u32(inbin, f);
      }
    }
    __syncthreads();
    const u64 d = sx[0];
    need -= (int)sx[1];
    const u64 inbin = sx[2];
    __syncthreads();
    prefix |= d << shift;
    top = shift;
    if (inbin == 1 && top > 0) {  // one key left in the bucket: it is the answer
      const u64 m2 = mask_above(top);
      for (int i = tid; i < cnt; i += 256)
        if (((keys[i] ^ prefix) & m2) == 0) sx[3] = keys[i];
      __syncthreads();
      prefix = sx[3];
      __syncthreads();
      break;
    }
  }
  return prefix;
}

// Working sets and keep-set of unit (entry at rank `rank`, layer l, KV head kvh), by one
// 256-thread block.
// The block's large LDS arrays, laid out back to back in one buffer (the fused kernel
// uses the same bytes to stage logits before the selection starts).
template <int KCAP>
struct FinishLds {
  u64 ms[kDists][256];          // read 1 bins; later refinement histograms
  float cand[cand_cap(KCAP)];   // crossing-bin elements
  u64 kbuf[KCAP];               // keep-set threshold buffer
};

template <int KCAP>
__device__ __forceinline__ void finish_unit(const FinishArgs& a, int rank, int l, int kvh, FinishLds<KCAP>& lds) {
  constexpr int kCandCap = cand_cap(KCAP);
  const Geo& g = a.g;
  u64 (*ms)[256] = lds.ms;
  float* cand = lds.cand;
  u64* kbuf = lds.kbuf;
  __shared__ float s_M[kDists];
  __shared__ double s_lse[kDists];
  __shared__ u64 s_T[kDists], s_above[kDists], s_Z[kDists];
  __shared__ uint32_t s_above_cnt[kDists], s_red[8];
  __shared__ int s_mode[kDists], s_bin[kDists], s_off[kDists], s_fill[kDists], s_ub[kDists], s_W[kDists];
  __shared__ int s_kcount, s_c2;
  __shared__ u64 s_ktau, s_x[8];
  // keep-set selection works in the read-1 bins, free between the crossing search and
  // the refinement: 256 digit counters, then up to 256 selected keys
  uint32_t* sel_hist = reinterpret_cast<uint32_t*>(&ms[0][0]);
  u64* sel_tmp = &ms[1][0];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = a.sp.order[rank];
  const int64_t u = ((int64_t)b * g.L + l) * g.Hkv + kvh;
  // statistics / working-set index of row k (rows of a missing head read their twin's)
  auto widx = [&](int k) { return (((int64_t)b * g.L + l) * g.Hq + kvh * g.G + row_head(k, g.G)) * 2 + (k & 1); };
  const bool real_row = tid < kDists && row_real(tid, g.G);
  if (a.sp.flags[b]) {
    if (real_row) a.ws_out[widx(tid)] = -1;
    return;
  }
  const int n = a.sp.n_tok[b];
  const int r = g.req_ids[b];
  constexpr int kcap = KCAP;
  const int kk = kept_slots(g.n_alloc[r], g.P, a.shrink != 0);  // slots a compaction keeps
  const int E = min(max(n - kk, 0), ev_stride(g.P));               // slots it evicts
  const int nl = min(max(a.n_local, 0), min(kk, n));
  const int cand_slots = n - nl;
  const int64_t ubase = (a.sp.tok_off[b] * g.L * g.Hkv + (int64_t)(l * g.Hkv + kvh) * logit_rows(n)) * kDists;
  const float* x = a.sp.logits + ubase;

  if (n == 0) {
    if (real_row) {
      a.ws_out[widx(tid)] = 0;
      a.sp.stats[widx(tid) * 2 + 1] = 0.f;
      if (a.stats_out) {
        a.stats_out[widx(tid) * 2] = a.sp.stats[widx(tid) * 2];
        a.stats_out[widx(tid) * 2 + 1] = 0.f;
      }
    }
    if (tid == 0) a.sp.e_unit[u] = 0;
    return;
  }

  // ---- read 1: binned masses (bin 255 collects the tail)
  for (int i = tid; i < kDists * 256; i += 256) (&ms[0][0])[i] = 0;
  if (tid < kDists) {
    s_M[tid] = a.sp.stats[widx(tid) * 2];
    s_above_cnt[tid] = 0;
  }
  __syncthreads();
  float M[kDists];
#pragma unroll
  for (int k = 0; k < kDists; ++k) M[k] = s_M[k];
  {
    float4 nlo[2], nhi[2];
    auto fetch = [&](int i0) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int i = i0 + 256 * t;
        nlo[t] = make_float4(0.f, 0.f, 0.f, 0.f);
        nhi[t] = nlo[t];
        if (i < n) {
          nlo[t] = *reinterpret_cast<const float4*>(x + (int64_t)i * kDists);
          nhi[t] = *reinterpret_cast<const float4*>(x + (int64_t)i * kDists + 4);
        }
      }
    };
    fetch(tid);
    for (int i0 = tid; i0 < n; i0 += 512) {
      float v[2][kDists];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        v[t][0] = nlo[t].x; v[t][1] = nlo[t].y; v[t][2] = nlo[t].z; v[t][3] = nlo[t].w;
        v[t][4] = nhi[t].x; v[t][5] = nhi[t].y; v[t][6] = nhi[t].z; v[t][7] = nhi[t].w;
      }
      if (i0 + 512 < n) fetch(i0 + 512);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (i0 + 256 * t >= n) break;
#pragma unroll
        for (int k = 0; k < kDists; ++k) {
          const float xv = M[k] - v[t][k];
          atomicAdd(&ms[k][x_bin(xv)], fixed_mass(-xv));
        }
      }
    }
  }
  __syncthreads();

  // ---- crossing bin of each row (wave w: rows 2w, 2w+1)
  for (int d2 = 0; d2 < 2; ++d2) {
    const int k = 2 * wave + d2;
    u64 ls = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) ls += ms[k][4 * lane + q];
    u64 Z = 0;
    wave_exscan_u64(ls, &Z);
    u64 T = 0;
    int mode = MODE_LDS, W = 0, chosen = kXBins;
    u64 mb = 0;
    uint32_t cb = 0;
    if (a.top_p >= 1.0f) {
      mode = MODE_DONE;
      W = n;
    } else {
      T = (u64)ceil((double)a.top_p * (double)Z);
      if (T == 0) {
        mode = MODE_DONE;
        W = 1;
      }
    }
    if (mode == MODE_LDS) {
      // T <= Z, so some bin reaches it; a crossing in the tail bin (only a near-tie
      // allows it) is refined by the block from global memory
      wave_find_crossing<false>(nullptr, &ms[k][0], 0, 0, T, lane, &chosen, &mb, &cb);
      if (chosen == kXBins) mode = MODE_GLOBAL;
    }
    if (lane == 0) {
      s_mode[k] = mode;
      s_W[k] = W;
      s_T[k] = T;
      s_Z[k] = Z;
      s_bin[k] = chosen;
      s_above[k] = mb;
      // upper bound on the elements of the crossing bin: each carries at least the mass
      // of x = (b+1)/16 (masses do not increase with x)
      int ub = 0;
      if (mode == MODE_LDS) {
        const u64 qmin = fixed_mass(-((float)(chosen + 1) / kBinsPerNat));
        const u64 mass = ms[k][chosen];
        ub = qmin ? (int)min(mass / qmin + 1, (u64)kCandCap + 1) : kCandCap + 1;
      }
      s_fill[k] = ub;  // temporarily: the bound
    }
  }
  __syncthreads();
  if (tid == 0) {
    int off = 0;
    for (int k = 0; k < kDists; ++k) {
      const int ub = s_fill[k];
      s_fill[k] = 0;
      s_off[k] = 0;
      s_ub[k] = ub;
      if (s_mode[k] != MODE_LDS) continue;
      if (off + ub <= kCandCap) {
        s_off[k] = off;
        off += ub;
      } else {
        s_mode[k] = MODE_GLOBAL;
      }
    }
    s_kcount = 0;
    s_ktau = ~0ull;
  }
  if (tid < kDists) {  // log of the softmax normaliser: ln(sum exp(l)) = M + ln Z
    const double z = (double)s_Z[tid] / (double)kMassScale;
    s_lse[tid] = (double)s_M[tid] + log(z);
  }
  __syncthreads();

  // ---- read 2: counts above the crossing bins, crossing-bin elements, keep-set candidates
  int mode[kDists], binstar[kDists], boff[kDists], bub[kDists];
  double lse[kDists];
  uint32_t above[kDists];
#pragma unroll
  for (int k = 0; k < kDists; ++k) {
    mode[k] = s_mode[k];
    binstar[k] = s_bin[k];
    boff[k] = s_off[k];
    bub[k] = s_ub[k];
    lse[k] = s_lse[k];
    above[k] = 0;
  }
  float4 nlo = make_float4(0.f, 0.f, 0.f, 0.f), nhi = nlo;
  if (tid < n) {
    nlo = *reinterpret_cast<const float4*>(x + (int64_t)tid * kDists);
    nhi = *reinterpret_cast<const float4*>(x + (int64_t)tid * kDists + 4);
  }
  for (int base = 0; base < n; base += 256) {
    const int i = base + tid;
    const float v8[kDists] = {nlo.x, nlo.y, nlo.z, nlo.w, nhi.x, nhi.y, nhi.z, nhi.w};
    if (i + 256 < n) {
      nlo = *reinterpret_cast<const float4*>(x + (int64_t)(i + 256) * kDists);
      nhi = *reinterpret_cast<const float4*>(x + (int64_t)(i + 256) * kDists + 4);
    }
    if (i < n) {
      // slot importance max over rows of exp(l - M) / Z, ranked by its negative log
      // nl = min over rows of (M + ln Z - l) >= 0 in float64: no underflow however far
      // below the maximum a slot lies, and no rounding beyond the logits' own
      double nl = INFINITY;
#pragma unroll
      for (int k = 0; k < kDists; ++k) {
        const float v = v8[k];
        const float xv = M[k] - v;
        const int bin = x_bin(xv);
        above[k] += bin < binstar[k] ? 1u : 0u;
        if (bin == binstar[k] && mode[k] != MODE_DONE) {  // counted for every row, kept for LDS rows
          const int p = atomicAdd(&s_fill[k], 1);
          if (mode[k] == MODE_LDS && p < bub[k]) cand[boff[k] + p] = v;  // beyond the bound: block path
        }
        nl = fmin(nl, lse[k] - (double)v);
      }
      if (E > 0 && i < cand_slots) {
        const u64 key = imp_key(nl, i);
        if (key < s_ktau) kbuf[atomicAdd(&s_kcount, 1)] = key;
      }
    }
    __syncthreads();
    const int cnt = s_kcount;
    // every thread holds the count before the next round adds to it: without this
    // barrier a wave that runs ahead could raise it under a slower one's read, and the
    // waves would disagree on entering the block-wide selection below
    __syncthreads();
    if (cnt > kcap - 256) {  // the next round might not fit: keep the E smallest
      const u64 K = block_kth_smallest(kbuf, cnt, E, sel_hist, s_x, tid);
      if (tid == 0) s_c2 = 0;
      __syncthreads();
      for (int j = tid; j < cnt; j += 256)
        if (kbuf[j] <= K) sel_tmp[atomicAdd(&s_c2, 1)] = kbuf[j];
      __syncthreads();
      for (int j = tid; j < E; j += 256) kbuf[j] = sel_tmp[j];
      if (tid == 0) {
        s_kcount = E;
        s_ktau = K;
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int k = 0; k < kDists; ++k) {
    const uint32_t c = (uint32_t)wave_sum_int((int)above[k]);
    if (lane == 0) atomicAdd(&s_above_cnt[k], c);
  }
  if (tid < kDists && s_mode[tid] == MODE_LDS && s_fill[tid] > s_ub[tid]) s_mode[tid] = MODE_GLOBAL;
  if (E > 0) {
    // the E smallest keys are the evicted slots; store them in slot order
    const int cnt = s_kcount;
    const u64 K = block_kth_smallest(kbuf, cnt, E, sel_hist, s_x, tid);
    uint32_t* sel = reinterpret_cast<uint32_t*>(sel_tmp);
    if (tid == 0) s_c2 = 0;
    __syncthreads();
    for (int j = tid; j < cnt; j += 256)
      if (kbuf[j] <= K) sel[atomicAdd(&s_c2, 1)] = (uint32_t)(kbuf[j] & kSlotMask);
    __syncthreads();
    for (int t = tid; t < E; t += 256) {  // E <= 2P <= 512
      const uint32_t s = sel[t];
      int rk = 0;
      for (int j = 0; j < E; ++j) rk += sel[j] < s ? 1 : 0;
      a.sp.ev[u * ev_stride(g.P) + rk] = (int)s;
      if (rk == 0) a.sp.e_unit[u] = (int)s;
    }
  } else if (tid == 0) {
    a.sp.e_unit[u] = n;
  }
  __syncthreads();

  // ---- refinement: rows held in LDS by their wave, the others by the block
  uint32_t* hcnt = reinterpret_cast<uint32_t*>(&ms[0][0]) + wave * 256;  // 4 x 1 KB (rows 0-1)
  u64* hms = &ms[2][0] + wave * 256;                                      // 4 x 2 KB (rows 2-5)
  for (int d2 = 0; d2 < 2; ++d2) {
    const int k = 2 * wave + d2;
    if (s_mode[k] == MODE_LDS) {
      const int Wr = wave_refine_lds(cand + s_off[k], s_fill[k], M[k], s_T[k], s_above[k], s_above_cnt[k],
                                     hcnt, hms, lane, n);
      if (lane == 0) s_W[k] = Wr;
    }
  }
  __syncthreads();
  // Rows refined by the block: their crossing-bin elements are collected into the (now
  // free) LDS candidate buffer by one filtered pass when they fit, and refined there;
  // larger bins are refined in global memory.
  for (int k = 0; k < kDists; ++k) {
    if (s_mode[k] != MODE_GLOBAL) continue;  // block-uniform
    const float Mk = s_M[k];
    if (s_fill[k] <= kCandCap) {
      if (tid == 0) s_c2 = 0;
      __syncthreads();
      const int bk = s_bin[k];
      for (int i = tid; i < n; i += 256) {
        const float v = x[(int64_t)i * kDists + k];
        if (x_bin(Mk - v) == bk) cand[atomicAdd(&s_c2, 1)] = v;
      }
      __syncthreads();
      if (wave == 0) {
        const int Wr = wave_refine_lds(cand, s_c2, Mk, s_T[k], s_above[k], s_above_cnt[k], hcnt, hms, lane, n);
        if (lane == 0) s_W[k] = Wr;
      }
    } else {
      const int Wr = block_refine_global(x + k, n, s_bin[k], Mk, s_T[k], s_above[k], s_above_cnt[k],
                                         reinterpret_cast<uint32_t*>(&ms[0][0]), &ms[2][0], s_red, tid);
      if (tid == 0) s_W[k] = Wr;
    }
    __syncthreads();
  }
  if (real_row) {
    const int k = tid;
    a.ws_out[widx(k)] = s_W[k];
    const float Zf = (float)((double)s_Z[k] / (double)kMassScale);
    a.sp.stats[widx(k) * 2 + 1] = Zf;
    if (a.stats_out) {
      a.stats_out[widx(k) * 2] = M[k];
      a.stats_out[widx(k) * 2 + 1] = Zf;
    }
  }
}

template <int KCAP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void finish_kernel(FinishArgs a) {
  __shared__ FinishLds<KCAP> lds;
  const int upr = a.g.L * a.g.Hkv;
  const int rank = blockIdx.x / upr;
  const int rem = blockIdx.x - rank * upr;
  const int l = rem / a.g.Hkv;
  finish_unit<KCAP>(a, rank, l, rem - l * a.g.Hkv, lds);
}

// The whole scan of one unit per block: the four waves compute the logits of a quarter
// of the unit's 16-token steps each on the matrix cores (logit_mfma.h), staging them in
// the selection's LDS (free until the selection starts) and writing them out in blocks;
// the block combines the row maxima and then selects from those logits while they are
// still in the caches, instead of a second kernel reading them back from HBM.
template <int D, int KCAP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void fused_scan_kernel(ScanArgs s,
                                                                                                FinishArgs f) {
  static_assert(sizeof(FinishLds<KCAP>) >= 4 * kStageBytes, "logit staging exceeds the selection LDS");
  __shared__ FinishLds<KCAP> lds;
  __shared__ float s_mw[4][kDists];
  const Geo& g = s.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform (a scalar register): the logit loop's bounds and page ids derive from it
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int upr = g.L * g.Hkv;
  const int rank = blockIdx.x / upr;
  const int rem = blockIdx.x - rank * upr;
  const int l = rem / g.Hkv;
  const int kvh = rem - l * g.Hkv;
  const int b = s.sp.order[rank];
  if (!s.sp.flags[b]) {
    const int n = s.sp.n_tok[b];
    const int r = g.req_ids[b];
    const int32_t* pt = g.page_table + (int64_t)r * g.max_pages;
    MfmaSummaries<D> A;
    A.load(s, r, l, kvh, lane);
    const int steps = (n + kMfmaTok - 1) / kMfmaTok;
    const int s0 = steps * wave / 4;
    const int s1 = steps * (wave + 1) / 4;
    float* lg = s.sp.logits + (s.sp.tok_off[b] * g.L * g.Hkv + (int64_t)(l * g.Hkv + kvh) * logit_rows(n)) * kDists;
    float* stage = reinterpret_cast<float*>(&lds) + wave * (kStageBytes / sizeof(float));
    f32x4_t mx = mfma_logit_steps<D>(s, A, pt, n, l, kvh, s0, s1, lg, stage, lane);
    // max over the 16 tokens (lanes) of each row group: lanes 0 and 16 end with rows 0..3, 4..7
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = mx[i];
      v = fmaxf(v, __shfl_xor(v, 1, 64));
      v = fmaxf(v, __shfl_xor(v, 2, 64));
      v = fmaxf(v, __shfl_xor(v, 4, 64));
      v = fmaxf(v, __shfl_xor(v, 8, 64));
      mx[i] = v;
    }
    if (lane == 0 || lane == 16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s_mw[wave][4 * (lane >> 4) + i] = mx[i];
    }
    __syncthreads();
    if (tid < kDists && row_real(tid, g.G)) {
      const float m = fmaxf(fmaxf(s_mw[0][tid], s_mw[1][tid]), fmaxf(s_mw[2][tid], s_mw[3][tid]));
      const int h = kvh * g.G + (tid >> 1);
      s.sp.stats[((((int64_t)b * g.L + l) * g.Hq + h) * 2 + (tid & 1)) * 2] = m;
    }
    __syncthreads();  // the unit's logits and maxima are visible to the whole block
  }
  finish_unit<KCAP>(f, rank, l, kvh, lds);
}

// Batches with fewer units than resident blocks (a few requests, or one layer): one block
// per unit would leave most of the chip idle and make each block's walk through a long
// unit a latency chain.  Here a unit's 16-token steps are cut into `parts` contiguous
// ranges, one block (four waves, the fused kernel's steps, staging and logit layout) per
// range; the parts' row maxima meet in the statistics through float atomics (set to -inf
// first), and finish_kernel then selects from the logits.

// Row maxima to -inf for every (entry, layer, query head, summary) of the batch.
__global__ __launch_bounds__(256) void init_max_kernel(ScratchPtrs sp, int64_t rows) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < rows; i += (int64_t)gridDim.x * 256)
    sp.stats[i * 2] = -INFINITY;
}

// Float max through integer atomics: non-negative floats order like their bit patterns
// as signed integers, negative ones in reverse as unsigned integers.  (-0 is made +0
// first, so that it is not taken for the smallest value; a NaN is ignored, as fmaxf
// ignores it in the fused kernel's combine.)
__device__ __forceinline__ void atomic_max_f32(float* p, float v) {
  if (v != v) return;
  v += 0.f;
  if (v >= 0.f)
    atomicMax(reinterpret_cast<int*>(p), __float_as_int(v));
  else
    atomicMin(reinterpret_cast<unsigned*>(p), __float_as_uint(v));
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void split_logit_kernel(ScanArgs s,
                                                                                                 int parts) {
  __shared__ float s_stage[4 * kStageBytes / sizeof(float)];
  __shared__ float s_mw[4][kDists];
  const Geo& g = s.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int unit = blockIdx.x / parts;
  const int part = blockIdx.x - unit * parts;
  const int upr = g.L * g.Hkv;
  const int rank = unit / upr;
  const int rem = unit - rank * upr;
  const int l = rem / g.Hkv;
  const int kvh = rem - l * g.Hkv;
  const int b = s.sp.order[rank];
  if (s.sp.flags[b]) return;
  const int n = s.sp.n_tok[b];
  const int steps = (n + kMfmaTok - 1) / kMfmaTok;
  const int p0 = (int)((int64_t)steps * part / parts);
  const int p1 = (int)((int64_t)steps * (part + 1) / parts);
  if (p0 >= p1) return;  // the whole block: nothing of this unit falls in the part
  const int r = g.req_ids[b];
  const int32_t* pt = g.page_table + (int64_t)r * g.max_pages;
  MfmaSummaries<D> A;
  A.load(s, r, l, kvh, lane);
  const int s0 = p0 + (p1 - p0) * wave / 4;
  const int s1 = p0 + (p1 - p0) * (wave + 1) / 4;
  float* lg = s.sp.logits + (s.sp.tok_off[b] * g.L * g.Hkv + (int64_t)(l * g.Hkv + kvh) * logit_rows(n)) * kDists;
  float* stage = s_stage + wave * (kStageBytes / sizeof(float));
  f32x4_t mx = mfma_logit_steps<D>(s, A, pt, n, l, kvh, s0, s1, lg, stage, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = mx[i];
    v = fmaxf(v, __shfl_xor(v, 1, 64));
    v = fmaxf(v, __shfl_xor(v, 2, 64));
    v = fmaxf(v, __shfl_xor(v, 4, 64));
    v = fmaxf(v, __shfl_xor(v, 8, 64));
    mx[i] = v;
  }
  if (lane == 0 || lane == 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s_mw[wave][4 * (lane >> 4) + i] = mx[i];
  }
  __syncthreads();
  if (tid < kDists && row_real(tid, g.G)) {
    const float m = fmaxf(fmaxf(s_mw[0][tid], s_mw[1][tid]), fmaxf(s_mw[2][tid], s_mw[3][tid]));
    const int h = kvh * g.G + (tid >> 1);
    atomic_max_f32(&s.sp.stats[((((int64_t)b * g.L + l) * g.Hq + h) * 2 + (tid & 1)) * 2], m);
  }
}

}  // namespace

hipError_t launch_split_scan(const ScanArgs& s, const FinishArgs& f, int parts, hipStream_t st) {
  const Geo& g = s.g;
  const int64_t units = (int64_t)g.n_req * g.L * g.Hkv;
  const int64_t rows = (int64_t)g.n_req * g.L * g.Hq * 2;
  hipLaunchKernelGGL(init_max_kernel, dim3((unsigned)std::min<int64_t>((rows + 255) / 256, 1024)), dim3(256), 0,
                     st, s.sp, rows);
  const dim3 grid((unsigned)(units * parts)), block(256);
  if (g.d == 128)
    hipLaunchKernelGGL((split_logit_kernel<128>), grid, block, 0, st, s, parts);
  else
    hipLaunchKernelGGL((split_logit_kernel<64>), grid, block, 0, st, s, parts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_finish(f, st);
}

hipError_t launch_fused_scan(const ScanArgs& s, const FinishArgs& f, hipStream_t st) {
  const int64_t units = (int64_t)f.g.n_req * f.g.L * f.g.Hkv;
  const dim3 grid((unsigned)units), block(256);
  const bool big = keep_cap(f.g.P) != 512;
  if (f.g.d == 128) {
    if (big) hipLaunchKernelGGL((fused_scan_kernel<128, 1024>), grid, block, 0, st, s, f);
    else hipLaunchKernelGGL((fused_scan_kernel<128, 512>), grid, block, 0, st, s, f);
  } else {
    if (big) hipLaunchKernelGGL((fused_scan_kernel<64, 1024>), grid, block, 0, st, s, f);
    else hipLaunchKernelGGL((fused_scan_kernel<64, 512>), grid, block, 0, st, s, f);
  }
  return hipGetLastError();
}

hipError_t launch_finish(const FinishArgs& a, hipStream_t st) {
  const int64_t units = (int64_t)a.g.n_req * a.g.L * a.g.Hkv;
  if (keep_cap(a.g.P) == 512)
    hipLaunchKernelGGL(finish_kernel<512>, dim3((unsigned)units), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(finish_kernel<1024>, dim3((unsigned)units), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace gp
