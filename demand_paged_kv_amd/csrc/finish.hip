// Working sets and keep-sets of one boundary batch, from the logits the scan wrote.
// (GrowPage review on evolve.pub, "Summary": Top-p attention working-set sizes of the
// two summaries; compaction keeps the slots with the maximum of both importance scores;
// FAQ "Is GrowPage's code available?": local retention quota.)
//
// One 256-thread block per (entry, layer, KV head) unit, two reads of the unit's logits
// ([n][8] float32, token-major, written by the logit kernel with each row's max M; a
// thread loads a token's 8 logits as two 16-byte vectors, two tokens at a time):
//
//   read 1  x = M - l >= 0 for every element of every row; elements with x < 255/16 go
//           to 255 bins of width 1/16 (count + softmax mass exp(-x) in 2^-40 fixed
//           point, LDS atomics), the rest only add their mass to a per-thread tail sum.
//           Integer sums make the normaliser Z exact and order-independent.  Bins are
//           walked from x = 0 (largest probabilities) until the mass reaches
//           T = ceil(top_p * Z): that bin holds the W-th element.
//   read 2  the elements of each row's crossing bin are gathered into LDS; in the same
//           pass the slot importance max_k exp(l_k - M_k) / Z_k feeds a threshold
//           buffer that keeps the n - k least important candidate slots (ties: older
//           slot first), i.e. the slots a compaction evicts.
//   refine  per row, an exact radix select over the crossing-bin elements only (one
//           wave per row), weighted by the same fixed-point masses, gives
//           W = (elements above the bin) + (elements of the bin needed to reach T).
//
// A crossing beyond the binned range (possible only when the W-th probability is below
// exp(-255/16), i.e. inside the near-tie band) or a crossing bin larger than the LDS
// candidate buffer falls back to the same radix select over the whole row in global
// memory.  All decisions are exact for the float32 logits the scan produced.
#include "device_util.h"
#include "gp_internal.h"

namespace gp {
namespace {

typedef unsigned long long u64;

constexpr int kXBins = 255;          // bins of width 1/16 covering x in [0, 255/16)
constexpr float kBinsPerNat = 16.0f;
constexpr int kCandCap = 4096;       // crossing-bin elements held in LDS (all 8 rows)
constexpr int kKeepCap = 512;        // threshold buffer of keep-set candidates

enum { MODE_DONE = 0, MODE_LDS = 1, MODE_GLOBAL = 2 };

__device__ __forceinline__ int x_bin(float xv) {
  const float f = xv * kBinsPerNat;
  return f < (float)kXBins ? (int)f : kXBins;  // kXBins = beyond the bins
}

__device__ __forceinline__ u64 wave_exscan_u64(u64 v, int lane, u64* total) {
  u64 x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const u64 y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  *total = __shfl(x, 63, 64);
  return x - v;
}

__device__ __forceinline__ uint32_t wave_exscan_u32(uint32_t v, int lane) {
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x - v;
}

// Walk 256 bins (lane l owns 4 consecutive bins in walk order; DESC walks bin 255 first)
// accumulating mass from (base_mass, base_cnt) and return the first bin where the
// accumulated mass reaches T, with the mass and count strictly before it.
template <bool DESC>
__device__ __forceinline__ bool wave_find_crossing(const uint32_t* cnt, const u64* ms, u64 base_mass,
                                                   uint32_t base_cnt, u64 T, int lane, int* chosen,
                                                   u64* mass_before, uint32_t* cnt_before,
                                                   u64* total_mass) {
  u64 m4[4];
  uint32_t c4[4];
  u64 ls = 0;
  uint32_t lc = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int bin = DESC ? 255 - (4 * lane + q) : 4 * lane + q;
    m4[q] = ms[bin];
    c4[q] = cnt[bin];
    ls += m4[q];
    lc += c4[q];
  }
  u64 tot = 0;
  u64 acc = base_mass + wave_exscan_u64(ls, lane, &tot);
  uint32_t ac = base_cnt + wave_exscan_u32(lc, lane);
  *total_mass = tot;
  int my = -1;
  u64 my_m = 0;
  uint32_t my_c = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (my < 0) {
      if (c4[q] > 0 && acc + m4[q] >= T) {
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
  *chosen = __shfl(my, f, 64);
  *mass_before = __shfl(my_m, f, 64);
  *cnt_before = __shfl(my_c, f, 64);
  return true;
}

// Exact weighted radix select run by one wave over m logits of one row: keys descending,
// (acc_cnt, acc_mass) already hold the elements above the range.  All four waves of the
// block call it the same number of times (inactive waves pass active = false) because it
// synchronises the block between passes.  Returns W on lane 0's view (uniform).
__device__ int wave_radix_refine(bool active, const float* src, int stride, int m, float M, u64 T,
                                 u64 acc_mass, uint32_t acc_cnt, uint32_t* hcnt, u64* hms, int lane,
                                 int n) {
  uint32_t prefix = 0, mask = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (active)
      for (int q = lane; q < 256; q += 64) {
        hcnt[q] = 0;
        hms[q] = 0;
      }
    __syncthreads();
    if (active)
      for (int c = lane; c < m; c += 64) {
        const float v = src[(int64_t)c * stride];
        const uint32_t key = ord_key(v);
        if ((key & mask) == prefix) {
          const uint32_t bin = (key >> shift) & 255u;
          atomicAdd(&hcnt[bin], 1u);
          atomicAdd(&hms[bin], (u64)fixed_mass(v - M));
        }
      }
    __syncthreads();
    if (active) {
      int chosen = 0;
      u64 mb = acc_mass, tot = 0;
      uint32_t cb = acc_cnt;
      if (wave_find_crossing<true>(hcnt, hms, acc_mass, acc_cnt, T, lane, &chosen, &mb, &cb, &tot)) {
        acc_mass = mb;
        acc_cnt = cb;
        prefix |= (uint32_t)chosen << shift;
        mask |= 255u << shift;
      } else {
        // unreachable when T <= the range mass; keep the widest answer
        prefix |= 0u;
        mask |= 255u << shift;
      }
    }
    __syncthreads();
  }
  if (!active) return 0;
  const float vstar = ord_key_inv(prefix);
  const u64 q = fixed_mass(vstar - M);
  const u64 need = T > acc_mass ? T - acc_mass : 0;
  const u64 jn = q ? (need + q - 1) / q : 1ull;
  return (int)min((u64)n, (u64)acc_cnt + max(jn, 1ull));
}

__device__ void bitonic_sort_512(u64* a, int tid) {
  for (int size = 2; size <= kKeepCap; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int lo = 2 * tid - (tid & (stride - 1));
      const int hi = lo + stride;
      const bool asc = (lo & size) == 0;
      const u64 x = a[lo], y = a[hi];
      if ((x > y) == asc) {
        a[lo] = y;
        a[hi] = x;
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(256) void finish_kernel(FinishArgs a) {
  const Geo& g = a.g;
  __shared__ uint32_t cnt[kDists][256];
  __shared__ u64 ms[kDists][256];
  __shared__ float cand[kCandCap];
  __shared__ u64 kbuf[kKeepCap];
  __shared__ float s_M[kDists], s_iz[kDists];
  __shared__ u64 s_tail[kDists], s_T[kDists], s_above[kDists], s_Z[kDists];
  __shared__ uint32_t s_above_cnt[kDists];
  __shared__ int s_mode[kDists], s_bin[kDists], s_off[kDists], s_cn[kDists], s_fill[kDists], s_W[kDists];
  __shared__ int s_kcount;
  __shared__ u64 s_ktau;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int upr = g.L * g.Hkv;
  const int rank = blockIdx.x / upr;
  const int rem = blockIdx.x - rank * upr;
  const int l = rem / g.Hkv;
  const int kvh = rem - l * g.Hkv;
  const int b = a.sp.order[rank];
  const int64_t u = ((int64_t)b * g.L + l) * g.Hkv + kvh;
  auto widx = [&](int k) { return (((int64_t)b * g.L + l) * g.Hq + kvh * kGroup + (k >> 1)) * 2 + (k & 1); };
  if (a.sp.flags[b]) {
    if (tid < kDists) a.ws_out[widx(tid)] = -1;
    return;
  }
  const int n = a.sp.n_tok[b];
  const int r = g.req_ids[b];
  const int kk = g.n_alloc[r] * g.P;                  // slots a compaction keeps
  const int E = min(max(n - kk, 0), g.P);             // slots it evicts (fill <= P)
  const int nl = min(max(a.n_local, 0), min(kk, n));
  const int cand_slots = n - nl;
  const int64_t ubase = (a.sp.tok_off[b] * g.L * g.Hkv + (int64_t)(l * g.Hkv + kvh) * n) * kDists;
  const float* x = a.sp.logits + ubase;

  if (n == 0) {
    if (tid < kDists) {
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

  // ---- read 1: x-bins and the tail mass
  for (int i = tid; i < kDists * 256; i += 256) {
    (&cnt[0][0])[i] = 0;
    (&ms[0][0])[i] = 0;
  }
  if (tid < kDists) {
    s_M[tid] = a.sp.stats[widx(tid) * 2];
    s_tail[tid] = 0;
  }
  __syncthreads();
  float M[kDists];
#pragma unroll
  for (int k = 0; k < kDists; ++k) M[k] = s_M[k];
  u64 tail[kDists];
#pragma unroll
  for (int k = 0; k < kDists; ++k) tail[k] = 0;
  for (int i0 = tid; i0 < n; i0 += 512) {
    float v[2][kDists];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int i = i0 + 256 * t;
      float4 lo = make_float4(0.f, 0.f, 0.f, 0.f), hi = lo;
      if (i < n) {
        lo = *reinterpret_cast<const float4*>(x + (int64_t)i * kDists);
        hi = *reinterpret_cast<const float4*>(x + (int64_t)i * kDists + 4);
      }
      v[t][0] = lo.x; v[t][1] = lo.y; v[t][2] = lo.z; v[t][3] = lo.w;
      v[t][4] = hi.x; v[t][5] = hi.y; v[t][6] = hi.z; v[t][7] = hi.w;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (i0 + 256 * t >= n) break;
#pragma unroll
      for (int k = 0; k < kDists; ++k) {
        const float xv = M[k] - v[t][k];
        const u64 q = fixed_mass(-xv);
        const int bin = x_bin(xv);
        if (bin < kXBins) {
          atomicAdd(&cnt[k][bin], 1u);
          atomicAdd(&ms[k][bin], q);
        } else {
          tail[k] += q;
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kDists; ++k) {
    u64 t = tail[k];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
    if (lane == 0) atomicAdd(&s_tail[k], t);
  }
  __syncthreads();

  // ---- crossing bin of each row (wave w: rows 2w, 2w+1)
  for (int d2 = 0; d2 < 2; ++d2) {
    const int k = 2 * wave + d2;
    int chosen = 0;
    u64 mb = 0, tot = 0;
    uint32_t cb = 0;
    // total first (T depends on it)
    u64 ls = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) ls += ms[k][4 * lane + q];
    u64 tot_bins = 0;
    wave_exscan_u64(ls, lane, &tot_bins);
    const u64 Z = tot_bins + s_tail[k];
    u64 T = 0;
    int mode = MODE_LDS, W = 0;
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
    bool found = false;
    if (mode == MODE_LDS)
      found = wave_find_crossing<false>(&cnt[k][0], &ms[k][0], 0, 0, T, lane, &chosen, &mb, &cb, &tot);
    if (lane == 0) {
      if (mode == MODE_LDS && !found) mode = MODE_GLOBAL;
      s_mode[k] = mode;
      s_W[k] = W;
      s_T[k] = T;
      s_Z[k] = Z;
      s_bin[k] = chosen;
      s_above[k] = mb;
      s_above_cnt[k] = cb;
      s_cn[k] = (mode == MODE_LDS) ? (int)cnt[k][chosen] : 0;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int off = 0;
    for (int k = 0; k < kDists; ++k) {
      s_fill[k] = 0;
      if (s_mode[k] != MODE_LDS) continue;
      if (off + s_cn[k] <= kCandCap) {
        s_off[k] = off;
        off += s_cn[k];
      } else {
        s_mode[k] = MODE_GLOBAL;
      }
    }
    s_kcount = 0;
    s_ktau = ~0ull;
  }
  if (tid < kDists) {
    const double z = (double)s_Z[tid] / (double)kMassScale;
    s_iz[tid] = (float)(1.0 / z);
  }
  __syncthreads();

  // ---- read 2: crossing-bin elements and keep-set candidates
  int mode[kDists], binstar[kDists];
  float iz[kDists];
#pragma unroll
  for (int k = 0; k < kDists; ++k) {
    mode[k] = s_mode[k];
    binstar[k] = s_bin[k];
    iz[k] = s_iz[k];
  }
  for (int base = 0; base < n; base += 256) {
    const int i = base + tid;
    if (i < n) {
      const float4 lo = *reinterpret_cast<const float4*>(x + (int64_t)i * kDists);
      const float4 hi = *reinterpret_cast<const float4*>(x + (int64_t)i * kDists + 4);
      const float v8[kDists] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      float imp = 0.f;
#pragma unroll
      for (int k = 0; k < kDists; ++k) {
        const float v = v8[k];
        const float xv = M[k] - v;
        if (mode[k] == MODE_LDS && x_bin(xv) == binstar[k]) {
          const int p = atomicAdd(&s_fill[k], 1);
          cand[s_off[k] + p] = v;
        }
        imp = fmaxf(imp, exp2f(-xv * kLog2e) * iz[k]);
      }
      if (E > 0 && i < cand_slots) {
        const u64 key = ((u64)__float_as_uint(imp) << 32) | (uint32_t)i;
        if (key < s_ktau) kbuf[atomicAdd(&s_kcount, 1)] = key;
      }
    }
    __syncthreads();
    if (s_kcount > 256) {
      for (int j = s_kcount + tid; j < kKeepCap; j += 256) kbuf[j] = ~0ull;
      __syncthreads();
      bitonic_sort_512(kbuf, tid);
      if (tid == 0) {
        s_kcount = E;
        s_ktau = kbuf[E - 1];
      }
      __syncthreads();
    }
  }
  if (E > 0) {
    for (int j = s_kcount + tid; j < kKeepCap; j += 256) kbuf[j] = ~0ull;
    __syncthreads();
    bitonic_sort_512(kbuf, tid);
    // the E smallest keys are the evicted slots; store them in slot order
    if (tid < E) {
      const uint32_t s = (uint32_t)(kbuf[tid] & 0xffffffffu);
      int rk = 0;
      for (int j = 0; j < E; ++j) rk += (uint32_t)(kbuf[j] & 0xffffffffu) < s ? 1 : 0;
      a.sp.ev[u * g.P + rk] = (int)s;
      if (rk == 0) a.sp.e_unit[u] = (int)s;
    }
  } else if (tid == 0) {
    a.sp.e_unit[u] = n;
  }
  __syncthreads();

  // ---- exact refinement (wave w: rows 2w, 2w+1); the histogram space is free now
  for (int d2 = 0; d2 < 2; ++d2) {
    const int k = 2 * wave + d2;
    const int md = s_mode[k];
    const bool act = md != MODE_DONE;
    const bool glob = md == MODE_GLOBAL;
    const float* src = glob ? x + k : cand + (act ? s_off[k] : 0);
    const int m = glob ? n : (act ? s_cn[k] : 0);
    const int Wr = wave_radix_refine(act, src, glob ? kDists : 1, m, M[k], s_T[k], glob ? 0ull : s_above[k],
                                     glob ? 0u : s_above_cnt[k], &cnt[2 * wave][0], &ms[2 * wave][0],
                                     lane, n);
    if (lane == 0) {
      const int W = act ? Wr : s_W[k];
      a.ws_out[widx(k)] = W;
      const float Zf = (float)((double)s_Z[k] / (double)kMassScale);
      a.sp.stats[widx(k) * 2 + 1] = Zf;
      if (a.stats_out) {
        a.stats_out[widx(k) * 2] = M[k];
        a.stats_out[widx(k) * 2 + 1] = Zf;
      }
    }
  }
}

}  // namespace

hipError_t launch_finish(const FinishArgs& a, hipStream_t st) {
  const int64_t units = (int64_t)a.g.n_req * a.g.L * a.g.Hkv;
  hipLaunchKernelGGL(finish_kernel, dim3((unsigned)units), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace gp
