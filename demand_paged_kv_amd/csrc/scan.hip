// Boundary scan: logits of both summaries against every retained key, per-head softmax
// statistics and the Top-p attention working-set size of each summary.
// (GrowPage review on evolve.pub, "Summary": the decision weighs the Top-p working set
// of the fast summary against that of the slow one, both summaries kept before RoPE.)
//
// plan_kernel    1 block: candidate slots n of every batch entry, scratch offsets and a
//                longest-first order of the entries.
// Then, for bf16 keys in pages of a multiple of 16 tokens, fused_scan_kernel (finish.hip):
// one block per (entry, layer, KV head) "unit" computes the unit's logits on the matrix
// cores (logit_mfma.h) and selects from them; a batch of at most kSplitUnits units runs
// the same logit steps split over several blocks per unit (split_logit_kernel) and then
// finish_kernel.  Otherwise two kernels:
//   logit_kernel   one wave per unit, launched longest-first.  The wave streams the
//                  unit's K rows through the page table once; 16 lanes share a token row
//                  (each holds D/16 contiguous elements), every lane keeps the matching
//                  slices of all 8 rotated summaries (4 query-head slots x 2 timescales) in
//                  registers, and a DPP transpose-reduce (3 steps within each 8-lane half,
//                  one across the halves) leaves lane j with the logit of summary j mod 8
//                  for its token.  Logits go to the scratch ([unit][n'][8] float32, n'
//                  = n rounded up to 16: one wave step writes 128 contiguous bytes), the
//                  running max to the statistics.
//   finish_kernel  one block per unit (finish.hip): exact Top-p working sets of the 8
//                  logit rows and the unit's keep-set, from two reads of the logits.
#include <algorithm>

#include "device_util.h"
#include "gp_internal.h"
#include "kv_chunk.h"

namespace gp {
namespace {

// ----------------------------------------------------------------------------- plan
constexpr int kPlanLds = 8192;

__global__ __launch_bounds__(1024) void plan_kernel(ScanArgs a) {
  __shared__ int tmp[16];
  __shared__ long long carry_s, carry_pad_s;
  __shared__ int nvals[kPlanLds];
  const int tid = threadIdx.x;
  const Geo& g = a.g;
  if (tid == 0) carry_s = carry_pad_s = 0;
  __syncthreads();
  // An entry overflows when the candidate tokens up to and including it exceed
  // max_tokens; its logit rows start at the padded running sum (logit_rows), which the
  // scratch sizes for max_tokens plus the padding of every entry.
  for (int base = 0; base < g.n_req; base += 1024) {
    const int b = base + tid;
    int n = 0;
    if (b < g.n_req) {
      const int r = g.req_ids[b];
      n = g.n_alloc[r] * g.P + g.fill[r];
    }
    int total = 0, total_pad = 0;
    const int ex = block_exscan_1024(n, tmp, &total);  // fits int: per chunk < 2^31 tokens
    const int ex_pad = block_exscan_1024((int)logit_rows(n), tmp, &total_pad);
    const long long off = carry_s + ex;
    const long long off_pad = carry_pad_s + ex_pad;
    if (b < g.n_req) {
      const bool over = off + n > a.max_tokens;
      a.sp.tok_off[b] = over ? 0 : off_pad;
      a.sp.n_tok[b] = over ? 0 : n;
      a.sp.flags[b] = over ? GP_REQ_OVERFLOW : 0;
      if (b < kPlanLds) nvals[b] = over ? -1 : n;
    }
    __syncthreads();
    if (tid == 0) {
      carry_s += total;
      carry_pad_s += total_pad;
    }
    __syncthreads();
  }
  // Longest-first order (rank sort, ties by batch index) so long units start first.
  if (g.n_req <= kPlanLds) {
    for (int b = tid; b < g.n_req; b += 1024) {
      const int nb = nvals[b];
      int rank = 0;
      for (int c = 0; c < g.n_req; ++c) {
        const int nc = nvals[c];
        rank += (nc > nb) || (nc == nb && c < b);
      }
      a.sp.order[rank] = b;
    }
  } else {
    for (int b = tid; b < g.n_req; b += 1024) a.sp.order[b] = b;
  }
}

// ----------------------------------------------------------------------------- logits
// 16 lanes share a token row: lane j (0..15) owns the D/16 contiguous elements
// [j*D/16, (j+1)*D/16), so one wave step covers 4 tokens of one page.
constexpr int kTokPerStep = 4;
#ifndef GP_SCAN_BATCH
#define GP_SCAN_BATCH 8
#endif
constexpr int kScanBatch = GP_SCAN_BATCH;  // steps whose loads are in flight together

// Summary index held in register slot i by lane j of an 8-lane group: slots 0..3 hold
// j^i and slots 4..7 hold j^7^i, so that the reduce steps (pairs j<->j^7 by half-row
// mirror, then j<->j^2, then j<->j^1) always add a partner's slot holding the same
// summary and lane j finishes with summary j.
__device__ __forceinline__ int slot_dist(int j, int i) { return i < 4 ? (j ^ i) : (j ^ 7 ^ (i - 4)); }

constexpr int kDppRowRor8 = 0x128;  // lane i <- lane (i + 8) mod 16 within each row of 16

// One step = 4 tokens of one page.  Accumulate the 8 scores of this lane's slice of its
// token, transpose-reduce them within each 8-lane half (lane j&7 ends with summary j&7)
// and add the other half of the row.
template <bool BF16, int D>
__device__ __forceinline__ float step_scores(const Chunk<BF16, D>& c, const float (&qr)[8][D / 16]) {
  constexpr int EL = D / 16;
  float kf[EL];
  unpack_chunk<BF16, D>(c, kf);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < EL; ++e) s = __builtin_fmaf(qr[i][e], kf[e], s);
    acc[i] = s;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] += dpp_mov<kDppHalfMirror>(acc[i + 4]);
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i] += dpp_mov<kDppQuadXor2>(acc[i + 2]);
  acc[0] += dpp_mov<kDppQuadXor1>(acc[1]);
  acc[0] += dpp_mov<kDppRowRor8>(acc[0]);
  return acc[0];
}

template <bool BF16, int D, int U>
__global__ __launch_bounds__(64) void logit_kernel(ScanArgs a) {
#pragma clang fp contract(off)
  constexpr int EL = D / 16;
  constexpr int E = BF16 ? 2 : 4;
  constexpr int TS = kTokPerStep;
  const Geo& g = a.g;
  const int lane = threadIdx.x;
  const int tl = lane >> 4;      // token of the step
  const int j = lane & 15;       // element slice
  const int js = lane & 7;       // summary this lane ends a step with
  const int upr = g.L * g.Hkv;
  const int rank = blockIdx.x / upr;
  const int rem = blockIdx.x - rank * upr;
  const int l = rem / g.Hkv;
  const int kvh = rem - l * g.Hkv;
  const int b = a.sp.order[rank];
  if (a.sp.flags[b]) return;
  const int n = a.sp.n_tok[b];
  const int r = g.req_ids[b];
  const int32_t* pt = g.page_table + (int64_t)r * g.max_pages;

  // Rotate the 8 summaries to the request position (rotate-half pairs c, c + D/2) and
  // fold in 1/sqrt(d); lane j keeps elements [j*EL, (j+1)*EL) of each.
  float qr[8][EL];
  const bool rope = a.rope_cos != nullptr;
  const int pos = rope ? min(max(a.pos[r], 0), a.rope_max_pos - 1) : 0;
  const bool first_half = j * EL < D / 2;
  const int c0 = (j * EL) & (D / 2 - 1);   // pair index of this lane's first element
  float cs[EL], sn[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) {
    cs[e] = rope ? a.rope_cos[(int64_t)pos * (D / 2) + c0 + e] : 1.f;
    sn[e] = rope ? a.rope_sin[(int64_t)pos * (D / 2) + c0 + e] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int dist = slot_dist(js, i);
    const float* s = ((dist & 1) ? a.sum_l : a.sum_s) +
                     (((int64_t)r * g.L + l) * g.Hq + kvh * g.G + row_head(dist, g.G)) * D;
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      const float x1 = s[c0 + e];
      const float x2 = s[D / 2 + c0 + e];
      qr[i][e] = first_half ? (x1 * cs[e] - x2 * sn[e]) * a.scale : (x2 * cs[e] + x1 * sn[e]) * a.scale;
    }
  }

  const int64_t unit_base =
      (a.sp.tok_off[b] * g.L * g.Hkv + (int64_t)(l * g.Hkv + kvh) * logit_rows(n)) * kDists;
  float* lg = a.sp.logits + unit_base + js + tl * kDists;  // token-major: [n][8]
  const bool writer = j < 8;
  const char* kb = reinterpret_cast<const char*>(g.k) + ((int64_t)l * g.s_layer + (int64_t)kvh * g.s_head) * E +
                   (int64_t)tl * g.s_tok * E;
  const int64_t page_bytes = g.s_page * E;
  const int64_t tok_bytes = g.s_tok * E;
  float m = -INFINITY;

  // Full batches of U steps, loads of the next batch issued before this one is reduced.
  // Page index and in-page offset are wave-uniform, so page ids come in by scalar loads,
  // fetched one batch ahead of the row loads that use them (indexes clamped to the
  // request's pages, so the look-ahead past the last batch stays in bounds).
  const int nfull = (n / (TS * U)) * (TS * U);
  const int npages = (n + g.P - 1) / g.P;
  int pj = 0, sub = 0;  // page index and in-page offset of the next step to load
  int fq = 0, fs = 0;   // the same for the next page-id fetch
  int pid[U];
  auto fetch_pids = [&]() {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      pid[u] = pt[min(fq, npages - 1)];
      fs += TS;
      if (fs == g.P) {
        fs = 0;
        ++fq;
      }
    }
  };
  auto load_batch = [&](Chunk<BF16, D>(&c)[U], const int (&ids)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const char* row = kb + (int64_t)ids[u] * page_bytes + (int64_t)sub * tok_bytes;
      load_chunk<BF16, D>(c[u], row, j);
      sub += TS;
      if (sub == g.P) {
        sub = 0;
        ++pj;
      }
    }
  };
  Chunk<BF16, D> cur[U], nxt[U];
  if (nfull > 0) {
    fetch_pids();
    int ids[U];
#pragma unroll
    for (int u = 0; u < U; ++u) ids[u] = pid[u];
    load_batch(cur, ids);
    fetch_pids();
  }
  for (int t0 = 0; t0 < nfull; t0 += TS * U) {
    if (t0 + TS * U < nfull) {
      int ids[U];
#pragma unroll
      for (int u = 0; u < U; ++u) ids[u] = pid[u];
      load_batch(nxt, ids);
      fetch_pids();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float x = step_scores<BF16, D>(cur[u], qr);
      if (writer) lg[(int64_t)(t0 + TS * u) * kDists] = x;
      m = fmaxf(m, x);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = nxt[u];
  }
  // Tail: single steps, the last one possibly partial.
  for (int t0 = nfull; t0 < n; t0 += TS) {
    Chunk<BF16, D> c{};
    const bool ok = t0 + tl < n;
    if (ok) load_chunk<BF16, D>(c, kb + (int64_t)pt[pj] * page_bytes + (int64_t)sub * tok_bytes, j);
    sub += TS;
    if (sub == g.P) {
      sub = 0;
      ++pj;
    }
    const float x = step_scores<BF16, D>(c, qr);
    if (ok) {
      if (writer) lg[(int64_t)t0 * kDists] = x;
      m = fmaxf(m, x);
    }
  }
  m = fmaxf(m, __shfl_xor(m, 16, 64));
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  if (lane < 8 && row_real(js, g.G)) {
    const int h = kvh * g.G + (js >> 1);
    const int64_t si = ((((int64_t)b * g.L + l) * g.Hq + h) * 2 + (js & 1)) * 2;
    a.sp.stats[si] = m;
  }
}

template <bool BF16, int D>
hipError_t launch_logits(const ScanArgs& a, int64_t units, hipStream_t st) {
  hipLaunchKernelGGL((logit_kernel<BF16, D, kScanBatch>), dim3((unsigned)units), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan(const Geo& g, const ScratchPtrs& sp, int64_t max_tokens,
                       const float* sum_s, const float* sum_l, const float* rope_cos,
                       const float* rope_sin, int32_t rope_max_pos, const int32_t* pos,
                       float top_p, int32_t n_local, int32_t shrink, int32_t* ws_out,
                       float* stats_out, hipStream_t st) {
  ScanArgs a;
  a.g = g;
  a.sp = sp;
  a.max_tokens = max_tokens;
  a.sum_s = sum_s;
  a.sum_l = sum_l;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.rope_max_pos = rope_max_pos;
  a.pos = pos;
  a.scale = (float)(1.0 / sqrt((double)g.d));
  a.ws_out = ws_out;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t units = (int64_t)g.n_req * g.L * g.Hkv;
  FinishArgs f{g, sp, top_p, n_local, shrink, ws_out, stats_out};
  if (g.dtype == GP_BF16 && g.P % kFusedPageMultiple == 0) {
    // Fewer units than the 1024 fused blocks resident at once (4 per CU): split each unit
    // into parts so that about 1024 blocks stream K, at most 8 parts per unit.
    if (units <= kSplitUnits) return launch_split_scan(a, f, (int)std::min<int64_t>(8, 1024 / units), st);
    return launch_fused_scan(a, f, st);
  }
  if (g.dtype == GP_BF16) {
    e = g.d == 128 ? launch_logits<true, 128>(a, units, st) : launch_logits<true, 64>(a, units, st);
  } else {
    e = g.d == 128 ? launch_logits<false, 128>(a, units, st) : launch_logits<false, 64>(a, units, st);
  }
  if (e != hipSuccess) return e;
  return launch_finish(f, st);
}

// ----------------------------------------------------------------------------- logit read-back
// Copy of batch entry `entry`'s logits from the scratch of the last scan: block u = l *
// Hkv + g writes out[l][g][t][8] for t < n (NaN where the scan held no row: t >= the
// entry's candidate count, or an entry over the token budget).
__global__ __launch_bounds__(256) void copy_logits_kernel(ScratchPtrs sp, int32_t L, int32_t Hkv, int32_t entry,
                                                          int32_t n, float* out) {
  const int u = blockIdx.x;
  const int nt = sp.flags[entry] ? 0 : sp.n_tok[entry];
  const float* src = sp.logits + (sp.tok_off[entry] * L * Hkv + (int64_t)u * logit_rows(nt)) * kDists;
  float* dst = out + (int64_t)u * n * kDists;
  for (int64_t i = threadIdx.x; i < (int64_t)n * kDists; i += 256)
    dst[i] = i < (int64_t)nt * kDists ? src[i] : __builtin_nanf("");
}

hipError_t launch_copy_logits(const Geo& g, const ScratchPtrs& sp, int32_t entry, int32_t n, float* out,
                              hipStream_t st) {
  hipLaunchKernelGGL(copy_logits_kernel, dim3((unsigned)(g.L * g.Hkv)), dim3(256), 0, st, sp, g.L, g.Hkv, entry,
                     n, out);
  return hipGetLastError();
}

}  // namespace gp
