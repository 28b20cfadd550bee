// Logits of a unit's 8 rotated summaries against its bf16 key rows on the matrix cores
// (pages of a multiple of 16 tokens).  Used by the fused scan kernel (finish.hip), whose
// four waves each take a contiguous range of 16-token steps of the unit.
//
// A step is 16 tokens of one page and one v_mfma_f32_16x16x32_bf16 per 32-element slice
// of d and per part: A = the 8 rotated, scaled summaries (rows 8..15 zero), B = the 16
// key rows.  Each float32 summary element is the exact sum of three bf16 parts (hi = its
// top 8 significant bits, mid = the next 8 of the remainder, lo = the rest, each split
// an exact subtraction), bf16 x bf16 products are exact in float32 and the matrix core
// sums in float32, so the logits carry float32 accumulation error only, like an FMA
// chain.  Lane layout (16x16x32): A lane l holds row l%16, elements 8(l/16)..+8 of the
// slice; B lane l holds column (token) l%16, the same elements; D lane l holds token
// l%16, rows 4(l/16)..+4, so lanes 0..31 end a step with the 8 logits of their token.
#pragma once

#include "device_util.h"
#include "gp_internal.h"

namespace gp {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kMfmaTok = 16;
// Logits are staged in LDS and written out every kStageSteps steps: on this target loads
// and stores share one completion counter, so a store in flight turns the next wait for
// a key load into a wait for everything outstanding (staging measured 1-5% faster than a
// store per step).  One more step of room holds the range's partial last step.
constexpr int kStageSteps = 16;
constexpr int kStageBytes = (kStageSteps + 1) * kMfmaTok * kDists * 4;

__device__ __forceinline__ uint32_t bf16_trunc_bits(float x) { return __float_as_uint(x) >> 16; }

// The 8 summaries of (entry r, layer l, KV head kvh) as A operands: row `col` (< 8) is
// summary 2 * (query head in group) + timescale, rotated to the request position (pairs
// c, c + D/2, both held by this lane since slices k and k + KS/2 are D/2 apart), scaled
// by 1/sqrt(d) and split in three bf16 parts.
template <int D>
struct MfmaSummaries {
  static constexpr int KS = D / 32;
  bf16x8_t hi[KS], mid[KS], lo[KS];

  __device__ __forceinline__ void load(const ScanArgs& a, int r, int l, int kvh, int lane) {
#pragma clang fp contract(off)
    const Geo& g = a.g;
    const int col = lane & 15;
    const int q = lane >> 4;
    float x[KS][8];
    const bool real = col < kDists;
    const bool rope = a.rope_cos != nullptr;
    const int pos = rope ? min(max(a.pos[r], 0), a.rope_max_pos - 1) : 0;
    const float* s = ((col & 1) ? a.sum_l : a.sum_s) +
                     (((int64_t)r * g.L + l) * g.Hq + kvh * g.G + row_head(col & 7, g.G)) * D;
#pragma unroll
    for (int k = 0; k < KS / 2; ++k) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 32 * k + 8 * q + e;  // pair index, < D/2
        const float x1 = real ? s[c] : 0.f;
        const float x2 = real ? s[c + D / 2] : 0.f;
        const float cs = rope ? a.rope_cos[(int64_t)pos * (D / 2) + c] : 1.f;
        const float sn = rope ? a.rope_sin[(int64_t)pos * (D / 2) + c] : 0.f;
        x[k][e] = (x1 * cs - x2 * sn) * a.scale;
        x[k + KS / 2][e] = (x2 * cs + x1 * sn) * a.scale;
      }
    }
#pragma unroll
    for (int k = 0; k < KS; ++k) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t h = bf16_trunc_bits(x[k][e]);
        const float r1 = x[k][e] - __uint_as_float(h << 16);
        const uint32_t m = bf16_trunc_bits(r1);
        const float r2 = r1 - __uint_as_float(m << 16);
        const uint32_t lw = bf16_trunc_bits(r2);  // r2 has at most 8 significant bits
        hi[k][e] = __builtin_bit_cast(__bf16, (uint16_t)h);
        mid[k][e] = __builtin_bit_cast(__bf16, (uint16_t)m);
        lo[k][e] = __builtin_bit_cast(__bf16, (uint16_t)lw);
      }
    }
  }

  // The 16 x 16 logit tile of one step from this lane's key slices.
  __device__ __forceinline__ f32x4_t scores(const uint4 (&kr)[KS]) const {
    f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const bf16x8_t bk = __builtin_bit_cast(bf16x8_t, kr[k]);
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi[k], bk, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mid[k], bk, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo[k], bk, c2, 0, 0, 0);
    }
    return (c0 + c1) + c2;
  }
};

// Steps [s0, s1) (16 tokens each) of a unit with n candidate slots: logits to lg_unit
// ([logit_rows(n)][8], token-major; lanes 0..31 put each step's tile in `stage`, the
// whole wave writes the stage out), returns this lane's running max
// of its 4 rows (-inf if it saw no token).  Two key buffers alternate: the next step's
// rows load while the current one is on the matrix cores, with no register copies
// between them (a copy would wait for the loads in flight).  A step never crosses a
// page, so its page id is wave-uniform; ids are fetched two steps ahead (clamped to the
// request's pages).
template <int D>
__device__ __forceinline__ f32x4_t mfma_logit_steps(const ScanArgs& a, const MfmaSummaries<D>& A,
                                                    const int32_t* pt, int n, int l, int kvh, int s0,
                                                    int s1, float* lg_unit, float* stage, int lane) {
  constexpr int KS = D / 32;
  const Geo& g = a.g;
  const int col = lane & 15;
  const int q = lane >> 4;
  const bool writer = lane < 32;
  const char* kb = reinterpret_cast<const char*>(g.k) + ((int64_t)l * g.s_layer + (int64_t)kvh * g.s_head) * 2 +
                   (int64_t)col * g.s_tok * 2 + (int64_t)q * 16;
  const int64_t page_bytes = g.s_page * 2;
  const int64_t tok_bytes = g.s_tok * 2;
  f32x4_t mx = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  const int npages = (n + g.P - 1) / g.P;
  const int t_beg = s0 * kMfmaTok;
  const int t_last = min(s1 * kMfmaTok, n);
  const int nfs = t_last > t_beg ? (t_last - t_beg) / kMfmaTok : 0;  // full steps
  int ld_sub = t_beg % g.P;                      // in-page offset of the next step to load
  int f_pg = t_beg / g.P, f_sub = ld_sub;        // position of the next page-id fetch
  // The scan never writes the page table, so its ids are read through the constant
  // address space: scalar loads, counted apart from the key loads.
  typedef const __attribute__((address_space(4))) int32_t* const_ids;
  const const_ids ptc = (const_ids)pt;
  auto fetch = [&]() {
    const int v = ptc[min(f_pg, npages - 1)];
    f_sub += kMfmaTok;
    if (f_sub == g.P) {
      f_sub = 0;
      ++f_pg;
    }
    return v;
  };
  // Key rows are read once: non-temporal loads let them leave the caches first, ahead of
  // the logits the block reads back (measured 2% faster scans on long contexts).
  typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
  auto load = [&](uint4 (&kr)[KS], int pid) {
    const char* row = kb + (int64_t)pid * page_bytes + (int64_t)ld_sub * tok_bytes;
#pragma unroll
    for (int k = 0; k < KS; ++k)
      kr[k] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(row + k * 64)));
    ld_sub += kMfmaTok;
    if (ld_sub == g.P) ld_sub = 0;
  };
  int st_t0 = t_beg;  // first token held in the stage
  int st_n = 0;       // steps held
  // Copy the staged tokens [st_t0, st_t0 + ntok) to the unit's logits, then wait for the
  // stores so that no store is in flight during the following key loads.
  auto flush = [&](int ntok) {
    wave_lds_sync();
    float* dst = lg_unit + (int64_t)st_t0 * kDists;
    for (int j = lane; j < ntok * 2; j += 64)
      *reinterpret_cast<f32x4_t*>(dst + 4 * j) = *reinterpret_cast<const f32x4_t*>(stage + 4 * j);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    wave_lds_sync();
    st_t0 += ntok;
    st_n = 0;
  };
  auto emit = [&](const uint4 (&kr)[KS]) {
    const f32x4_t x = A.scores(kr);
    if (writer) *reinterpret_cast<f32x4_t*>(stage + (st_n * kMfmaTok + col) * kDists + 4 * q) = x;
    ++st_n;
#pragma unroll
    for (int i = 0; i < 4; ++i) mx[i] = fmaxf(mx[i], x[i]);
  };
  uint4 ka[KS], kc[KS];
  int p_odd = 0, p_even = 0;  // page ids of the next odd / even step to load
  if (nfs > 0) {
    p_even = fetch();  // step 0
    p_odd = fetch();   // step 1
    load(ka, p_even);
    p_even = fetch();  // step 2
  }
  // ka holds step i in flight, p_odd is step i+1's page, p_even step i+2's.  The loop
  // body loads unconditionally (steps i+1 and i+2 exist), so every iteration has the
  // same loads in flight and each wait covers only the buffer about to be used.
  int i = 0;
  for (; i + 2 < nfs; i += 2) {
    load(kc, p_odd);
    p_odd = fetch();  // step i+3
    emit(ka);
    load(ka, p_even);
    p_even = fetch();  // step i+4
    emit(kc);
    if (st_n == kStageSteps) flush(kStageSteps * kMfmaTok);
  }
  if (i + 1 < nfs) {  // at most kStageSteps - 2 steps are staged here
    load(kc, p_odd);
    emit(ka);
    emit(kc);
  } else if (i < nfs) {
    emit(ka);
  }
  // The unit's last step when partial: missing rows read as zero; they are staged but
  // neither written out nor counted.
  const int tp = t_beg + kMfmaTok * nfs;
  if (tp < t_last) {
    uint4 kr[KS];
    const bool ok = tp + col < n;
    const int pg = tp / g.P;
#pragma unroll
    for (int k = 0; k < KS; ++k) kr[k] = make_uint4(0u, 0u, 0u, 0u);
    if (ok) {
      const char* row = kb + (int64_t)pt[pg] * page_bytes + (int64_t)(tp - pg * g.P) * tok_bytes;
#pragma unroll
      for (int k = 0; k < KS; ++k) kr[k] = *reinterpret_cast<const uint4*>(row + k * 64);
    }
    const f32x4_t x = A.scores(kr);
    if (writer) *reinterpret_cast<f32x4_t*>(stage + (st_n * kMfmaTok + col) * kDists + 4 * q) = x;
    ++st_n;
    if (ok) {
#pragma unroll
      for (int i = 0; i < 4; ++i) mx[i] = fmaxf(mx[i], x[i]);
    }
  }
  if (st_n > 0) flush(t_last - st_t0);
  return mx;
}

}  // namespace
}  // namespace gp
