// Decode attention over the paged cache: the consumer of the pages the boundary engine
// rewrites (GrowPage review on evolve.pub, abstract and FAQ "How does GrowPage differ
// from Zipage?": the engine sits inside PagedAttention serving, next to the decode
// kernel that reads the compacted pages).
//
// One wave per (entry, layer, KV head) unit serves the unit's G <= 4 query heads (4 slots;
// with G < 4 the spare slots repeat the last head and are not written).  Like the
// scan, 16 lanes share a token row (lane j holds D/16 contiguous elements of K and V)
// and a wave step covers 4 tokens of one page.  Each lane keeps the slices of the 4
// rotated queries (pre-scaled by log2(e)/sqrt(d)), a 16-lane butterfly of DPP rotations
// gives every lane of a token its 4 scores, and each token slot (lanes 16t..16t+15)
// runs its own online softmax over the tokens it sees -- running max, running sum and
// the weighted sum of its V slice.  The four slots are merged at the end.
#include "device_util.h"
#include "gp_internal.h"
#include "kv_chunk.h"

namespace gp {
namespace {

constexpr int kDppRowRor1 = 0x121;
constexpr int kDppRowRor2 = 0x122;
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

// Sum over the 16 lanes of a row: lane i adds lanes i+8, then +4, +2, +1 (mod 16).
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<kDppRowRor8>(x);
  x += dpp_mov<kDppRowRor4>(x);
  x += dpp_mov<kDppRowRor2>(x);
  x += dpp_mov<kDppRowRor1>(x);
  return x;
}

struct AttnArgs {
  Geo g;
  const void* q;
  int64_t q_sr, q_sl, q_sh;  // element strides of q
  const float* rope_cos;
  const float* rope_sin;
  int32_t rope_max_pos;
  const int32_t* pos;
  float scale;               // log2(e) / sqrt(d)
  float* out;                // [n_req][L][Hq][d]
};

template <bool BF16, int D, bool QBF16>
__global__ __launch_bounds__(64) void attn_kernel(AttnArgs a) {
#pragma clang fp contract(off)
  constexpr int EL = D / 16;
  constexpr int E = BF16 ? 2 : 4;
  constexpr int TS = 4;
  const Geo& g = a.g;
  const int lane = threadIdx.x;
  const int tl = lane >> 4;
  const int j = lane & 15;
  const int upr = g.L * g.Hkv;
  const int b = blockIdx.x / upr;
  const int rem = blockIdx.x - b * upr;
  const int l = rem / g.Hkv;
  const int kvh = rem - l * g.Hkv;
  const int r = g.req_ids[b];
  const int n = g.n_alloc[r] * g.P + g.fill[r];
  const int32_t* pt = g.page_table + (int64_t)r * g.max_pages;

  // rotated, pre-scaled query slices of the 4 heads
  float qr[kGroup][EL];
  const bool rope = a.rope_cos != nullptr;
  const int pos = rope ? min(max(a.pos[r], 0), a.rope_max_pos - 1) : 0;
  const bool first_half = j * EL < D / 2;
  const int c0 = (j * EL) & (D / 2 - 1);
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    // slots beyond the group (G < 4) repeat its last head; only real heads are written
    const int64_t qo = (int64_t)b * a.q_sr + (int64_t)l * a.q_sl + (int64_t)(kvh * g.G + min(h, g.G - 1)) * a.q_sh;
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      float x1, x2;
      if constexpr (QBF16) {
        const uint16_t* q16 = reinterpret_cast<const uint16_t*>(a.q) + qo;
        x1 = __uint_as_float((uint32_t)q16[c0 + e] << 16);
        x2 = __uint_as_float((uint32_t)q16[D / 2 + c0 + e] << 16);
      } else {
        const float* q32 = reinterpret_cast<const float*>(a.q) + qo;
        x1 = q32[c0 + e];
        x2 = q32[D / 2 + c0 + e];
      }
      const float cs = rope ? a.rope_cos[(int64_t)pos * (D / 2) + c0 + e] : 1.f;
      const float sn = rope ? a.rope_sin[(int64_t)pos * (D / 2) + c0 + e] : 0.f;
      qr[h][e] = first_half ? (x1 * cs - x2 * sn) * a.scale : (x2 * cs + x1 * sn) * a.scale;
    }
  }

  float m[kGroup], ls[kGroup], acc[kGroup][EL];
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    m[h] = -INFINITY;
    ls[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EL; ++e) acc[h][e] = 0.f;
  }
  const int64_t hoff = ((int64_t)l * g.s_layer + (int64_t)kvh * g.s_head) * E + (int64_t)tl * g.s_tok * E;
  const char* kb = reinterpret_cast<const char*>(g.k) + hoff;
  const char* vb = reinterpret_cast<const char*>(g.v) + hoff;
  const int64_t page_bytes = g.s_page * E;
  const int64_t tok_bytes = g.s_tok * E;
  int pj = 0, sub = 0;
  for (int t0 = 0; t0 < n; t0 += TS) {
    const bool ok = t0 + tl < n;
    const int64_t ro = (int64_t)pt[pj] * page_bytes + (int64_t)sub * tok_bytes;
    Chunk<BF16, D> ck{}, cv{};
    if (ok) {
      load_chunk<BF16, D>(ck, kb + ro, j);
      load_chunk<BF16, D>(cv, vb + ro, j);
    }
    sub += TS;
    if (sub == g.P) {
      sub = 0;
      ++pj;
    }
    float kf[EL], vf[EL];
    unpack_chunk<BF16, D>(ck, kf);
    unpack_chunk<BF16, D>(cv, vf);
    float s[kGroup];
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      float x = 0.f;
#pragma unroll
      for (int e = 0; e < EL; ++e) x = __builtin_fmaf(qr[h][e], kf[e], x);
      s[h] = row16_sum(x);
    }
    if (ok) {
#pragma unroll
      for (int h = 0; h < kGroup; ++h) {
        const float mn = fmaxf(m[h], s[h]);
        const float c = __builtin_amdgcn_exp2f(m[h] - mn);  // 0 on the first token
        const float p = __builtin_amdgcn_exp2f(s[h] - mn);
        ls[h] = ls[h] * c + p;
#pragma unroll
        for (int e = 0; e < EL; ++e) acc[h][e] = acc[h][e] * c + p * vf[e];
        m[h] = mn;
      }
    }
  }
  // merge the 4 token slots (lanes j, j+16, j+32, j+48 hold the same elements)
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    float M = fmaxf(m[h], __shfl_xor(m[h], 16, 64));
    M = fmaxf(M, __shfl_xor(M, 32, 64));
    const float c = m[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[h] - M);
    float lsum = ls[h] * c;
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      float x = acc[h][e] * c;
      x += __shfl_xor(x, 16, 64);
      x += __shfl_xor(x, 32, 64);
      acc[h][e] = x * inv;
    }
  }
  if (tl == 0) {
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      if (h >= g.G) break;
      float* o = a.out + ((((int64_t)b * g.L + l) * g.Hq) + kvh * g.G + h) * D + j * EL;
#pragma unroll
      for (int e = 0; e < EL; ++e) o[e] = acc[h][e];
    }
  }
}

template <bool BF16, int D>
hipError_t launch_attn_t(const AttnArgs& a, int32_t q_dtype, unsigned units, hipStream_t st) {
  if (q_dtype == GP_BF16)
    hipLaunchKernelGGL((attn_kernel<BF16, D, true>), dim3(units), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((attn_kernel<BF16, D, false>), dim3(units), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_attention(const Geo& g, const void* q, int32_t q_dtype, int64_t sr, int64_t sl,
                                   int64_t sh, const float* rope_cos, const float* rope_sin,
                                   int32_t rope_max_pos, const int32_t* pos, float* out,
                                   hipStream_t st) {
  AttnArgs a;
  a.g = g;
  a.q = q;
  a.q_sr = sr;
  a.q_sl = sl;
  a.q_sh = sh;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.rope_max_pos = rope_max_pos;
  a.pos = pos;
  a.scale = (float)(1.4426950408889634 / sqrt((double)g.d));
  a.out = out;
  const unsigned units = (unsigned)((int64_t)g.n_req * g.L * g.Hkv);
  if (g.dtype == GP_BF16)
    return g.d == 128 ? launch_attn_t<true, 128>(a, q_dtype, units, st)
                      : launch_attn_t<true, 64>(a, q_dtype, units, st);
  return g.d == 128 ? launch_attn_t<false, 128>(a, q_dtype, units, st)
                    : launch_attn_t<false, 64>(a, q_dtype, units, st);
}

}  // namespace gp
