// Summary update: S <- beta_s*S + (1-beta_s)*q and L <- beta_l*L + (1-beta_l)*q
// (GrowPage review on evolve.pub, "Summary": two moving averages of the queries, taken
// before RoPE; FAQ "Is GrowPage's code available?": factors 0.9 and 0.999).
//
// Float32, each product and the sum rounded on their own (no contraction), so the
// result is bit-identical to any IEEE implementation of the same expression.  Pure
// streaming: per element 2 (bf16) or 4 (fp32) bytes of q plus 16 bytes of summary
// traffic; one thread per 4 consecutive elements, 16-byte summary accesses.
#include "gp_internal.h"

namespace gp {
namespace {

__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__global__ __launch_bounds__(256) void ema_kernel(const void* __restrict__ q, int32_t q_dtype,
                                                  int64_t sr, int64_t sl, int64_t sh,
                                                  const int32_t* __restrict__ req_ids, int32_t L,
                                                  int32_t Hq, int32_t d, float* __restrict__ S,
                                                  float* __restrict__ Lg, float bs, float obs,
                                                  float bl, float obl, int64_t total4) {
#pragma clang fp contract(off)
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total4) return;
  const int32_t d4 = d >> 2;
  const int32_t e = (int32_t)(i % d4) * 4;
  int64_t t = i / d4;
  const int32_t h = (int32_t)(t % Hq);
  t /= Hq;
  const int32_t l = (int32_t)(t % L);
  const int32_t b = (int32_t)(t / L);
  const int64_t qo = (int64_t)b * sr + (int64_t)l * sl + (int64_t)h * sh + e;
  float qv[4];
  if (q_dtype == GP_BF16) {
    const uint2 raw = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(q) + qo);
    qv[0] = bf16_to_f32(raw.x & 0xffffu);
    qv[1] = bf16_to_f32(raw.x >> 16);
    qv[2] = bf16_to_f32(raw.y & 0xffffu);
    qv[3] = bf16_to_f32(raw.y >> 16);
  } else {
    const float4 raw = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(q) + qo);
    qv[0] = raw.x;
    qv[1] = raw.y;
    qv[2] = raw.z;
    qv[3] = raw.w;
  }
  const int32_t r = req_ids[b];
  const int64_t so = (((int64_t)r * L + l) * Hq + h) * d + e;
  float4 s = *reinterpret_cast<const float4*>(S + so);
  float4 g = *reinterpret_cast<const float4*>(Lg + so);
  s.x = bs * s.x + obs * qv[0];
  s.y = bs * s.y + obs * qv[1];
  s.z = bs * s.z + obs * qv[2];
  s.w = bs * s.w + obs * qv[3];
  g.x = bl * g.x + obl * qv[0];
  g.y = bl * g.y + obl * qv[1];
  g.z = bl * g.z + obl * qv[2];
  g.w = bl * g.w + obl * qv[3];
  *reinterpret_cast<float4*>(S + so) = s;
  *reinterpret_cast<float4*>(Lg + so) = g;
}

}  // namespace

hipError_t launch_ema(const void* q, int32_t q_dtype, int64_t sr, int64_t sl, int64_t sh,
                      const int32_t* req_ids, int32_t n_req, int32_t L, int32_t Hq, int32_t d,
                      float* sum_s, float* sum_l, float beta_s, float beta_l, hipStream_t st) {
  const int64_t total4 = (int64_t)n_req * L * Hq * (d / 4);
  if (total4 == 0) return hipSuccess;
  // (1 - beta) formed in float32 on the host, exactly as the expression states.
  volatile float one = 1.0f;
  const float obs = one - beta_s;
  const float obl = one - beta_l;
  const int64_t blocks = (total4 + 255) / 256;
  hipLaunchKernelGGL(ema_kernel, dim3((unsigned)blocks), dim3(256), 0, st, q, q_dtype, sr, sl, sh,
                     req_ids, L, Hq, d, sum_s, sum_l, beta_s, obs, beta_l, obl, total4);
  return hipGetLastError();
}

}  // namespace gp
