// Device helpers shared by the kernel files of libgrowpage (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gp {

// DPP lane moves inside a row of 16 lanes (CDNA dpp_ctrl encodings).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7-i within each 8 lanes

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Monotone map float -> uint32 (ascending float = ascending key, -0 < +0).
__device__ __forceinline__ uint32_t ord_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord_key_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// exp(y) for y <= 0 as a 2^-40 fixed-point integer, truncated: exact integer sums
// make the softmax masses and their totals independent of summation order.  The
// hardware exp2 is used directly (results below 2^-40 truncate to 0 anyway, so its
// handling of tiny results does not matter); floor(e * 2^40) is assembled from the
// integer and fractional parts of e * 2^8, both exact in float32.
constexpr float kMassScale = 1099511627776.0f;  // 2^40
__device__ __forceinline__ uint64_t fixed_mass(float y) {
  const float e = __builtin_amdgcn_exp2f(y * 1.4426950408889634f);
  const float h = e * 256.0f;                                   // in [0, 256]
  const uint32_t hi = (uint32_t)h;
  const uint32_t lo = (uint32_t)((h - (float)hi) * 4294967296.0f);
  return ((uint64_t)hi << 32) | lo;
}

// Block-wide exclusive prefix sum for blockDim.x == 256; returns the exclusive prefix of
// `v` and writes the block total to *total.  `tmp` must hold 4 ints.
__device__ __forceinline__ int block_exscan_256(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += tmp[i];
  const int tot = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Same for blockDim.x == 1024 (16 waves); `tmp` holds 16 ints.
__device__ __forceinline__ int block_exscan_1024(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < 16; ++i) {
    if (i < w) base += tmp[i];
    tot += tmp[i];
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ long long wave_sum_i64(long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace gp
