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

// Order the LDS accesses of one wave without a block barrier.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- wave64 prefix scans and reductions on DPP lane moves (no LDS traffic).  Each
// step moves a value within rows of 16 lanes (row_shr) or from the last lane of one row
// to the following rows (row_bcast15 / row_bcast31); lanes a step does not write keep
// the identity passed as `old`.  Call with all 64 lanes active.
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v, uint64_t old = 0) {
  const uint32_t lo = dpp_u32<CTRL, ROW_MASK>((uint32_t)old, (uint32_t)v);
  const uint32_t hi = dpp_u32<CTRL, ROW_MASK>((uint32_t)(old >> 32), (uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Inclusive prefix sums over lanes 0..63.
__device__ __forceinline__ uint32_t wave_incl_sum_u32(uint32_t x) {
  x += dpp_u32<kDppRowShr1, 0xF>(0u, x);
  x += dpp_u32<kDppRowShr2, 0xF>(0u, x);
  x += dpp_u32<kDppRowShr4, 0xF>(0u, x);
  x += dpp_u32<kDppRowShr8, 0xF>(0u, x);
  x += dpp_u32<kDppRowBcast15, 0xA>(0u, x);
  x += dpp_u32<kDppRowBcast31, 0xC>(0u, x);
  return x;
}
__device__ __forceinline__ uint64_t wave_incl_sum_u64(uint64_t x) {
  x += dpp_u64<kDppRowShr1, 0xF>(x);
  x += dpp_u64<kDppRowShr2, 0xF>(x);
  x += dpp_u64<kDppRowShr4, 0xF>(x);
  x += dpp_u64<kDppRowShr8, 0xF>(x);
  x += dpp_u64<kDppRowBcast15, 0xA>(x);
  x += dpp_u64<kDppRowBcast31, 0xC>(x);
  return x;
}
// Value of lane `lane` (wave-uniform) in every lane.
__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int lane) {
  return ((uint64_t)lane_u32((uint32_t)(v >> 32), lane) << 32) | lane_u32((uint32_t)v, lane);
}
// Minimum / maximum over the wave (prefix min/max, then lane 63).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  constexpr uint32_t I = 0xffffffffu;
  x = min(x, dpp_u32<kDppRowShr1, 0xF>(I, x));
  x = min(x, dpp_u32<kDppRowShr2, 0xF>(I, x));
  x = min(x, dpp_u32<kDppRowShr4, 0xF>(I, x));
  x = min(x, dpp_u32<kDppRowShr8, 0xF>(I, x));
  x = min(x, dpp_u32<kDppRowBcast15, 0xA>(I, x));
  x = min(x, dpp_u32<kDppRowBcast31, 0xC>(I, x));
  return lane_u32(x, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u32<kDppRowShr1, 0xF>(0u, x));
  x = max(x, dpp_u32<kDppRowShr2, 0xF>(0u, x));
  x = max(x, dpp_u32<kDppRowShr4, 0xF>(0u, x));
  x = max(x, dpp_u32<kDppRowShr8, 0xF>(0u, x));
  x = max(x, dpp_u32<kDppRowBcast15, 0xA>(0u, x));
  x = max(x, dpp_u32<kDppRowBcast31, 0xC>(0u, x));
  return lane_u32(x, 63);
}

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t x) {
  constexpr uint64_t I = ~0ull;
  x = min(x, dpp_u64<kDppRowShr1, 0xF>(x, I));
  x = min(x, dpp_u64<kDppRowShr2, 0xF>(x, I));
  x = min(x, dpp_u64<kDppRowShr4, 0xF>(x, I));
  x = min(x, dpp_u64<kDppRowShr8, 0xF>(x, I));
  x = min(x, dpp_u64<kDppRowBcast15, 0xA>(x, I));
  x = min(x, dpp_u64<kDppRowBcast31, 0xC>(x, I));
  return lane_u64(x, 63);
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  x = max(x, dpp_u64<kDppRowShr1, 0xF>(x));
  x = max(x, dpp_u64<kDppRowShr2, 0xF>(x));
  x = max(x, dpp_u64<kDppRowShr4, 0xF>(x));
  x = max(x, dpp_u64<kDppRowShr8, 0xF>(x));
  x = max(x, dpp_u64<kDppRowBcast15, 0xA>(x));
  x = max(x, dpp_u64<kDppRowBcast31, 0xC>(x));
  return lane_u64(x, 63);
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
