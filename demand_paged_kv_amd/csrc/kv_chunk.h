// Row slices of the paged K/V pools as a lane loads them: with 16 lanes per token row,
// lane j (0..15) owns the D/16 contiguous elements [j*D/16, (j+1)*D/16) of the row.
// Shared by the scan and the decode-attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gp {
namespace {

template <bool BF16, int D>
struct Chunk;  // the D/16 elements a lane owns in one row, as raw bits

template <>
struct Chunk<true, 128> {  // 8 bf16 = 16 B
  uint4 c;
};
template <>
struct Chunk<true, 64> {  // 4 bf16 = 8 B
  uint2 c;
};
template <>
struct Chunk<false, 64> {  // 4 f32 = 16 B
  uint4 c;
};
template <>
struct Chunk<false, 128> {  // 8 f32 = 32 B
  uint4 c, c2;
};

template <bool BF16, int D>
__device__ __forceinline__ void load_chunk(Chunk<BF16, D>& c, const char* row, int j) {
  constexpr int EL = D / 16;
  constexpr int E = BF16 ? 2 : 4;
  const char* p = row + (size_t)j * EL * E;
  if constexpr (BF16 && D == 64) {
    c.c = *reinterpret_cast<const uint2*>(p);
  } else if constexpr (!BF16 && D == 128) {
    c.c = *reinterpret_cast<const uint4*>(p);
    c.c2 = *reinterpret_cast<const uint4*>(p + 16);
  } else {
    c.c = *reinterpret_cast<const uint4*>(p);
  }
}

__device__ __forceinline__ void unpack_bf16x2(uint32_t w, float& lo, float& hi) {
  lo = __uint_as_float(w << 16);
  hi = __uint_as_float(w & 0xffff0000u);
}

template <bool BF16, int D>
__device__ __forceinline__ void unpack_chunk(const Chunk<BF16, D>& c, float* kf) {
  if constexpr (BF16 && D == 128) {
    unpack_bf16x2(c.c.x, kf[0], kf[1]);
    unpack_bf16x2(c.c.y, kf[2], kf[3]);
    unpack_bf16x2(c.c.z, kf[4], kf[5]);
    unpack_bf16x2(c.c.w, kf[6], kf[7]);
  } else if constexpr (BF16 && D == 64) {
    unpack_bf16x2(c.c.x, kf[0], kf[1]);
    unpack_bf16x2(c.c.y, kf[2], kf[3]);
  } else if constexpr (!BF16 && D == 64) {
    kf[0] = __uint_as_float(c.c.x);
    kf[1] = __uint_as_float(c.c.y);
    kf[2] = __uint_as_float(c.c.z);
    kf[3] = __uint_as_float(c.c.w);
  } else {
    kf[0] = __uint_as_float(c.c.x);
    kf[1] = __uint_as_float(c.c.y);
    kf[2] = __uint_as_float(c.c.z);
    kf[3] = __uint_as_float(c.c.w);
    kf[4] = __uint_as_float(c.c2.x);
    kf[5] = __uint_as_float(c.c2.y);
    kf[6] = __uint_as_float(c.c2.z);
    kf[7] = __uint_as_float(c.c2.w);
  }
}

}  // namespace
}  // namespace gp
