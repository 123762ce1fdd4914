// Device-side building blocks shared by the write and decode kernels (gfx950,
// wave64).  Host code does not include this file.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {

constexpr int kWave = 64;

// ---------------------------------------------------------------- scalar codecs

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> nearest bf16 value (ties to even), returned widened to fp32.
// Adding 0x7FFF plus the last kept bit carries into the kept half exactly when
// the discarded half is above 0x8000, or equal to it with an odd kept half.
__device__ __forceinline__ float round_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return __uint_as_float(u & 0xFFFF0000u);
}

// fp32 -> OCP E4M3FN byte: saturate to +-448, round to nearest, ties to even,
// subnormals (multiples of 2^-9) kept, sign of -0 kept.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);
  const uint32_t ua = __float_as_uint(a);
  const int e = int(ua >> 23) - 127;
  uint32_t code;
  if (e < -6) {
    // below the smallest normal 2^-6: a multiple of 2^-9; a*512 is exact and
    // rintf rounds half to even
    code = uint32_t(rintf(a * 512.0f));
  } else {
    const uint32_t mant = ua & 0x7FFFFFu;
    const uint32_t keep = mant >> 20;          // 3 mantissa bits
    const uint32_t rest = mant & 0xFFFFFu;     // 20 discarded bits
    const uint32_t up = (rest > 0x80000u) | ((rest == 0x80000u) & (keep & 1u));
    code = (uint32_t(e + 7) << 3) + keep + up; // a carry moves into the exponent
  }
  return code | sign;
}

// fp32 -> OCP E2M1 nibble (NVFP4's element): saturate to +-6, round to
// nearest, ties to even, sign of -0 kept.  Each binade of the grid is an
// evenly spaced set (steps 0.5 below 2, 1 in [2, 4), 2 in [4, 6]); scaled to
// integers there (exactly), rintf rounds half to even, and an even grid
// index is an even mantissa.  Index q of a binade maps to nibble q, q + 2,
// q + 4.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 28) & 0x8u;
  const float a = fminf(fabsf(v), 6.0f);
  uint32_t mag;
  if (a < 2.0f) mag = uint32_t(rintf(a * 2.0f));
  else if (a < 4.0f) mag = uint32_t(rintf(a)) + 2u;
  else mag = uint32_t(rintf(a * 0.5f)) + 4u;
  return mag | sign;
}

// E4M3FN byte -> fp32 value (NaN codes are never produced by the encoder).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : float(m) * 0.001953125f;
  return (c & 0x80u) ? -mag : mag;
}

// ---------------------------------------------------------------- cross-lane sums

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N = 1..64, power of two); every lane of
// a group receives the group's sum.  Within a row of 16 lanes DPP does the
// exchange (quad permutes, half-row and row mirrors); across rows a swizzle.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp_mov<0x141>(x);   // row_half_mirror
  if constexpr (N >= 16) x += dpp_mov<0x140>(x);  // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp_mov<0xB1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp_mov<0x4E>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp_mov<0x141>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp_mov<0x140>(x));
  if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (N >= 64) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

// ---------------------------------------------------------------- launch mapping

// Workgroups are handed to the 8 XCDs round-robin (workgroup i runs on XCD
// i % 8, each XCD with its own L2).  A tile is a (unit, kv head) pair, a unit
// being a (sequence, split).  All kv heads of a unit go to one XCD, dispatched
// back to back, so they share the L2 lines their interleaved rows live in;
// consecutive units rotate over the XCDs, which keeps the XCDs evenly loaded
// when sequence lengths differ.  The grid has ceil(units/8)*8*heads
// workgroups; the padding ones get valid == false.
__device__ __forceinline__ bool xcd_unit_tile(uint32_t i, uint32_t nunits, uint32_t nheads, uint32_t& unit,
                                              uint32_t& head) {
  const uint32_t x = i & 7u, rest = i >> 3;
  head = rest % nheads;
  unit = (rest / nheads) * 8u + x;
  return unit < nunits;
}

}  // namespace kvq
