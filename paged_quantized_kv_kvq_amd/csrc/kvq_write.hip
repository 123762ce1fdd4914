// Cache write: quantize new K/V rows and scatter them into the paged pools.
//
// "metrale_model_layers/layers/ops/kv_cache_bf16k_turbov.rs",
// reshape_and_cache_bf16k_turbo{2,3,4}v (slot_mapping scatter of [tokens,
// kv_heads, head_dim] rows); "spark_runtime/kv_cache.rs", KvCacheDtype
// (bf16 copy, fp8 E4M3 with a per-tensor scale, turbo: wht_bf16_inplace then
// Lloyd-Max codes with one E4M3 scale per 16 elements; Turbo8: the same
// rotation, then E4M3 values with one BF16 scale per 16 elements; Nvfp4:
// no rotation, E2M1 nibbles with one E4M3 scale per 16 elements, in turbo4's
// byte layout).
//
// One wave64 writes the K and the V row of one (token, kv head): head_dim/64
// values per lane and side.  Both source rows and the slot are requested
// together (the rows do not depend on the slot), so a wave waits for one
// memory round trip before it computes.  The rotation is done in registers: butterfly strides below the
// per-lane count stay in the lane, the rest are lane-xor exchanges.  Group
// absmax and code packing are lane reductions; nothing touches LDS.
//
// Bit-exactness: every rounding step is a single IEEE fp32 operation in a
// fixed order (file compiled with -ffp-contract=off):
//   butterflies (ascending stride) -> * RN32(1/sqrt(d)) -> round to bf16 ->
//   group absmax -> s = absmax * RN32(1/c_max) -> E4M3(s) = sigma, s_q ->
//   code = #{k : y >= s_q * t_k} -> little-endian bit packing.
// Turbo8 after the rounding to bf16: group absmax -> s = absmax * RN32(1/448)
//   -> bf16(s) = sigma, s_q -> byte = E4M3(y / s_q) (0 for s_q = 0).
#include "kvq_device.h"

namespace kvq {
namespace {

template <int E>
__device__ __forceinline__ void load_bf16(const uint16_t* __restrict__ p, int lane, uint32_t (&raw)[E]) {
  if constexpr (E == 1) {
    raw[0] = p[lane];
  } else if constexpr (E == 2) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(p)[lane];
    raw[0] = w & 0xFFFFu;
    raw[1] = w >> 16;
  } else {
    const uint2 w = reinterpret_cast<const uint2*>(p)[lane];
    raw[0] = w.x & 0xFFFFu;
    raw[1] = w.x >> 16;
    raw[2] = w.y & 0xFFFFu;
    raw[3] = w.y >> 16;
  }
}

// Store E bytes (packed little-endian in `v`) at dst + lane*E.
template <int E>
__device__ __forceinline__ void store_bytes(uint8_t* __restrict__ dst, int lane, uint32_t v) {
  if constexpr (E == 1) dst[lane] = uint8_t(v);
  else if constexpr (E == 2) reinterpret_cast<uint16_t*>(dst)[lane] = uint16_t(v);
  else reinterpret_cast<uint32_t*>(dst)[lane] = v;
}

// The lane's E values of the row after the rotation and the rounding to
// bf16; returns the absmax of the lane's group of 16.
template <int HD>
__device__ __forceinline__ float rotate_row(const uint32_t (&raw)[HD / 64], float (&y)[HD / 64],
                                            const WriteArgs& a, int lane) {
  constexpr int E = HD / 64;
#pragma unroll
  for (int e = 0; e < E; ++e) y[e] = bf16_bits_to_float(raw[e]);
  // in-lane butterflies (stride < E)
#pragma unroll
  for (int h = 1; h < E; h <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if ((e & h) == 0) {
        const float lo = y[e], hi = y[e + h];
        y[e] = lo + hi;
        y[e + h] = lo - hi;
      }
    }
  }
  // cross-lane butterflies: element stride h = m*E pairs lane with lane ^ m
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float other = __shfl_xor(y[e], m);
      y[e] = (lane & m) ? (other - y[e]) : (y[e] + other);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    y[e] = round_to_bf16(y[e] * a.wht_scale);
    amax = fmaxf(amax, fabsf(y[e]));
  }
  return group_max<16 / E>(amax);  // one group of 16 elements = 16/E lanes
}

template <int HD, int BITS>
__device__ __forceinline__ void write_turbo(const uint32_t (&raw)[HD / 64], uint8_t* __restrict__ blk,
                                            uint32_t row, uint64_t data_bytes, const WriteArgs& a,
                                            int lane) {
  constexpr int E = HD / 64;
  constexpr int L = 1 << BITS;
  float y[E];
  const float amax = rotate_row<HD>(raw, y, a, lane);
  const float s = amax * a.cb.inv_cmax[BITS - 2];
  const uint32_t sigma = e4m3_encode(s);
  const float sq = e4m3_decode(sigma);
  float t[L];
#pragma unroll
  for (int k = 1; k < L; ++k) t[k] = sq * a.cb.threshold[BITS - 2][k];
  // pack: a unit of U elements fills whole bytes (4 bytes, or 3 for 3-bit)
  constexpr int U = (BITS == 3) ? 8 : 32 / BITS;
  constexpr int LU = U / E;  // lanes per unit
  uint32_t part = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    uint32_t c = 0;
#pragma unroll
    for (int k = 1; k < L; ++k) c += (y[e] >= t[k]) ? 1u : 0u;
    part |= c << (BITS * ((lane * E + e) % U));
  }
#pragma unroll
  for (int m = 1; m < LU; m <<= 1) part |= uint32_t(__shfl_xor(int(part), m));
  uint8_t* codes = blk + uint64_t(row) * (HD * BITS / 8);
  if ((lane % LU) == 0) {
    const int unit = lane / LU;
    if constexpr (BITS == 3) {
      uint8_t* d = codes + unit * 3;
      d[0] = uint8_t(part);
      d[1] = uint8_t(part >> 8);
      d[2] = uint8_t(part >> 16);
    } else {
      reinterpret_cast<uint32_t*>(codes)[unit] = part;
    }
  }
  if ((lane % (16 / E)) == 0) {
    blk[data_bytes + uint64_t(row) * (HD / 16) + lane / (16 / E)] = uint8_t(sigma);
  }
}

template <int HD>
__device__ __forceinline__ void write_turbo8(const uint32_t (&raw)[HD / 64], uint8_t* __restrict__ blk,
                                             uint32_t row, uint64_t data_bytes, const WriteArgs& a, int lane) {
  constexpr int E = HD / 64;
  constexpr float kInvE4m3Max = 1.0f / 448.0f;  // RN32(1/448)
  float y[E];
  const float amax = rotate_row<HD>(raw, y, a, lane);
  const float s = amax * kInvE4m3Max;
  const float sq = round_to_bf16(s);
  const uint32_t sigma = __float_as_uint(sq) >> 16;
  uint32_t packed = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) packed |= (sq > 0.0f ? e4m3_encode(y[e] / sq) : 0u) << (8 * e);
  store_bytes<E>(blk + uint64_t(row) * HD, lane, packed);
  if ((lane % (16 / E)) == 0) {
    reinterpret_cast<uint16_t*>(blk + data_bytes + uint64_t(row) * (HD / 8))[lane / (16 / E)] = uint16_t(sigma);
  }
}

// NVFP4: no rotation; per group of 16 of the row itself, the E4M3 scale of
// absmax / 6, then the E2M1 nibble of x / scale (IEEE division; a zero
// scale stores zero nibbles), packed as turbo4's codes.
template <int HD>
__device__ __forceinline__ void write_nvfp4(const uint32_t (&raw)[HD / 64], uint8_t* __restrict__ blk,
                                            uint32_t row, uint64_t data_bytes, int lane) {
  constexpr int E = HD / 64;
  constexpr float kInvE2m1Max = 1.0f / 6.0f;  // RN32(1/6)
  constexpr int LU = 8 / E;                    // lanes per 32-bit word of nibbles
  float x[E];
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    x[e] = bf16_bits_to_float(raw[e]);
    amax = fmaxf(amax, fabsf(x[e]));
  }
  amax = group_max<16 / E>(amax);
  const uint32_t sigma = e4m3_encode(amax * kInvE2m1Max);
  const float sq = e4m3_decode(sigma);
  uint32_t part = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t c = sq > 0.0f ? e2m1_encode(x[e] / sq) : 0u;
    part |= c << (4 * ((lane * E + e) % 8));
  }
#pragma unroll
  for (int m = 1; m < LU; m <<= 1) part |= uint32_t(__shfl_xor(int(part), m));
  if ((lane % LU) == 0) reinterpret_cast<uint32_t*>(blk + uint64_t(row) * (HD / 2))[lane / LU] = part;
  if ((lane % (16 / E)) == 0) blk[data_bytes + uint64_t(row) * (HD / 16) + lane / (16 / E)] = uint8_t(sigma);
}

template <int HD>
__device__ __forceinline__ void write_row(int fmt, const uint32_t (&raw)[HD / 64], uint8_t* __restrict__ blk,
                                          uint32_t row, uint64_t data_bytes, float scale,
                                          const WriteArgs& a, int lane) {
  constexpr int E = HD / 64;
  if (fmt == KVQ_BF16) {
    uint8_t* dst = blk + uint64_t(row) * HD * 2;
    if constexpr (E == 1) reinterpret_cast<uint16_t*>(dst)[lane] = uint16_t(raw[0]);
    else if constexpr (E == 2) reinterpret_cast<uint32_t*>(dst)[lane] = raw[0] | (raw[1] << 16);
    else reinterpret_cast<uint2*>(dst)[lane] = make_uint2(raw[0] | (raw[1] << 16), raw[2] | (raw[3] << 16));
  } else if (fmt == KVQ_FP8_E4M3) {
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) packed |= e4m3_encode(bf16_bits_to_float(raw[e]) / scale) << (8 * e);
    store_bytes<E>(blk + uint64_t(row) * HD, lane, packed);
  } else if (fmt == KVQ_TURBO2) {
    write_turbo<HD, 2>(raw, blk, row, data_bytes, a, lane);
  } else if (fmt == KVQ_TURBO3) {
    write_turbo<HD, 3>(raw, blk, row, data_bytes, a, lane);
  } else if (fmt == KVQ_TURBO4) {
    write_turbo<HD, 4>(raw, blk, row, data_bytes, a, lane);
  } else if (fmt == KVQ_NVFP4) {
    write_nvfp4<HD>(raw, blk, row, data_bytes, lane);
  } else {
    write_turbo8<HD>(raw, blk, row, data_bytes, a, lane);
  }
}

// Work item w = (token, kv head) and, with SIDES, w = (token, kv head, side)
// with the side fastest; one wave per item writes its row of each side.  A
// wave that writes both sides waits for one round trip for two rows, which
// pays on large writes; a small write (every wave resident at once) finishes
// sooner with one side per wave, two shorter chains in parallel.
template <int HD, bool SIDES>
__global__ __launch_bounds__(256) void write_kernel(const WriteArgs a) {
  constexpr int E = HD / 64;
  constexpr uint32_t per_item = SIDES ? 2u : 1u;
  const uint32_t item = blockIdx.x * 4u + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (item >= a.num_tokens * a.num_kv_heads * per_item) return;
  const uint32_t th = item / per_item;  // (token, kv head)
  const uint32_t t = th / a.num_kv_heads;
  const uint32_t h = th - t * a.num_kv_heads;
  const uint16_t* ksrc = a.key + uint64_t(t) * a.key_stride + h * HD;
  const uint16_t* vsrc = a.value + uint64_t(t) * a.value_stride + h * HD;
  const int64_t slot = a.slots[t];
  // The empty asm statements read the loaded values: the compiler must issue
  // the loads before them, and does not move the row loads below the branch
  // on the slot.
  if constexpr (SIDES) {
    const bool vside = (item & 1u) != 0;
    uint32_t raw[E];
    load_bf16<E>(vside ? vsrc : ksrc, lane, raw);
    asm volatile("" ::"v"(raw[0]), "v"(uint32_t(slot)));
    if (slot < 0) return;
    const uint64_t blk = uint64_t(slot) >> a.log2_bs;
    const uint32_t row = (uint32_t(slot) & ((1u << a.log2_bs) - 1u)) * a.num_kv_heads + h;
    if (!vside) write_row<HD>(a.k_format, raw, a.k_cache + blk * a.k_stride, row, a.k_data, a.k_scale, a, lane);
    else write_row<HD>(a.v_format, raw, a.v_cache + blk * a.v_stride, row, a.v_data, a.v_scale, a, lane);
  } else {
    uint32_t kraw[E], vraw[E];
    load_bf16<E>(ksrc, lane, kraw);
    load_bf16<E>(vsrc, lane, vraw);
    asm volatile("" ::"v"(kraw[0]), "v"(vraw[0]), "v"(uint32_t(slot)));
    if (slot < 0) return;
    const uint64_t blk = uint64_t(slot) >> a.log2_bs;
    const uint32_t row = (uint32_t(slot) & ((1u << a.log2_bs) - 1u)) * a.num_kv_heads + h;
    write_row<HD>(a.k_format, kraw, a.k_cache + blk * a.k_stride, row, a.k_data, a.k_scale, a, lane);
    write_row<HD>(a.v_format, vraw, a.v_cache + blk * a.v_stride, row, a.v_data, a.v_scale, a, lane);
  }
}

// Writes of at most this many (token, kv head) rows take one wave per side.
constexpr uint64_t kSplitSidesRows = 2048;

}  // namespace

hipError_t launch_write(int head_dim, const WriteArgs& a, hipStream_t st) {
  const uint64_t rows = uint64_t(a.num_tokens) * a.num_kv_heads;
  const bool sides = rows <= kSplitSidesRows;
  const uint64_t items = rows * (sides ? 2u : 1u);
  const dim3 grid(uint32_t((items + 3) / 4)), block(256);
  switch (head_dim * 2 + (sides ? 1 : 0)) {
    case 128: hipLaunchKernelGGL((write_kernel<64, false>), grid, block, 0, st, a); break;
    case 129: hipLaunchKernelGGL((write_kernel<64, true>), grid, block, 0, st, a); break;
    case 256: hipLaunchKernelGGL((write_kernel<128, false>), grid, block, 0, st, a); break;
    case 257: hipLaunchKernelGGL((write_kernel<128, true>), grid, block, 0, st, a); break;
    case 512: hipLaunchKernelGGL((write_kernel<256, false>), grid, block, 0, st, a); break;
    case 513: hipLaunchKernelGGL((write_kernel<256, true>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
