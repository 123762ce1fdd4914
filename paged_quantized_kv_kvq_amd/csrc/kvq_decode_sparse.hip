// Decode kernels that depend only on the V side: the sparse-V pass (which
// writes the output, or its parts' sums and then their merge) and the dense
// path's merge (log-sum-exp over splits, with the inverse rotation of a
// rotated V side); and the row map of chunked prefill run as decode rows.
#include "kvq_decode.h"

namespace kvq {
namespace {

template <int VF, int HD>
hipError_t sparse_g(int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  const dim3 grid(nwg), block(kVWaves * kWave);
  switch (g) {
    case 1: hipLaunchKernelGGL((sparse_v_kernel<VF, HD, 1>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((sparse_v_kernel<VF, HD, 2>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((sparse_v_kernel<VF, HD, 4>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((sparse_v_kernel<VF, HD, 8>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int VF>
hipError_t sparse_hd(int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  switch (hd) {
    case 64: return sparse_g<VF, 64>(g, a, nwg, st);
    case 128: return sparse_g<VF, 128>(g, a, nwg, st);
    case 256: return sparse_g<VF, 256>(g, a, nwg, st);
    default: return hipErrorInvalidValue;
  }
}

template <int HD>
hipError_t sparse_merge_hd(bool vrot, int g, const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(uint32_t((uint64_t(a.num_seqs) * a.num_q_heads + 3) / 4)), block(256);
  if (vrot) hipLaunchKernelGGL((sparse_v_merge_kernel<HD, true>), grid, block, 0, st, a, uint32_t(g));
  else hipLaunchKernelGGL((sparse_v_merge_kernel<HD, false>), grid, block, 0, st, a, uint32_t(g));
  return hipGetLastError();
}

template <int HD>
hipError_t merge_hd(bool vrot, int g, const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(uint32_t((uint64_t(a.num_seqs) * a.num_q_heads + 3) / 4)), block(256);
  if (vrot) hipLaunchKernelGGL((merge_kernel<HD, true>), grid, block, 0, st, a, g);
  else hipLaunchKernelGGL((merge_kernel<HD, false>), grid, block, 0, st, a, g);
  return hipGetLastError();
}

// Decode row v = s * mq + i is query i of sequence s: its query row and its
// length (position + 1, the causal span), or no query (i past the chunk, or
// a position below 0, which the caller's contract excludes).
__global__ void prefill_rows_kernel(const int32_t* query_start, const int32_t* seq_lens, uint32_t num_seqs,
                                    uint32_t mq, int32_t* vrow, int32_t* vlen) {
  const uint64_t v = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (v >= uint64_t(num_seqs) * mq) return;
  const uint32_t s = uint32_t(v / mq), i = uint32_t(v % mq);
  const int q0 = query_start[s], n = query_start[s + 1] - q0;
  const int p = seq_lens[s] - n + int(i);
  const bool ok = int(i) < n && p >= 0;
  vrow[2 * v] = ok ? int32_t(s) : -1;
  vrow[2 * v + 1] = ok ? q0 + int32_t(i) : -1;
  vlen[v] = ok ? p + 1 : 0;
}

// A split kernel's units in order of decreasing length, bucketed by `width`
// positions (a counting sort in one workgroup; units of one bucket in any
// order).  Decode units are (split * S + sequence) with the split's length;
// prefill units (mode 1) are ((sequence * Hkv + kv head) * nsplit + split)
// with the key range of the unit's last tile within the split.  Started longest first, the units leave short
// ones for the end of the launch, when fewer workgroups share the memory
// bandwidth: a unit's workgroup streams its K rows at a limited rate, so a
// long unit started late would stretch the launch.
__global__ __launch_bounds__(1024) void unit_order_kernel(const DecodeArgs a, int mode, int width) {
  constexpr int NB = (KVQ_MAX_SPLIT > kMaxSparseSplit ? KVQ_MAX_SPLIT : kMaxSparseSplit) / kChunk + 1;
  constexpr int BPL = (NB + kWave - 1) / kWave;  // buckets per lane of the scan
  __shared__ uint32_t cnt[BPL * kWave];
  const uint32_t n = a.num_seqs * a.nsplit * (mode ? a.num_kv_heads : 1u);
  for (int b = threadIdx.x; b < BPL * kWave; b += 1024) cnt[b] = 0u;
  __syncthreads();
  auto bucket = [&](uint32_t u) {
    int len = 0;
    if (mode == 0) {
      const SeqSpan sp = split_span(a, u % a.num_seqs, u / a.num_seqs);
      len = sp.pe > sp.pb ? sp.pe - sp.pb : 0;
    } else {
      const uint32_t s = u / (a.num_kv_heads * a.nsplit), split = u % a.nsplit;
      const int nq = a.query_start[s + 1] - a.query_start[s];
      if (nq > 0) {
        const PrefillTile pt = prefill_tile(a, s, min(uint32_t(nq - 1) / a.qt, a.ntiles - 1u));
        len = pt.nq > 0 ? pt.hi - pt.lo : 0;
        if (a.nsplit > 1) len = max(0, min(int(a.split_len), len - int(split * a.split_len)));
      }
    }
    return min((len + width - 1) / width, NB - 1);
  };
  // the first kKeep units of each thread keep their bucket in registers for
  // the second pass (the rest are recomputed there)
  constexpr int kKeep = 4;
  int keep[kKeep];
#pragma unroll
  for (int k = 0; k < kKeep; ++k) {
    const uint32_t u = threadIdx.x + 1024u * k;
    keep[k] = u < n ? bucket(u) : 0;
  }
  // a wave whose units all fall in one bucket (equal lengths: the common
  // case) counts them with one atomic instead of 64 on the same address
  const int lane = threadIdx.x & 63;
  auto wave_uniform = [&](int k, uint64_t& valid) {
    valid = __ballot(threadIdx.x + 1024u * k < n);
    const int b0 = __shfl(keep[k], valid ? __builtin_ctzll(valid) : 0);
    return valid != 0 && __ballot(threadIdx.x + 1024u * k < n && keep[k] == b0) == valid;
  };
#pragma unroll
  for (int k = 0; k < kKeep; ++k) {
    uint64_t valid;
    if (wave_uniform(k, valid)) {
      if (lane == __builtin_ctzll(valid)) atomicAdd(&cnt[keep[k]], uint32_t(__popcll(valid)));
    } else if (threadIdx.x + 1024u * k < n) {
      atomicAdd(&cnt[keep[k]], 1u);
    }
  }
  for (uint32_t u = threadIdx.x + 1024u * kKeep; u < n; u += 1024) atomicAdd(&cnt[bucket(u)], 1u);
  __syncthreads();
  if (threadIdx.x < kWave) {  // first slot of each bucket, the longest bucket first: one wave's scan
    const int lane = threadIdx.x;
    uint32_t c[BPL], sum = 0;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {  // lane l takes buckets top - l * BPL - i (descending)
      c[i] = cnt[BPL * kWave - 1 - (lane * BPL + i)];
      sum += c[i];
    }
    uint32_t pre = sum;  // inclusive scan over the lanes
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const uint32_t v = __shfl_up(pre, off);
      if (lane >= off) pre += v;
    }
    uint32_t at = pre - sum;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      cnt[BPL * kWave - 1 - (lane * BPL + i)] = at;
      at += c[i];
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kKeep; ++k) {
    const uint32_t u = threadIdx.x + 1024u * k;
    uint64_t valid;
    if (wave_uniform(k, valid)) {
      const int lead = __builtin_ctzll(valid);
      uint32_t base = 0;
      if (lane == lead) base = atomicAdd(&cnt[keep[k]], uint32_t(__popcll(valid)));
      base = __shfl(base, lead);
      if (u < n) a.order[base + __popcll(valid & ((1ull << lane) - 1ull))] = u;
    } else if (u < n) {
      a.order[atomicAdd(&cnt[keep[k]], 1u)] = u;
    }
  }
  for (uint32_t u = threadIdx.x + 1024u * kKeep; u < n; u += 1024) a.order[atomicAdd(&cnt[bucket(u)], 1u)] = u;
}

}  // namespace

hipError_t launch_unit_order(const DecodeArgs& a, hipStream_t st, int mode, int width) {
  hipLaunchKernelGGL(unit_order_kernel, dim3(1), dim3(1024), 0, st, a, mode, width);
  return hipGetLastError();
}

hipError_t launch_prefill_rows(const int32_t* query_start, const int32_t* seq_lens, uint32_t num_seqs,
                               uint32_t max_query_len, int32_t* vrow, int32_t* vlen, hipStream_t st) {
  const uint64_t rows = uint64_t(num_seqs) * max_query_len;
  hipLaunchKernelGGL(prefill_rows_kernel, dim3(uint32_t((rows + 255) / 256)), dim3(256), 0, st, query_start, seq_lens,
                     num_seqs, max_query_len, vrow, vlen);
  return hipGetLastError();
}

hipError_t launch_sparse_v(int vf, int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  switch (vf) {
    case KVQ_BF16: return sparse_hd<KVQ_BF16>(hd, g, a, nwg, st);
    case KVQ_FP8_E4M3: return sparse_hd<KVQ_FP8_E4M3>(hd, g, a, nwg, st);
    case KVQ_TURBO2: return sparse_hd<KVQ_TURBO2>(hd, g, a, nwg, st);
    case KVQ_TURBO3: return sparse_hd<KVQ_TURBO3>(hd, g, a, nwg, st);
    case KVQ_TURBO4: return sparse_hd<KVQ_TURBO4>(hd, g, a, nwg, st);
    case KVQ_TURBO8: return sparse_hd<KVQ_TURBO8>(hd, g, a, nwg, st);
    case KVQ_NVFP4: return sparse_hd<KVQ_NVFP4>(hd, g, a, nwg, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_sparse_v_merge(bool v_rotated, int hd, int g, const DecodeArgs& a, hipStream_t st) {
  switch (hd) {
    case 64: return sparse_merge_hd<64>(v_rotated, g, a, st);
    case 128: return sparse_merge_hd<128>(v_rotated, g, a, st);
    case 256: return sparse_merge_hd<256>(v_rotated, g, a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_merge(bool v_rotated, int hd, int g, const DecodeArgs& a, hipStream_t st) {
  switch (hd) {
    case 64: return merge_hd<64>(v_rotated, g, a, st);
    case 128: return merge_hd<128>(v_rotated, g, a, st);
    case 256: return merge_hd<256>(v_rotated, g, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
