// Paged decode attention kernels (templates; instantiated per K format in
// kvq_decode_k*.hip and per V format in kvq_decode_sparse.hip).
//
// "metrale_model_layers/layers/ops/kv_cache_bf16k_turbov.rs",
// paged_decode_attn_bf16k_turbo{2,3,4}v: block_tables / seq_lens walk, GQA,
// inv_sqrt_d, sliding_window, and the sparse-V skip ("skips a position's V
// load and dequant when its attention weight is at most" the threshold).
// "combs_models/kv.rs", attend: softmax(q K^T * scale) V, no mask for a single
// decode query.  "spark_runtime/kv_cache.rs", is_wht_rotated: rotated K sides
// are scored against WHT(q); rotated V sides give WHT(out), rotated back.
//
// Work decomposition (differs from the pages' one-block-per-(q head, seq)):
//   * split-K over positions: a workgroup handles (sequence, kv head, split of
//     split_len positions) and ALL G = Hq/Hkv query heads of that kv head, so
//     every K/V byte is read once, not G times;
//   * inside a wave, T = head_dim/8 lanes share one position (8 dims per
//     lane) and 64/T positions are in flight per step, kUnroll steps deep;
//     a score is a T-lane DPP sum;
//   * every lane-slot keeps its own online softmax state (log2 domain), merged
//     across slots and waves at the end of the split;
//   * dense (threshold 0): partial (max, sum, unnormalized output) per split,
//     combined by merge_kernel (which also applies the iWHT);
//   * sparse (threshold > 0): scores_kernel stores only candidate positions
//     (split-local weight above thr: an upper bound on the global weight), then
//     sparse_v_kernel recomputes the exact global softmax weight of each
//     candidate and loads V only where some head of the group keeps it.
//   * workgroup ids are remapped so the kv heads of one (sequence, split) run
//     on the same XCD and share L2 lines (heads of a page are interleaved).
#pragma once

#include "kvq_device.h"

namespace kvq {

constexpr int kWaves = 4;        // waves per workgroup
constexpr int kDims = 8;         // head_dim elements per lane
constexpr int kUnroll = 4;       // positions in flight per lane slot
constexpr int kMaxPages = 512;   // page ids of one split staged in LDS
constexpr int kMaxSparseSplit = 1024;

template <int F>
struct Fmt {
  static constexpr int bits = (F == KVQ_BF16) ? 16 : (F == KVQ_FP8_E4M3) ? 8 : F;
  static constexpr bool turbo = F >= KVQ_TURBO2;
  static constexpr int words = (bits == 16) ? 4 : (bits == 8) ? 2 : 1;
};

template <int F>
struct Raw {
  uint32_t w[Fmt<F>::words];
  uint32_t sc;
};

// Bytes of one lane's 8 elements of row `row` (8 elements = `bits` bytes).
template <int F, int HD>
__device__ __forceinline__ void load_chunk(const uint8_t* __restrict__ blk, uint32_t row, int t,
                                           uint64_t data_bytes, Raw<F>& r) {
  constexpr int bits = Fmt<F>::bits;
  const uint8_t* p = blk + uint64_t(row) * (HD * bits / 8) + t * bits;
  if constexpr (bits == 16) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else if constexpr (bits == 8) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    r.w[0] = v.x; r.w[1] = v.y;
  } else if constexpr (bits == 4) {
    r.w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (bits == 2) {
    r.w[0] = *reinterpret_cast<const uint16_t*>(p);
  } else {
    r.w[0] = uint32_t(p[0]) | (uint32_t(p[1]) << 8) | (uint32_t(p[2]) << 16);
  }
  if constexpr (Fmt<F>::turbo) r.sc = blk[data_bytes + uint64_t(row) * (HD / 16) + (t >> 1)];
  else r.sc = 0;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Raw chunk -> 8 fp32 values.  bf16: exact; fp8: the E4M3 value (the tensor
// scale is applied by the caller); turbo: the codebook centroid (the group
// scale is returned in `sq`).
template <int F>
__device__ __forceinline__ void dequant(const Raw<F>& r, const float* __restrict__ cen, float (&v)[kDims],
                                        float& sq) {
  constexpr int bits = Fmt<F>::bits;
  sq = 1.0f;
  if constexpr (bits == 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(r.w[i] << 16);
      v[2 * i + 1] = __uint_as_float(r.w[i] & 0xFFFF0000u);
    }
  } else if constexpr (bits == 8) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(r.w[i]), false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(r.w[i]), true);
      v[4 * i] = lo.x; v[4 * i + 1] = lo.y; v[4 * i + 2] = hi.x; v[4 * i + 3] = hi.y;
    }
  } else {
    constexpr uint32_t mask = (1u << bits) - 1u;
#pragma unroll
    for (int i = 0; i < kDims; ++i) v[i] = cen[(r.w[0] >> (bits * i)) & mask];
    sq = e4m3_decode(r.sc);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Shared prologue: q rows of the G heads in LDS (rotated when K is), the
// codebook(s) and the split's page ids.
template <int KF, int VF, int HD, int G>
struct Smem {
  float q[G][HD];
  float kcen[16];
  float vcen[16];
  int32_t pages[kMaxPages];
};

template <int KF, int VF, int HD, int G>
__device__ __forceinline__ void prologue(const DecodeArgs& a, Smem<KF, VF, HD, G>& sm, uint32_t s, uint32_t g,
                                         int pb, int pe) {
  const int tid = threadIdx.x;
  const uint16_t* qg = a.q + uint64_t(s) * a.q_stride + uint64_t(g) * G * HD;
  for (int i = tid; i < G * HD; i += kWaves * kWave) sm.q[i / HD][i % HD] = bf16_bits_to_float(qg[i]);
  if (tid < 16) {
    if constexpr (Fmt<KF>::turbo) sm.kcen[tid] = tid < (1 << Fmt<KF>::bits) ? a.cb.centroid[KF - 2][tid] : 0.0f;
    if constexpr (Fmt<VF>::turbo) sm.vcen[tid] = tid < (1 << Fmt<VF>::bits) ? a.cb.centroid[VF - 2][tid] : 0.0f;
  }
  if (pe > pb) {
    const int first = pb >> a.log2_bs;
    const int n = ((pe - 1) >> a.log2_bs) - first + 1;
    const int32_t* bt = a.block_tables + uint64_t(s) * a.max_blocks + first;
    for (int i = tid; i < n; i += kWaves * kWave) sm.pages[i] = bt[i];
  }
  __syncthreads();
  if constexpr (Fmt<KF>::turbo) {
    // unnormalized WHT of every q row (the 1/sqrt(d) goes into the score scale)
    for (int h2 = 1; h2 < HD; h2 <<= 1) {
      for (int i = tid; i < G * HD / 2; i += kWaves * kWave) {
        const int hh = i / (HD / 2), k = i % (HD / 2);
        const int lo = (k / h2) * 2 * h2 + (k % h2);
        const float x = sm.q[hh][lo], y = sm.q[hh][lo + h2];
        sm.q[hh][lo] = x + y;
        sm.q[hh][lo + h2] = x - y;
      }
      __syncthreads();
    }
  }
}

struct SeqSpan {
  int L, j0, pb, pe;
};

__device__ __forceinline__ SeqSpan split_span(const DecodeArgs& a, uint32_t s, uint32_t split) {
  SeqSpan r;
  r.L = a.seq_lens[s];
  r.j0 = (a.window != 0u && r.L > int(a.window)) ? r.L - int(a.window) : 0;
  r.pb = r.j0 + int(split * a.split_len);
  r.pe = min(r.L, r.pb + int(a.split_len));
  return r;
}

// Scores of up to kUnroll positions of one lane slot (log2 units; -inf when
// the position is past the end), with their K chunks loaded in one batch.
template <int KF, int VF, int HD, int G, bool LOAD_V>
__device__ __forceinline__ void score_step(const DecodeArgs& a, const Smem<KF, VF, HD, G>& sm,
                                           const float (&qr)[G][kDims], int c0, int pb, int pe, uint32_t g,
                                           int t, int r, float (&sc)[kUnroll][G], Raw<VF> (&vr)[kUnroll],
                                           bool (&valid)[kUnroll]) {
  constexpr int T = HD / kDims;
  constexpr int P = kWave / T;
  const int first = pb >> a.log2_bs;
  const uint32_t bmask = (1u << a.log2_bs) - 1u;
  Raw<KF> kr[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int j = c0 + u * P + r;
    valid[u] = j < pe;
    if (valid[u]) {
      const uint64_t page = uint64_t(uint32_t(sm.pages[(j >> a.log2_bs) - first]));
      const uint32_t row = (uint32_t(j) & bmask) * a.num_kv_heads + g;
      load_chunk<KF, HD>(a.k_cache + page * a.k_stride, row, t, a.k_data, kr[u]);
      if constexpr (LOAD_V) load_chunk<VF, HD>(a.v_cache + page * a.v_stride, row, t, a.v_data, vr[u]);
    } else {
      // past the end: zero bytes decode to finite values, so p = 0 times them stays 0
#pragma unroll
      for (int k = 0; k < Fmt<KF>::words; ++k) kr[u].w[k] = 0;
      kr[u].sc = 0;
#pragma unroll
      for (int k = 0; k < Fmt<VF>::words; ++k) vr[u].w[k] = 0;
      vr[u].sc = 0;
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    float kv[kDims], sq;
    dequant<KF>(kr[u], sm.kcen, kv, sq);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < kDims; ++i) part = fmaf(qr[h][i], kv[i], part);
      if constexpr (Fmt<KF>::turbo) part *= sq;
      part = group_sum<T>(part);
      sc[u][h] = valid[u] ? part : -INFINITY;
    }
  }
}

// ------------------------------------------------------------------ dense split

template <int KF, int VF, int HD, int G>
struct SplitSmem {
  Smem<KF, VF, HD, G> base;
  float red[kWaves][G][HD + 2];
};

template <int KF, int VF, int HD, int G>
__global__ __launch_bounds__(kWaves * kWave) void split_kernel(const DecodeArgs a) {
  constexpr int T = HD / kDims;
  constexpr int P = kWave / T;
  constexpr int CH = P * kUnroll;
  __shared__ SplitSmem<KF, VF, HD, G> sm;
  const uint32_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const uint32_t g = tile % a.num_kv_heads;
  const uint32_t split = (tile / a.num_kv_heads) % a.nsplit;
  const uint32_t s = tile / (a.num_kv_heads * a.nsplit);
  const SeqSpan sp = split_span(a, s, split);
  if (sp.pb >= sp.L) return;
  prologue<KF, VF, HD, G>(a, sm.base, s, g, sp.pb, sp.pe);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t = lane % T, r = lane / T;
  const float qscale = a.qk_scale * (Fmt<KF>::turbo ? a.wht_scale : 1.0f);
  float qr[G][kDims];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < kDims; ++i) qr[h][i] = sm.base.q[h][t * kDims + i] * qscale;

  float m[G], l[G], acc[G][kDims];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < kDims; ++i) acc[h][i] = 0.0f;
  }

  for (int c0 = sp.pb + w * CH; c0 < sp.pe; c0 += kWaves * CH) {
    float sc[kUnroll][G];
    Raw<VF> vr[kUnroll];
    bool valid[kUnroll];
    score_step<KF, VF, HD, G, true>(a, sm.base, qr, c0, sp.pb, sp.pe, g, t, r, sc, vr, valid);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = sc[0][h];
#pragma unroll
      for (int u = 1; u < kUnroll; ++u) mx = fmaxf(mx, sc[u][h]);
      if (mx > m[h]) {
        const float alpha = fast_exp2(m[h] - mx);  // 0 while m is -inf
        l[h] *= alpha;
#pragma unroll
        for (int i = 0; i < kDims; ++i) acc[h][i] *= alpha;
        m[h] = mx;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float vv[kDims], sq;
      dequant<VF>(vr[u], sm.base.vcen, vv, sq);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = valid[u] ? fast_exp2(sc[u][h] - m[h]) : 0.0f;
        l[h] += p;
        const float pw = p * sq;
#pragma unroll
        for (int i = 0; i < kDims; ++i) acc[h][i] = fmaf(pw, vv[i], acc[h][i]);
      }
    }
  }

  // merge the P lane slots of the wave (same dims, different positions)
#pragma unroll
  for (int off = T; off < kWave; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off);
      const float lo = __shfl_xor(l[h], off);
      const float M = fmaxf(m[h], mo);
      const float a1 = m[h] > -INFINITY ? fast_exp2(m[h] - M) : 0.0f;
      const float a2 = mo > -INFINITY ? fast_exp2(mo - M) : 0.0f;
      l[h] = l[h] * a1 + lo * a2;
#pragma unroll
      for (int i = 0; i < kDims; ++i) acc[h][i] = acc[h][i] * a1 + __shfl_xor(acc[h][i], off) * a2;
      m[h] = M;
    }
  }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int i = 0; i < kDims; ++i) sm.red[w][h][t * kDims + i] = acc[h][i];
      if (t == 0) {
        sm.red[w][h][HD] = m[h];
        sm.red[w][h][HD + 1] = l[h];
      }
    }
  }
  __syncthreads();
  const uint64_t base = (uint64_t(s) * a.num_kv_heads + g) * a.nsplit + split;
  for (int i = tid; i < G * HD; i += kWaves * kWave) {
    const int h = i / HD, d = i % HD;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm.red[ww][h][HD]);
    float o = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float mw = sm.red[ww][h][HD];
      if (mw > -INFINITY) o += fast_exp2(mw - M) * sm.red[ww][h][d];
    }
    a.part[(base * G + h) * HD + d] = o;
  }
  if (tid < G) {
    const int h = tid;
    float M = -INFINITY;
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm.red[ww][h][HD]);
    float sum = 0.0f;
    for (int ww = 0; ww < kWaves; ++ww) {
      const float mw = sm.red[ww][h][HD];
      if (mw > -INFINITY) sum += fast_exp2(mw - M) * sm.red[ww][h][HD + 1];
    }
    a.ml[(base * G + h) * 2] = M;
    a.ml[(base * G + h) * 2 + 1] = sum;
  }
}

// ------------------------------------------------------------------ merge

// Rotate an LDS row of HD values by the orthonormal WHT (used to bring a
// rotated V side's output back).  All threads of the block take part.
template <int HD>
__device__ __forceinline__ void lds_wht(float* x, float scale) {
  const int tid = threadIdx.x;
  for (int h2 = 1; h2 < HD; h2 <<= 1) {
    for (int k = tid; k < HD / 2; k += kWaves * kWave) {
      const int lo = (k / h2) * 2 * h2 + (k % h2);
      const float u = x[lo], v = x[lo + h2];
      x[lo] = u + v;
      x[lo + h2] = u - v;
    }
    __syncthreads();
  }
  for (int d = tid; d < HD; d += kWaves * kWave) x[d] *= scale;
  __syncthreads();
}

// One workgroup per (sequence, q head): combine the split partials.
template <int HD, bool VROT>
__global__ __launch_bounds__(kWaves * kWave) void merge_kernel(const DecodeArgs a, int G) {
  __shared__ float o[HD];
  const uint32_t hq = blockIdx.x % a.num_q_heads;
  const uint32_t s = blockIdx.x / a.num_q_heads;
  const uint32_t g = hq / G, h = hq % G;
  const SeqSpan sp = split_span(a, s, 0);
  const int span = sp.L - sp.j0;
  const int ns = span > 0 ? (span + int(a.split_len) - 1) / int(a.split_len) : 0;
  const int tid = threadIdx.x;
  const uint64_t base = (uint64_t(s) * a.num_kv_heads + g) * a.nsplit;
  float M = -INFINITY;
  for (int k = 0; k < ns; ++k) M = fmaxf(M, a.ml[((base + k) * G + h) * 2]);
  float sum = 0.0f;
  for (int k = 0; k < ns; ++k) {
    const float mk = a.ml[((base + k) * G + h) * 2];
    if (mk > -INFINITY) sum += fast_exp2(mk - M) * a.ml[((base + k) * G + h) * 2 + 1];
  }
  const float inv = sum > 0.0f ? a.v_scale / sum : 0.0f;
  for (int d = tid; d < HD; d += kWaves * kWave) {
    float acc = 0.0f;
    for (int k = 0; k < ns; ++k) {
      const float mk = a.ml[((base + k) * G + h) * 2];
      if (mk > -INFINITY) acc += fast_exp2(mk - M) * a.part[((base + k) * G + h) * HD + d];
    }
    o[d] = acc * inv;
  }
  __syncthreads();
  if constexpr (VROT) lds_wht<HD>(o, a.wht_scale);
  float* dst = a.out + (uint64_t(s) * a.num_q_heads + hq) * HD;
  for (int d = tid; d < HD; d += kWaves * kWave) dst[d] = o[d];
}

// ------------------------------------------------------------------ sparse V

template <int KF, int HD, int G>
struct ScoreSmem {
  Smem<KF, KVQ_BF16, HD, G> base;
  float sc[kMaxSparseSplit * G];
  float wred[kWaves][G];
  float stat[G][2];
  int wcount[kWaves];
};

// Scores of one split; stores the split's (max, sum) and the candidate
// positions whose split-local weight exceeds thr * (1 - 1e-4).  Since the
// global normalizer is at least the split's, a position that is not a
// candidate has global weight <= thr and is provably skipped.
template <int KF, int HD, int G>
__global__ __launch_bounds__(kWaves * kWave) void scores_kernel(const DecodeArgs a) {
  constexpr int T = HD / kDims;
  constexpr int P = kWave / T;
  constexpr int CH = P * kUnroll;
  __shared__ ScoreSmem<KF, HD, G> sm;
  const uint32_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const uint32_t g = tile % a.num_kv_heads;
  const uint32_t split = (tile / a.num_kv_heads) % a.nsplit;
  const uint32_t s = tile / (a.num_kv_heads * a.nsplit);
  const SeqSpan sp = split_span(a, s, split);
  if (sp.pb >= sp.L) return;
  prologue<KF, KVQ_BF16, HD, G>(a, sm.base, s, g, sp.pb, sp.pe);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t = lane % T, r = lane / T;
  const float qscale = a.qk_scale * (Fmt<KF>::turbo ? a.wht_scale : 1.0f);
  float qr[G][kDims];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < kDims; ++i) qr[h][i] = sm.base.q[h][t * kDims + i] * qscale;

  float mloc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mloc[h] = -INFINITY;
  for (int c0 = sp.pb + w * CH; c0 < sp.pe; c0 += kWaves * CH) {
    float sc[kUnroll][G];
    Raw<KVQ_BF16> vr[kUnroll];
    bool valid[kUnroll];
    score_step<KF, KVQ_BF16, HD, G, false>(a, sm.base, qr, c0, sp.pb, sp.pe, g, t, r, sc, vr, valid);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = c0 + u * P + r;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        mloc[h] = fmaxf(mloc[h], sc[u][h]);
        if (valid[u] && t == 0) sm.sc[(j - sp.pb) * G + h] = sc[u][h];
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mw = group_max<kWave>(mloc[h]);
    if (lane == 0) sm.wred[w][h] = mw;
  }
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY;
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm.wred[ww][tid]);
    sm.stat[tid][0] = M;
  }
  __syncthreads();
  const int n = sp.pe - sp.pb;
  float lsum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) lsum[h] = 0.0f;
  for (int i = tid; i < n; i += kWaves * kWave) {
#pragma unroll
    for (int h = 0; h < G; ++h) lsum[h] += fast_exp2(sm.sc[i * G + h] - sm.stat[h][0]);
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float lw = group_sum<kWave>(lsum[h]);
    if (lane == 0) sm.wred[w][h] = lw;
  }
  __syncthreads();
  if (tid < G) {
    float sum = 0.0f;
    for (int ww = 0; ww < kWaves; ++ww) sum += sm.wred[ww][tid];
    sm.stat[tid][1] = sum;
  }
  __syncthreads();
  const uint64_t base = (uint64_t(s) * a.num_kv_heads + g) * a.nsplit + split;
  if (tid < G) {
    a.ml[(base * G + tid) * 2] = sm.stat[tid][0];
    a.ml[(base * G + tid) * 2 + 1] = sm.stat[tid][1];
  }
  // candidates, compacted in position order
  float cut[G];
#pragma unroll
  for (int h = 0; h < G; ++h) cut[h] = a.thr * (1.0f - 1e-4f) * sm.stat[h][1];
  int32_t* cidx = a.cidx + base * a.split_len;
  float* cs = a.cscore + base * a.split_len * G;
  int total = 0;
  for (int c = 0; c < n; c += kWaves * kWave) {
    const int i = c + tid;
    bool cand = false;
    if (i < n) {
#pragma unroll
      for (int h = 0; h < G; ++h) cand |= fast_exp2(sm.sc[i * G + h] - sm.stat[h][0]) > cut[h];
    }
    const uint64_t ballot = __ballot(cand);
    const int before = __popcll(ballot & ((1ull << lane) - 1ull));
    if (lane == 0) sm.wcount[w] = __popcll(ballot);
    __syncthreads();
    int off = total;
    for (int ww = 0; ww < w; ++ww) off += sm.wcount[ww];
    if (cand) {
      const int k = off + before;
      cidx[k] = sp.pb + i;
#pragma unroll
      for (int h = 0; h < G; ++h) cs[k * G + h] = sm.sc[i * G + h];
    }
    for (int ww = 0; ww < kWaves; ++ww) total += sm.wcount[ww];
    __syncthreads();
  }
  if (tid == 0) a.cnt[base] = total;
}

template <int VF, int HD, int G>
struct SparseSmem {
  float mz[G][2];
  float vcen[16];
  float red[kWaves][G][HD];
};

// One workgroup per (sequence, kv head): exact global weights of the
// candidates, V loaded only where some head of the group keeps the position.
template <int VF, int HD, int G>
__global__ __launch_bounds__(kWaves * kWave) void sparse_v_kernel(const DecodeArgs a) {
  constexpr int T = HD / kDims;
  constexpr int P = kWave / T;
  constexpr int NS = kWaves * P;  // lane slots per workgroup
  __shared__ SparseSmem<VF, HD, G> sm;
  const uint32_t g = blockIdx.x % a.num_kv_heads;
  const uint32_t s = blockIdx.x / a.num_kv_heads;
  const SeqSpan sp = split_span(a, s, 0);
  const int span = sp.L - sp.j0;
  const int ns = span > 0 ? (span + int(a.split_len) - 1) / int(a.split_len) : 0;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t = lane % T, r = lane / T;
  const uint64_t base = (uint64_t(s) * a.num_kv_heads + g) * a.nsplit;
  if (tid < G) {
    float M = -INFINITY;
    for (int k = 0; k < ns; ++k) M = fmaxf(M, a.ml[((base + k) * G + tid) * 2]);
    float z = 0.0f;
    for (int k = 0; k < ns; ++k) {
      const float mk = a.ml[((base + k) * G + tid) * 2];
      if (mk > -INFINITY) z += fast_exp2(mk - M) * a.ml[((base + k) * G + tid) * 2 + 1];
    }
    sm.mz[tid][0] = M;
    sm.mz[tid][1] = z > 0.0f ? 1.0f / z : 0.0f;
  }
  if (tid < 16) {
    if constexpr (Fmt<VF>::turbo) sm.vcen[tid] = tid < (1 << Fmt<VF>::bits) ? a.cb.centroid[VF - 2][tid] : 0.0f;
  }
  __syncthreads();
  float M[G], iz[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    M[h] = sm.mz[h][0];
    iz[h] = sm.mz[h][1];
  }
  float acc[G][kDims];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < kDims; ++i) acc[h][i] = 0.0f;
  const int32_t* bt = a.block_tables + uint64_t(s) * a.max_blocks;
  const uint32_t bmask = (1u << a.log2_bs) - 1u;
  const int slot = w * P + r;
  for (int k = 0; k < ns; ++k) {
    const int cnt = a.cnt[base + k];
    const int32_t* cidx = a.cidx + (base + k) * a.split_len;
    const float* cs = a.cscore + (base + k) * a.split_len * G;
    for (int i = slot; i < cnt; i += NS) {
      const int j = cidx[i];
      float p[G];
      bool any = false;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        p[h] = fast_exp2(cs[i * G + h] - M[h]) * iz[h];
        p[h] = p[h] > a.thr ? p[h] : 0.0f;
        any |= p[h] > 0.0f;
      }
      if (any) {
        const uint64_t page = uint64_t(uint32_t(bt[j >> a.log2_bs]));
        const uint32_t row = (uint32_t(j) & bmask) * a.num_kv_heads + g;
        Raw<VF> vr;
        load_chunk<VF, HD>(a.v_cache + page * a.v_stride, row, t, a.v_data, vr);
        float vv[kDims], sq;
        dequant<VF>(vr, sm.vcen, vv, sq);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float pw = p[h] * sq;
#pragma unroll
          for (int i2 = 0; i2 < kDims; ++i2) acc[h][i2] = fmaf(pw, vv[i2], acc[h][i2]);
        }
      }
    }
  }
#pragma unroll
  for (int off = T; off < kWave; off <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < kDims; ++i) acc[h][i] += __shfl_xor(acc[h][i], off);
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < kDims; ++i) sm.red[w][h][t * kDims + i] = acc[h][i];
  }
  __syncthreads();
  for (int i = tid; i < G * HD; i += kWaves * kWave) {
    const int h = i / HD, d = i % HD;
    float o = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) o += sm.red[ww][h][d];
    sm.red[0][h][d] = o * a.v_scale;
  }
  __syncthreads();
  if constexpr (Fmt<VF>::turbo) {
    for (int h = 0; h < G; ++h) lds_wht<HD>(sm.red[0][h], a.wht_scale);
  }
  for (int i = tid; i < G * HD; i += kWaves * kWave) {
    const int h = i / HD, d = i % HD;
    a.out[(uint64_t(s) * a.num_q_heads + g * G + h) * HD + d] = sm.red[0][h][d];
  }
}

// ------------------------------------------------------------------ dispatch

template <int KF, int VF, int HD>
hipError_t launch_split_g(int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  const dim3 grid(nwg), block(kWaves * kWave);
  switch (g) {
    case 1: hipLaunchKernelGGL((split_kernel<KF, VF, HD, 1>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((split_kernel<KF, VF, HD, 2>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((split_kernel<KF, VF, HD, 4>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((split_kernel<KF, VF, HD, 8>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KF, int VF>
hipError_t launch_split_hd(int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  switch (hd) {
    case 64: return launch_split_g<KF, VF, 64>(g, a, nwg, st);
    case 128: return launch_split_g<KF, VF, 128>(g, a, nwg, st);
    case 256: return launch_split_g<KF, VF, 256>(g, a, nwg, st);
    default: return hipErrorInvalidValue;
  }
}

template <int KF>
hipError_t launch_split_k(int vf, int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  switch (vf) {
    case KVQ_BF16: return launch_split_hd<KF, KVQ_BF16>(hd, g, a, nwg, st);
    case KVQ_FP8_E4M3: return launch_split_hd<KF, KVQ_FP8_E4M3>(hd, g, a, nwg, st);
    case KVQ_TURBO2: return launch_split_hd<KF, KVQ_TURBO2>(hd, g, a, nwg, st);
    case KVQ_TURBO3: return launch_split_hd<KF, KVQ_TURBO3>(hd, g, a, nwg, st);
    case KVQ_TURBO4: return launch_split_hd<KF, KVQ_TURBO4>(hd, g, a, nwg, st);
    default: return hipErrorInvalidValue;
  }
}

template <int KF, int HD>
hipError_t launch_scores_g(int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  const dim3 grid(nwg), block(kWaves * kWave);
  switch (g) {
    case 1: hipLaunchKernelGGL((scores_kernel<KF, HD, 1>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((scores_kernel<KF, HD, 2>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((scores_kernel<KF, HD, 4>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((scores_kernel<KF, HD, 8>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KF>
hipError_t launch_scores_k(int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  switch (hd) {
    case 64: return launch_scores_g<KF, 64>(g, a, nwg, st);
    case 128: return launch_scores_g<KF, 128>(g, a, nwg, st);
    case 256: return launch_scores_g<KF, 256>(g, a, nwg, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
