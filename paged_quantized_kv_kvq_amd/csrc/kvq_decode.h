// Paged decode attention kernels (templates; instantiated per K format in
// kvq_decode_k*.hip and per V format in kvq_decode_sparse.hip).
//
// "metrale_model_layers/layers/ops/kv_cache_bf16k_turbov.rs",
// paged_decode_attn_bf16k_turbo{2,3,4}v: block_tables / seq_lens walk, GQA,
// inv_sqrt_d, sliding_window, and the sparse-V skip (a position's V is not
// loaded or dequantized when its attention weight is at most the threshold).
// "combs_models/kv.rs", attend: softmax(q K^T * scale) V, no mask for a single
// decode query.  "spark_runtime/kv_cache.rs", is_wht_rotated: rotated K sides
// are scored against WHT(q); rotated V sides give WHT(out), rotated back.
//
// Work decomposition of the VALU kernels here (differs from the pages'
// one-block-per-(q head, seq); the matrix-core split kernel is in
// kvq_decode_mfma.h):
//   * split-K over positions: a workgroup handles (sequence, kv head, split of
//     split_len positions) and ALL G = Hq/Hkv query heads of that kv head, so
//     every K/V byte is read once, not G times;
//   * a wave walks 16-position chunks (wave w of NW: chunks w, w + NW, ...);
//     each lane finds its position's page in an LDS copy of the split's page
//     table; chunk loads run one chunk ahead of their use, all issued inside
//     the loop;
//   * inside a chunk, T = head_dim/D lanes share one position (D = 16 dims
//     per lane, 8 for G = 8) and 64/T positions are side by side; a score is
//     a T-lane DPP sum of bf16 dot products (v_dot2_f32_bf16 for bf16 K and
//     for fp8 K widened exactly to bf16) or fp32 FMAs (rotated turbo K);
//   * every lane slot keeps its own online softmax state (log2 domain),
//     merged across slots and waves at the end of the split;
//   * dense (threshold 0): partial (max, sum, unnormalized output) per split,
//     combined by merge_kernel (which also applies the inverse rotation);
//   * sparse (threshold > 0): scores_kernel keeps only candidate positions
//     (split-local weight above thr: an upper bound on the global weight),
//     each wave in its own segment (a grouped-scale K side is scored on the
//     matrix cores); sparse_v_kernel, one or more workgroups ("parts") per
//     (sequence, kv head), recomputes each candidate's exact global weight,
//     loads V only where some head of the group keeps it, and writes the
//     output (fp8 V scale, inverse rotation), or with several parts their
//     sums, which sparse_v_merge_kernel adds;
//   * workgroup ids are renumbered so the kv heads of one (sequence, split)
//     run on the same XCD, and consecutive units rotate over the XCDs; the
//     units can be taken longest first (unit_order_kernel, or
//     inline_unit_order in the score kernel).
#pragma once

#include "kvq_device.h"

namespace kvq {

constexpr int kWaves = KVQ_WAVES;  // waves per workgroup
constexpr int kChunk = 16;         // positions per wave iteration
constexpr int kMaxPages = KVQ_MAX_PAGES;  // page offsets of one split staged in LDS
constexpr int kMaxSparseSplit = KVQ_MAX_SPARSE_SPLIT;

template <int F>
struct Fmt {
  static constexpr int bits = (F == KVQ_BF16) ? 16 : (F == KVQ_FP8_E4M3) ? 8 : (F == KVQ_NVFP4) ? 4 : F;
  static constexpr bool turbo = F >= KVQ_TURBO2;             // per-16 group scales (turbo sides, NVFP4)
  static constexpr bool rot = turbo && F != KVQ_NVFP4;       // rotated side (is_wht_rotated)
  static constexpr bool cb = turbo && F != KVQ_TURBO8;       // 4-bit or smaller codes through a table
  static constexpr int sgb = cb ? 1 : (F == KVQ_TURBO8 ? 2 : 0);  // scale bytes per group of 16
};

// Lane geometry for a head size and a number of dims per lane.
template <int HD, int DIMS>
struct Geo {
  static constexpr int D = DIMS;          // dims per lane
  static constexpr int T = HD / D;        // lanes per position
  static constexpr int P = kWave / T;     // positions side by side in a wave
  static constexpr int U = kChunk / P;    // steps per chunk
  static_assert(P >= 1 && P <= kChunk && kChunk % P == 0, "chunk geometry");
};

// Dims per lane of the dense split kernel and of the sparse score kernel:
// 16 (fewer lanes per position, cheaper sums) unless the G accumulators or
// query registers of 16 dims would cost too many registers.
template <int G>
struct LaneDims {
  static constexpr int dense = (G <= 4) ? 16 : 8;
  static constexpr int score = KVQ_SCORE_DIMS > 0 ? KVQ_SCORE_DIMS : dense;
};

// One lane's bytes of one position: D elements (+ the group scale byte).
template <int F, int D>
struct Raw {
  static constexpr int bytes = D * Fmt<F>::bits / 8;
  static constexpr int words = (bytes + 3) / 4;
  uint32_t w[words];
  uint32_t sc;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Cache rows are streamed once per decode: optionally tag the loads non-temporal.
__device__ __forceinline__ u32x4 load16(const uint8_t* p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
#if KVQ_NT_LOADS
  return __builtin_nontemporal_load(q);
#else
  return *q;
#endif
}
__device__ __forceinline__ u32x2 load8(const uint8_t* p) {
  const u32x2* q = reinterpret_cast<const u32x2*>(p);
#if KVQ_NT_LOADS
  return __builtin_nontemporal_load(q);
#else
  return *q;
#endif
}
__device__ __forceinline__ uint32_t load4(const uint8_t* p) {
  const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
#if KVQ_NT_LOADS
  return __builtin_nontemporal_load(q);
#else
  return *q;
#endif
}

template <int F, int HD, int D>
__device__ __forceinline__ void load_lane(const uint8_t* __restrict__ blk, uint32_t row, int t,
                                          uint64_t data_bytes, Raw<F, D>& r) {
  constexpr int B = Raw<F, D>::bytes;
  const uint8_t* p = blk + uint64_t(row) * (HD * Fmt<F>::bits / 8) + t * B;
  if constexpr (B == 32) {
    const u32x4 a = load16(p), b = load16(p + 16);
    r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
    r.w[4] = b.x; r.w[5] = b.y; r.w[6] = b.z; r.w[7] = b.w;
  } else if constexpr (B == 16) {
    const u32x4 a = load16(p);
    r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
  } else if constexpr (B == 8) {
    const u32x2 a = load8(p);
    r.w[0] = a.x; r.w[1] = a.y;
  } else if constexpr (B == 4) {
    r.w[0] = load4(p);
  } else if constexpr (B == 2) {
    r.w[0] = *reinterpret_cast<const uint16_t*>(p);
  } else {
    // 3-bit codes: 3 or 6 bytes at any alignment.  Read the two aligned
    // dwords that cover them (at most 2 bytes past the row end, still inside
    // the block: the scale section follows the codes) and shift.
    const uintptr_t ad = reinterpret_cast<uintptr_t>(p);
    const uint32_t* q = reinterpret_cast<const uint32_t*>(ad & ~uintptr_t(3));
    const uint64_t v = (uint64_t(q[1]) << 32 | q[0]) >> ((ad & 3u) * 8u);
    r.w[0] = uint32_t(v);
    if constexpr (Raw<F, D>::words > 1) r.w[1] = uint32_t(v >> 32) & 0xFFFFu;
  }
  // The scale (an E4M3 byte, or turbo8's BF16 word) is read as the aligned
  // dword that holds it (scale_shift selects it at the use), so no byte
  // extension sits next to the load.
  if constexpr (Fmt<F>::turbo) {
    constexpr int SG = Fmt<F>::sgb;
    r.sc = *reinterpret_cast<const uint32_t*>(blk + data_bytes + uint64_t(row) * (HD / 16 * SG) +
                                             ((((t * D) / 16) * SG) & ~3));
  } else {
    r.sc = 0;
  }
}

// Bit offset of a lane's scale inside the dword load_lane reads (SG scale
// bytes per group).
template <int D, int SG = 1>
__device__ __forceinline__ uint32_t scale_shift(int t) {
  return 8u * uint32_t((((t * D) / 16) * SG) & 3);
}

// The group scale a lane reads: an E4M3 byte, or turbo8's BF16 word.
template <int F>
__device__ __forceinline__ float group_scale(uint32_t word, uint32_t shift) {
  if constexpr (Fmt<F>::cb) return e4m3_decode(word >> shift);
  else return __uint_as_float((word >> shift) << 16);
}

template <int F, int D>
__device__ __forceinline__ void zero_raw(Raw<F, D>& r) {
#pragma unroll
  for (int i = 0; i < Raw<F, D>::words; ++i) r.w[i] = 0;
  r.sc = 0;
}

// code i of a lane's turbo chunk
template <int BITS, int D>
__device__ __forceinline__ uint32_t code_at(const uint32_t* w, int i) {
  if constexpr (BITS == 3 && D == 16) {
    return uint32_t(((uint64_t(w[1]) << 32) | w[0]) >> (3 * i)) & 7u;
  } else if constexpr (BITS == 3) {
    return (w[0] >> (3 * i)) & 7u;
  } else {
    const int bit = BITS * i;
    return (w[bit / 32] >> (bit % 32)) & ((1u << BITS) - 1u);
  }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// two E4M3 bytes (low or high half of w) -> two bf16 (exact: every E4M3 value is a bf16 value)
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w), 1.0f, HI));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Rotate a row of E * 64 values held by a wave (lane l holds elements l * E
// ... l * E + E - 1) by the orthonormal WHT, which brings a rotated V side's
// output back: butterflies inside the lane for the low index bits, then lane
// exchanges, in the order of increasing stride; then x scale.
template <int E>
__device__ __forceinline__ void wave_wht(float (&x)[E], int lane, float scale) {
#pragma unroll
  for (int h2 = 1; h2 < E; h2 <<= 1)
#pragma unroll
    for (int i = 0; i < E; ++i)
      if (!(i & h2)) {
        const float p = x[i], q = x[i + h2];
        x[i] = p + q;
        x[i + h2] = p - q;
      }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1)
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float o = __shfl_xor(x[i], m);
      x[i] = (lane & m) ? o - x[i] : x[i] + o;
    }
#pragma unroll
  for (int i = 0; i < E; ++i) x[i] *= scale;
}

// Query registers of one lane: packed bf16 pairs (bf16 / fp8 K) or the rotated
// fp32 query (turbo K), for the lane's D dims of each of the G heads.
template <int KF, int D, int G>
struct QReg {
  static constexpr bool packed = !Fmt<KF>::turbo;
  uint32_t qp[packed ? G : 1][packed ? D / 2 : 1];
  float qf[packed ? 1 : G][packed ? 1 : D];
  uint32_t scsh;  // scale_shift of the lane (turbo K)
  uint32_t vsh;   // ... of the V side (turbo V)
};

// Partial score of one lane for every head (before the T-lane sum).
template <int KF, int D, int G>
__device__ __forceinline__ void lane_scores(const QReg<KF, D, G>& q, const Raw<KF, D>& k,
                                            const float* __restrict__ kcen, float (&part)[G]) {
  if constexpr (KF == KVQ_BF16) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < D / 2; ++i) s = dot2_bf16(q.qp[h][i], k.w[i], s);
      part[h] = s;
    }
  } else if constexpr (KF == KVQ_FP8_E4M3) {
    uint32_t kb[D / 2];
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      kb[2 * i] = fp8x2_to_bf16x2<false>(k.w[i]);
      kb[2 * i + 1] = fp8x2_to_bf16x2<true>(k.w[i]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < D / 2; ++i) s = dot2_bf16(q.qp[h][i], kb[i], s);
      part[h] = s;
    }
  } else {
    float kv[D];
    if constexpr (Fmt<KF>::cb) {
#pragma unroll
      for (int i = 0; i < D; ++i) kv[i] = kcen[code_at<Fmt<KF>::bits, D>(k.w, i)];
    } else {
#pragma unroll
      for (int i = 0; i < D / 4; ++i) {
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(k.w[i]), false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(k.w[i]), true);
        kv[4 * i] = lo.x; kv[4 * i + 1] = lo.y; kv[4 * i + 2] = hi.x; kv[4 * i + 3] = hi.y;
      }
    }
    const float sq = group_scale<KF>(k.sc, q.scsh);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < D; ++i) s = fmaf(q.qf[h][i], kv[i], s);
      part[h] = s * sq;
    }
  }
}

// V chunk -> D fp32 values (bf16 exact, fp8 the E4M3 value, turbo the
// centroid with the group scale in `sq`).
template <int VF, int D>
__device__ __forceinline__ void v_values(const Raw<VF, D>& v, const float* __restrict__ vcen, float (&x)[D],
                                         float& sq, uint32_t scsh) {
  sq = 1.0f;
  if constexpr (VF == KVQ_BF16) {
#pragma unroll
    for (int i = 0; i < D / 2; ++i) {
      x[2 * i] = __uint_as_float(v.w[i] << 16);
      x[2 * i + 1] = __uint_as_float(v.w[i] & 0xFFFF0000u);
    }
  } else if constexpr (VF == KVQ_FP8_E4M3) {
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(v.w[i]), false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(v.w[i]), true);
      x[4 * i] = lo.x; x[4 * i + 1] = lo.y; x[4 * i + 2] = hi.x; x[4 * i + 3] = hi.y;
    }
  } else if constexpr (Fmt<VF>::cb) {
#pragma unroll
    for (int i = 0; i < D; ++i) x[i] = vcen[code_at<Fmt<VF>::bits, D>(v.w, i)];
    sq = e4m3_decode(v.sc >> scsh);
  } else {
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(v.w[i]), false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(v.w[i]), true);
      x[4 * i] = lo.x; x[4 * i + 1] = lo.y; x[4 * i + 2] = hi.x; x[4 * i + 3] = hi.y;
    }
    sq = group_scale<VF>(v.sc, scsh);
  }
}

// The query / output row and the block-table row of decode row s: both s in
// a plain decode call; chunked prefill run as decode rows maps them.
__device__ __forceinline__ uint32_t row_query(const DecodeArgs& a, uint32_t s) {
  return a.vrow ? uint32_t(a.vrow[2 * s + 1]) : s;
}
__device__ __forceinline__ uint32_t row_table(const DecodeArgs& a, uint32_t s) {
  return a.vrow ? uint32_t(a.vrow[2 * s]) : s;
}

// Positions [pb, pe) of a split of sequence s, whose window is [j0, L).  A
// sequence's span takes n = ceil(span / split_len) splits: all full but the
// last, or (a.eq_split) all of q = ceil(span / n) positions but the last,
// where q >= n keeps the last split non-empty (otherwise the former).
struct SeqSpan {
  int L, j0, pb, pe;
};

__device__ __forceinline__ SeqSpan split_span(const DecodeArgs& a, uint32_t s, uint32_t split) {
  SeqSpan r;
  r.L = a.seq_lens[s];
  r.j0 = (a.window != 0u && r.L > int(a.window)) ? r.L - int(a.window) : 0;
  int sl = int(a.split_len);
  const int span = r.L - r.j0;
  if (a.eq_split && span > 0) {
    const int n = (span + sl - 1) / sl, q = (span + n - 1) / n;
    if (q >= n) sl = q;  // n splits of q positions (q >= n: split n - 1 is not empty)
  }
  r.pb = r.j0 + int(split) * sl;
  r.pe = min(r.L, r.pb + sl);
  return r;
}

// Chunked prefill: tile `tile` of sequence s holds queries qrow0 .. qrow0 +
// nq - 1 (rows of q and out), at positions p0 .. p0 + nq - 1, and attends the
// key range [lo, hi); split k of the tile covers [lo + k split_len,
// min(hi, lo + (k + 1) split_len)).  A chunk longer than its sequence (the
// caller's contract excludes it) leaves its leading tiles empty.
struct PrefillTile {
  int qrow0, nq, p0, lo, hi;
};

__device__ __forceinline__ PrefillTile prefill_tile(const DecodeArgs& a, uint32_t s, uint32_t tile) {
  PrefillTile t;
  const int q0 = a.query_start[s], q1 = a.query_start[s + 1];
  t.qrow0 = q0 + int(tile * a.qt);
  t.nq = min(int(a.qt), q1 - t.qrow0);
  t.p0 = a.seq_lens[s] - (q1 - q0) + int(tile * a.qt);
  if (t.nq <= 0 || t.p0 < 0) {
    t.nq = 0;
    t.lo = t.hi = 0;
    return t;
  }
  t.hi = t.p0 + t.nq;
  t.lo = a.window != 0u ? max(0, t.p0 + 1 - int(a.window)) : 0;
  return t;
}

struct Tile {
  uint32_t s, g, split;
  bool valid;
};

// (sequence, split, kv head) of this workgroup; `per_seq` units per sequence.
// Units are numbered split-major (unit = split * S + sequence): the units of
// one split index rotate over the XCDs, and so do the (fewer) later splits
// that only long sequences have.  With a.order, the workgroups take the units
// in its order instead (the sparse score kernel: longest first).
//
// MODE 1 keeps the kv heads of a unit on one XCD; MODE 0 numbers workgroups
// unit-major (wg = unit * Hkv + head), so that with 8 kv heads each XCD takes
// one head of every unit.
template <int MODE>
__device__ __forceinline__ Tile unit_tile(const DecodeArgs& a, uint32_t per_seq) {
  uint32_t unit, head;
  Tile t;
  if constexpr (MODE == 1) {
    t.valid = xcd_unit_tile(blockIdx.x, a.num_seqs * per_seq, a.num_kv_heads, unit, head);
  } else {
    unit = blockIdx.x / a.num_kv_heads;
    head = blockIdx.x % a.num_kv_heads;
    t.valid = unit < a.num_seqs * per_seq;
  }
  if (t.valid && a.order) unit = a.order[unit];
  t.g = head;
  t.s = unit % a.num_seqs;
  t.split = unit / a.num_seqs;
  return t;
}

template <int KF, int HD, int G>
struct PrologueSmem {
  float q[Fmt<KF>::turbo ? G : 1][Fmt<KF>::turbo ? HD : 1];
  float kcen[16];
  float vcen[16];
  uint64_t kbase[kMaxPages];  // byte offset of each page of the split in the K pool
  uint64_t vbase[kMaxPages];  // ... and in the V pool
  uint32_t page[kMaxPages];   // page ids (for candidate records)
};

// Page ids of the split, codebooks, and (turbo K) the rotated query in LDS;
// then the lane's query registers.
template <int KF, int VF, int HD, int G, int D, int NW = kWaves>
__device__ __forceinline__ void prologue(const DecodeArgs& a, PrologueSmem<KF, HD, G>& sm, uint32_t s,
                                         uint32_t g, int pb, int pe, int t, QReg<KF, D, G>& q) {
  const int tid = threadIdx.x;
  const uint16_t* qg = a.q + uint64_t(row_query(a, s)) * a.q_stride + uint64_t(g) * G * HD;
  q.scsh = scale_shift<D, Fmt<KF>::sgb == 2 ? 2 : 1>(t);
  q.vsh = scale_shift<D, Fmt<VF>::sgb == 2 ? 2 : 1>(t);
  if constexpr (!Fmt<KF>::turbo) {
    // bf16 query pairs straight from memory (the score scale is applied
    // later); requested first so that their latency overlaps the page table's
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4* src = reinterpret_cast<const uint4*>(qg + h * HD + t * D);
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
        const uint4 v = src[i];
        q.qp[h][4 * i] = v.x; q.qp[h][4 * i + 1] = v.y; q.qp[h][4 * i + 2] = v.z; q.qp[h][4 * i + 3] = v.w;
      }
    }
  }
  // The page ids of the split (one per thread), the turbo K query rows (in
  // 16-byte pieces, rotated in LDS below) and the centroids are all requested
  // before any is stored: one round trip.
  static_assert(kMaxPages <= NW * kWave, "a page id per thread");
  const int first = pb >> a.log2_bs;
  const int n = ((pe - 1) >> a.log2_bs) - first + 1;
  const int32_t* bt = a.block_tables + uint64_t(row_table(a, s)) * a.max_blocks + first;
  const uint32_t page = tid < n ? uint32_t(bt[tid]) : 0u;
  // (turbo K: query row h goes to wave h % NW, lane l taking elements
  // l * QE ... l * QE + QE - 1)
  const int lane = tid & 63, wq = tid >> 6;
  constexpr int QE = HD / kWave, QR = Fmt<KF>::turbo ? (G + NW - 1) / NW : 1;
  float qx[QR][QE];
  if constexpr (Fmt<KF>::turbo) {
#pragma unroll
    for (int k = 0; k < QR; ++k) {
      const int h = wq + k * NW;
      const uint16_t* src = qg + (h < G ? h : 0) * HD + lane * QE;
      if constexpr (QE == 4) {
        const uint2 v = *reinterpret_cast<const uint2*>(src);
        qx[k][0] = __uint_as_float(v.x << 16); qx[k][1] = __uint_as_float(v.x & 0xFFFF0000u);
        qx[k][2] = __uint_as_float(v.y << 16); qx[k][3] = __uint_as_float(v.y & 0xFFFF0000u);
      } else if constexpr (QE == 2) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(src);
        qx[k][0] = __uint_as_float(v << 16); qx[k][1] = __uint_as_float(v & 0xFFFF0000u);
      } else {
        qx[k][0] = bf16_bits_to_float(*src);
      }
    }
  }
  float kc = 0.0f, vc = 0.0f;
  if constexpr (Fmt<KF>::cb) kc = tid < (1 << Fmt<KF>::bits) ? a.cb.centroid[KF - 2][tid & 15] : 0.0f;
  if constexpr (Fmt<VF>::cb) vc = tid < (1 << Fmt<VF>::bits) ? a.cb.centroid[VF - 2][tid & 15] : 0.0f;
  if (tid < 16) {
    if constexpr (Fmt<KF>::cb) sm.kcen[tid] = kc;
    if constexpr (Fmt<VF>::cb) sm.vcen[tid] = vc;
  }
  if (tid < n) {
    sm.kbase[tid] = uint64_t(page) * a.k_stride;
    sm.vbase[tid] = uint64_t(page) * a.v_stride;
    sm.page[tid] = page;
  }
  if constexpr (!Fmt<KF>::turbo) {
    // Every load so far is complete before the chunk loop starts: the loop
    // then begins with only chunk loads outstanding on every path, and the
    // compiler's wait counts inside it stay exact.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  } else {
    // unnormalized WHT of every query row in its wave's registers (1/sqrt(d)
    // goes into the score scale); an NVFP4 K side is scored against the query
    // as it is
#pragma unroll
    for (int k = 0; k < QR; ++k) {
      const int h = wq + k * NW;
      if constexpr (Fmt<KF>::rot) wave_wht<QE>(qx[k], lane, 1.0f);
      if (h < G) {
#pragma unroll
        for (int i = 0; i < QE; ++i) sm.q[h][lane * QE + i] = qx[k][i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < D; ++i) q.qf[h][i] = sm.q[h][t * D + i];
  }
}

// Load one 16-position chunk (starting at c, a multiple of 16) for a lane.
// Every load is issued unconditionally: a position outside [pb, pe) reads
// the clamped position's bytes (always inside a page of this split) and is
// masked afterwards.  Loads without branches let the compiler keep the next
// chunk's loads in flight while the current chunk is computed.
template <int KF, int VF, int HD, int G, int D, bool LOAD_V>
__device__ __forceinline__ void load_chunk(const DecodeArgs& a, const PrologueSmem<KF, HD, G>& sm, int first, int c,
                                           int pb, int pe, uint32_t g, int t, int r,
                                           Raw<KF, D> (&kr)[Geo<HD, D>::U], Raw<VF, D> (&vr)[Geo<HD, D>::U],
                                           bool (&ok)[Geo<HD, D>::U]) {
  using GE = Geo<HD, D>;
  const uint32_t bmask = (1u << a.log2_bs) - 1u;
#pragma unroll
  for (int u = 0; u < GE::U; ++u) {
    const int j = c + u * GE::P + r;
    ok[u] = j >= pb && j < pe;
    const int jc = min(max(j, pb), pe - 1);
    const int bi = (jc >> a.log2_bs) - first;
    const uint32_t row = (uint32_t(jc) & bmask) * a.num_kv_heads + g;
    load_lane<KF, HD, GE::D>(a.k_cache + sm.kbase[bi], row, t, a.k_data, kr[u]);
    if constexpr (LOAD_V) load_lane<VF, HD, GE::D>(a.v_cache + sm.vbase[bi], row, t, a.v_data, vr[u]);
  }
}

template <int F, int D>
__device__ __forceinline__ void mask_raw(Raw<F, D>& r, bool ok) {
#pragma unroll
  for (int i = 0; i < Raw<F, D>::words; ++i) r.w[i] = ok ? r.w[i] : 0u;
  r.sc = ok ? r.sc : 0u;
}

// Scores (log2 units, -inf outside the split) of a loaded chunk.
template <int KF, int HD, int G, int D>
__device__ __forceinline__ void chunk_scores(const QReg<KF, D, G>& q, const float* kcen, float qscale,
                                             const Raw<KF, D> (&kr)[Geo<HD, D>::U], const bool (&ok)[Geo<HD, D>::U],
                                             float (&sc)[Geo<HD, D>::U][G]) {
  using GE = Geo<HD, D>;
#pragma unroll
  for (int u = 0; u < GE::U; ++u) {
    float part[G];
    lane_scores<KF, GE::D, G>(q, kr[u], kcen, part);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float v = group_sum<GE::T>(part[h]) * qscale;
      sc[u][h] = ok[u] ? v : -INFINITY;
    }
  }
}

// ------------------------------------------------------------------ dense split

template <int KF, int VF, int HD, int G>
struct SplitSmem {
  PrologueSmem<KF, HD, G> pro;
  float red[kWaves][G][HD + 2];
};

template <int G, int D>
struct DenseState {
  float m[G], l[G], acc[G][D];
};

template <int KF, int VF, int HD, int G, int D>
__device__ __forceinline__ void dense_chunk(const Raw<KF, D> (&kr)[Geo<HD, D>::U],
                                            const Raw<VF, D> (&vr)[Geo<HD, D>::U],
                                            const bool (&ok)[Geo<HD, D>::U], const QReg<KF, D, G>& q,
                                            const float* kcen, const float* vcen, float qscale,
                                            DenseState<G, D>& st) {
  using GE = Geo<HD, D>;
  float sc[GE::U][G];
  chunk_scores<KF, HD, G, D>(q, kcen, qscale, kr, ok, sc);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = sc[0][h];
#pragma unroll
    for (int u = 1; u < GE::U; ++u) mx = fmaxf(mx, sc[u][h]);
    if (mx > st.m[h]) {
      const float alpha = fast_exp2(st.m[h] - mx);  // 0 while m is -inf
      st.l[h] *= alpha;
#pragma unroll
      for (int i = 0; i < GE::D; ++i) st.acc[h][i] *= alpha;
      st.m[h] = mx;
    }
  }
#pragma unroll
  for (int u = 0; u < GE::U; ++u) {
    Raw<VF, GE::D> vm = vr[u];
    mask_raw(vm, ok[u]);  // a masked position adds 0 * (finite value)
    float x[GE::D], sq;
    v_values<VF, GE::D>(vm, vcen, x, sq, q.vsh);  // V lanes hold the same dims as K lanes
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p = ok[u] ? fast_exp2(sc[u][h] - st.m[h]) : 0.0f;
      st.l[h] += p;
      const float pw = p * sq;
#pragma unroll
      for (int i = 0; i < GE::D; ++i) st.acc[h][i] = fmaf(pw, x[i], st.acc[h][i]);
    }
  }
}

template <int KF, int VF, int HD, int G>
__global__ __launch_bounds__(kWaves * kWave) void split_kernel(const DecodeArgs a) {
  constexpr int D = LaneDims<G>::dense;
  using GE = Geo<HD, D>;
  constexpr int T = GE::T;
  __shared__ SplitSmem<KF, VF, HD, G> sm;
  const Tile tl = unit_tile<KVQ_TILE_DENSE>(a, a.nsplit);
  if (!tl.valid) return;
  const SeqSpan sp = split_span(a, tl.s, tl.split);
  if (sp.pb >= sp.L) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int t = lane % T, r = lane / T;
  QReg<KF, D, G> q;
  prologue<KF, VF, HD, G, D>(a, sm.pro, tl.s, tl.g, sp.pb, sp.pe, t, q);
  const float qscale = a.qk_scale * (Fmt<KF>::rot ? a.wht_scale : 1.0f);
  const int first = sp.pb >> a.log2_bs;

  DenseState<G, D> st;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = -INFINITY;
    st.l[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < D; ++i) st.acc[h][i] = 0.0f;
  }

  // Chunk n of the wave sits in buffer n % NB and is loaded NB - 1 chunks
  // ahead, every load inside the loop (the first NB - 1 uses are of empty,
  // all-masked buffers); whole rounds of NB chunks, one exit at the bottom (a
  // chunk past the end is all masked and reads the clamped last position).
  constexpr int NB = KVQ_DENSE_BUFS;
  Raw<KF, D> kb[NB][GE::U];
  Raw<VF, D> vb[NB][GE::U];
  bool ob[NB][GE::U];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int u = 0; u < GE::U; ++u) {
      zero_raw(kb[i][u]);
      zero_raw(vb[i][u]);
      ob[i][u] = false;
    }
  constexpr int step = kWaves * kChunk;
  int c = (sp.pb & ~(kChunk - 1)) + w * kChunk;  // next chunk to load
  if (c < sp.pe) {
    const int rounds = ((sp.pe - 1 - c) / step + 2 * NB - 1) / NB;  // covers chunks + NB - 1 uses
    for (int it = 0; it < rounds; ++it) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        load_chunk<KF, VF, HD, G, D, true>(a, sm.pro, first, c, sp.pb, sp.pe, tl.g, t, r, kb[(i + NB - 1) % NB],
                                           vb[(i + NB - 1) % NB], ob[(i + NB - 1) % NB]);
        dense_chunk<KF, VF, HD, G, D>(kb[i], vb[i], ob[i], q, sm.pro.kcen, sm.pro.vcen, qscale, st);
        c += step;
      }
    }
  }

  // merge the lane slots of the wave (same dims, different positions)
#pragma unroll
  for (int off = T; off < kWave; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(st.m[h], off);
      const float lo = __shfl_xor(st.l[h], off);
      const float M = fmaxf(st.m[h], mo);
      const float a1 = st.m[h] > -INFINITY ? fast_exp2(st.m[h] - M) : 0.0f;
      const float a2 = mo > -INFINITY ? fast_exp2(mo - M) : 0.0f;
      st.l[h] = st.l[h] * a1 + lo * a2;
#pragma unroll
      for (int i = 0; i < D; ++i) st.acc[h][i] = st.acc[h][i] * a1 + __shfl_xor(st.acc[h][i], off) * a2;
      st.m[h] = M;
    }
  }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int i = 0; i < D; ++i) sm.red[w][h][t * D + i] = st.acc[h][i];
      if (t == 0) {
        sm.red[w][h][HD] = st.m[h];
        sm.red[w][h][HD + 1] = st.l[h];
      }
    }
  }
  __syncthreads();
  const uint64_t base = (uint64_t(tl.s) * a.num_kv_heads + tl.g) * a.nsplit + tl.split;
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

// Log-sum-exp merge of the ns split partials of one output row, by one wave
// (lane l: elements l * E ...): split k has its (max, sum) pair at ml + k *
// mls and its unnormalized row at part + k * ps.  M = max m_k, Z = sum_k
// 2^(m_k - M) l_k, and o[d] = scale / Z * sum_k 2^(m_k - M) part_k[d];
// splits with m_k = -inf (nothing attended) add nothing.  A row of at most B
// splits is read in one batch (one wait); a longer row walks its splits B at
// a time in three loops, each batch's loads issued before any is used.  The
// additions keep the split order, so the result does not depend on B or on
// the path.
template <int E, int B>
__device__ __forceinline__ void merge_row(const float* ml, uint32_t mls, const float* part, uint32_t ps, int ns,
                                          float scale, float (&o)[E]) {
  if (ns <= B) {
    float m[B], l[B], v[B][E];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const bool in = u < ns;
      m[u] = in ? ml[uint64_t(u) * mls] : -INFINITY;
      l[u] = in ? ml[uint64_t(u) * mls + 1] : 0.0f;
#pragma unroll
      for (int i = 0; i < E; ++i) v[u][i] = in ? part[uint64_t(u) * ps + i] : 0.0f;
    }
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < B; ++u) M = fmaxf(M, m[u]);
    float sum = 0.0f, acc[E];
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (m[u] > -INFINITY) {
        const float wgt = fast_exp2(m[u] - M);
        sum += wgt * l[u];
#pragma unroll
        for (int i = 0; i < E; ++i) acc[i] += wgt * v[u][i];
      }
    const float inv = sum > 0.0f ? scale / sum : 0.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) o[i] = acc[i] * inv;
    return;
  }
  float M = -INFINITY;
  for (int k0 = 0; k0 < ns; k0 += B) {
    float m[B];
#pragma unroll
    for (int u = 0; u < B; ++u) m[u] = k0 + u < ns ? ml[uint64_t(k0 + u) * mls] : -INFINITY;
#pragma unroll
    for (int u = 0; u < B; ++u) M = fmaxf(M, m[u]);
  }
  float sum = 0.0f;
  for (int k0 = 0; k0 < ns; k0 += B) {
    float m[B], l[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const bool in = k0 + u < ns;
      m[u] = in ? ml[uint64_t(k0 + u) * mls] : -INFINITY;
      l[u] = in ? ml[uint64_t(k0 + u) * mls + 1] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (m[u] > -INFINITY) sum += fast_exp2(m[u] - M) * l[u];
  }
  const float inv = sum > 0.0f ? scale / sum : 0.0f;
  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.0f;
  for (int k0 = 0; k0 < ns; k0 += B) {
    float m[B], v[B][E];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const bool in = k0 + u < ns;
      m[u] = in ? ml[uint64_t(k0 + u) * mls] : -INFINITY;
#pragma unroll
      for (int i = 0; i < E; ++i) v[u][i] = in ? part[uint64_t(k0 + u) * ps + i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (m[u] > -INFINITY) {
        const float wgt = fast_exp2(m[u] - M);
#pragma unroll
        for (int i = 0; i < E; ++i) acc[i] += wgt * v[u][i];
      }
  }
#pragma unroll
  for (int i = 0; i < E; ++i) o[i] = acc[i] * inv;
}

// Dense path: one wave per output row (sequence, q head), four rows per
// workgroup, combines the split partials with log-sum-exp weights, then
// applies the fp8 V scale and the inverse rotation.
template <int HD, bool VROT>
__global__ __launch_bounds__(256) void merge_kernel(const DecodeArgs a, int G) {
  constexpr int E = HD / kWave;
  const uint64_t rowq = uint64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);  // s * num_q_heads + q head
  if (rowq >= uint64_t(a.num_seqs) * a.num_q_heads) return;
  const uint32_t s = uint32_t(rowq / a.num_q_heads), hq = uint32_t(rowq % a.num_q_heads);
  const uint32_t g = hq / G, h = hq % G;
  if (a.vrow && a.vrow[2 * s] < 0) return;  // a prefill row without a query: no output row
  const SeqSpan sp = split_span(a, s, 0);
  const int span = sp.L - sp.j0;
  const int ns = span > 0 ? (span + int(a.split_len) - 1) / int(a.split_len) : 0;
  const int lane = threadIdx.x & 63;
  const uint64_t row = ((uint64_t(s) * a.num_kv_heads + g) * a.nsplit) * G + h;  // split 0's row
  float o[E];
  merge_row<E, 16>(a.ml + row * 2, uint32_t(G) * 2, a.part + row * HD + lane * E, uint32_t(G) * HD, ns,
                   a.v_scale, o);
  if constexpr (VROT) wave_wht<E>(o, lane, a.wht_scale);
  float* dst = a.out + (uint64_t(row_query(a, s)) * a.num_q_heads + hq) * HD + lane * E;
#pragma unroll
  for (int i = 0; i < E; ++i) dst[i] = o[i];
}

// LDS writes of a wave visible to its own lanes (no workgroup barrier)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace kvq

#include "kvq_decode_mfma.h"

namespace kvq {

// ------------------------------------------------------------------ sparse V

// The unit (split * S + sequence) at rank r of the longest-first order of a
// launch's units, computed by a whole workgroup of NW waves (every workgroup
// of the launch computes the same order: a counting sort over 16-position
// buckets, longest first, units of one bucket by increasing index), for
// launches of at most NW * 64 units.  This replaces the sorting launch ahead
// of the kernel.  `lds` holds at least 2 * NB + NW + 2 words and is free.
template <int NW>
__device__ uint32_t inline_unit_order(const DecodeArgs& a, uint32_t r, uint32_t* lds) {
  constexpr int NB = kMaxSparseSplit / kChunk + 1;
  uint32_t* cnt = lds;          // [NB] units per bucket
  uint32_t* start = lds + NB;   // [NB] first rank of each bucket
  uint32_t* wcnt = start + NB;  // [NW] units of the found bucket per wave
  uint32_t* res = wcnt + NW;    // [0] the found bucket, [1] the unit
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint32_t n = a.num_seqs * a.nsplit;
  int b = -1;
  if (uint32_t(tid) < n) {
    const SeqSpan sp = split_span(a, uint32_t(tid) % a.num_seqs, uint32_t(tid) / a.num_seqs);
    const int len = sp.pe > sp.pb ? sp.pe - sp.pb : 0;
    b = min((len + kChunk - 1) / kChunk, NB - 1);
  }
  for (int i = tid; i < NB; i += NW * kWave) cnt[i] = 0u;
  __syncthreads();
  if (b >= 0) atomicAdd(&cnt[b], 1u);
  __syncthreads();
  if (tid < kWave) {  // first rank of each bucket, the longest bucket first (one wave's scan)
    constexpr int BPL = (NB + kWave - 1) / kWave;
    uint32_t c[BPL], sum = 0;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {  // lane l takes buckets NB - 1 - l * BPL - i
      const int bb = NB - 1 - (lane * BPL + i);
      c[i] = bb >= 0 ? cnt[bb] : 0u;
      sum += c[i];
    }
    uint32_t pre = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const uint32_t v = __shfl_up(pre, off);
      if (lane >= off) pre += v;
    }
    uint32_t at = pre - sum;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const int bb = NB - 1 - (lane * BPL + i);
      if (bb >= 0) start[bb] = at;
      at += c[i];
    }
  }
  __syncthreads();
  for (int i = tid; i < NB; i += NW * kWave)
    if (cnt[i] > 0u && start[i] <= r && r < start[i] + cnt[i]) res[0] = uint32_t(i);
  __syncthreads();
  const int bf = int(res[0]);
  const uint64_t m = __ballot(b == bf);
  if (lane == 0) wcnt[w] = uint32_t(__popcll(m));
  __syncthreads();
  if (b == bf) {
    uint32_t k = uint32_t(__popcll(m & ((1ull << lane) - 1ull)));
    for (int ww = 0; ww < w; ++ww) k += wcnt[ww];
    if (start[bf] + k == r) res[1] = uint32_t(tid);
  }
  __syncthreads();
  const uint32_t unit = res[1];
  __syncthreads();  // the area is the score array, written next
  return unit;
}

template <int KF, int HD, int G, bool MF>
struct ScoreSmem {
  static constexpr int NW = score_waves(MF);
  PrologueSmem<KF, HD, G> pro;
  float sc[kMaxSparseSplit * G];
  float wm[NW][G];  // per-wave max and sum of exp2(score - max)
  float wz[NW][G];
  // matrix-core scores of a codebook K side: centroids of every pair of adjacent codes
  f32x2 kpair[MF && Fmt<KF>::cb ? 1 << (2 * Fmt<KF>::bits) : 1];
};

// Scores of one split; stores the split's (max, sum) and the candidate
// positions whose split-local weight exceeds thr * (1 - 1e-4).  The global
// normalizer is at least the split's, so a position that is not a candidate
// has global weight <= thr and is provably skipped.
//
// Wave w scores chunks w, w + kWaves, ... of 16 positions; after the loop it
// reduces its own scores (max, sum), one barrier combines the waves, and each
// wave then compacts its own candidates into its own segment of the record
// list (no further barriers).  A record is (page id, position, G log2 scores).
//
// MF: the K side is scored on the matrix cores as in the dense kernel (lane l
// takes quarter l / 16 of position l % 16's row, v_mfma_f32_4x4x1_16b_f32
// against the rotated query, a permlane reduce-scatter of the quarters), so
// lane l ends with the score of head l / 16 at position l % 16; the rest is
// the same.  The VALU version spent 62 instructions per (position, kv head)
// on turbo3 K at head_dim 256 (code unpacking, lookups, four heads' FMAs,
// 16-lane sums).
template <int KF, int HD, int G, bool MF>
__global__ __launch_bounds__(score_waves(MF) * kWave) void scores_kernel(const DecodeArgs a) {
  constexpr int D = LaneDims<G>::score;
  using GE = Geo<HD, D>;
  constexpr int T = GE::T;
  constexpr int RS = cand_record_words(G);
  static_assert(!MF || mfma_scores_ok(KF, HD, G), "matrix-core scores");
  constexpr int NW = int(score_waves(MF));  // waves, one record segment each
  __shared__ ScoreSmem<KF, HD, G, MF> sm;
  Tile tl = unit_tile<KVQ_TILE_SCORES>(a, a.nsplit);
  if (!tl.valid) return;
  if (a.lpt_inline) {  // the unit of this rank in the longest-first order, found by the workgroup
    const uint32_t unit = inline_unit_order<NW>(a, tl.split * a.num_seqs + tl.s, reinterpret_cast<uint32_t*>(sm.sc));
    tl.s = unit % a.num_seqs;
    tl.split = unit / a.num_seqs;
  }
  const SeqSpan sp = split_span(a, tl.s, tl.split);
  if (sp.pb >= sp.L) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int t = lane % T, r = lane / T;
  QReg<KF, D, G> q;
  prologue<KF, KVQ_BF16, HD, G, D, NW>(a, sm.pro, tl.s, tl.g, sp.pb, sp.pe, t, q);
  const float qscale = a.qk_scale * (Fmt<KF>::rot ? a.wht_scale : 1.0f);
  const int first = sp.pb >> a.log2_bs;

  float mloc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mloc[h] = -INFINITY;
  constexpr int step = NW * kChunk;
  const int cs = sp.pb & ~(kChunk - 1);
  if constexpr (MF) {
    using MG = MfmaGeo<KF, KVQ_BF16, HD, 4>;
    if constexpr (Fmt<KF>::cb) {  // from the centroids the prologue put in LDS
      constexpr int BITS = Fmt<KF>::bits;
      for (int e = tid; e < (1 << (2 * BITS)); e += NW * kWave) {
        sm.kpair[e].x = sm.pro.kcen[e & ((1 << BITS) - 1)];
        sm.kpair[e].y = sm.pro.kcen[e >> BITS];
      }
    }
    // operand A: the rotated query of head lane % 4 over quarter lane / 16
    float qf[MG::KQ];
    {
      const int h = lane & 3;
#pragma unroll
      for (int k = 0; k < MG::KQ; ++k) qf[k] = h < G ? sm.pro.q[h][(lane >> 4) * MG::KQ + k] : 0.0f;
    }
    __builtin_amdgcn_s_waitcnt(0);  // the chunk loop starts with only its own loads outstanding
    __syncthreads();
    const uint32_t nkv = a.num_kv_heads, bmask = (1u << a.log2_bs) - 1u;
    const uint32_t koff = ((uint32_t(lane) & 15u) * nkv + tl.g) * MG::RBK + (uint32_t(lane) >> 4) * MG::KQB;
    const uint32_t ksb = (uint32_t(lane) >> 4) * MG::KGQ * MG::KSG;
    const uint32_t ksoff = a.k_data + ((uint32_t(lane) & 15u) * nkv + tl.g) * (HD / 16 * MG::KSG) + (ksb & ~3u);
    const int ksh = int(ksb & 3u) * 8;
    const int clast = (sp.pe - 1) & ~(kChunk - 1);
    const int head = lane >> 4;
    struct KChunk {
      uint32_t k[MG::KQB / 4];
      uint32_t ks[MG::KSW];
    };
    auto load = [&](int c, KChunk& ck) {
      const int cl = min(c, clast);  // past the end: reread the last chunk (all masked)
      const int pg = (cl >> a.log2_bs) - first;
      const uint64_t kpage = uniform_u64(sm.pro.kbase[pg]);
      const uint32_t within = uint32_t(cl) & bmask;
      load_words<MG::KQB>(a.k_cache + kpage + uint64_t(within) * nkv * MG::RBK + koff, ck.k);
#pragma unroll
      for (int i = 0; i < MG::KSW; ++i)
        ck.ks[i] = load4(a.k_cache + kpage + uint64_t(within) * nkv * (HD / 16 * MG::KSG) + ksoff + 4 * i);
    };
    auto consume = [&](int c, const KChunk& ck) {
      const f32x4 d = mfma_qk_turbo<KF, HD, KVQ_SCORE_LOOKUPS>(ck.k, ck.ks, ksh, qf, sm.kpair);
      const int j = c + (lane & 15);
      const bool ok = j >= sp.pb && j < sp.pe;
      // the swaps exchange values between the lanes of one position, which
      // share the mask: a swap never reads an inactive lane
      const float sc = ok ? quarter_sum(d) * qscale : -INFINITY;
#pragma unroll
      for (int h = 0; h < G; ++h)
        if (h == head) mloc[h] = fmaxf(mloc[h], sc);
      if (ok && head < G) sm.sc[(j - sp.pb) * G + head] = sc;
    };
    // the wave's chunks c, c + step, ...; chunk n sits in buffer n % NB and
    // is loaded NB - 1 chunks ahead of its use, as in the VALU loop below
    constexpr int NB = KVQ_SCORE_MFMA_BUFS;
    KChunk kb[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
#pragma unroll
      for (int k = 0; k < MG::KQB / 4; ++k) kb[i].k[k] = 0u;
#pragma unroll
      for (int k = 0; k < MG::KSW; ++k) kb[i].ks[k] = 0u;
    }
    int c = cs + w * kChunk;
    if (c < sp.pe) {
      const int rounds = ((sp.pe - 1 - c) / step + 2 * NB - 1) / NB;
      for (int it = 0; it < rounds; ++it) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          load(c, kb[(i + NB - 1) % NB]);
          consume(c - (NB - 1) * step, kb[i]);
          c += step;
        }
      }
    }
  } else {
    auto consume = [&](int c, const Raw<KF, D>(&kr)[GE::U], const bool(&ok)[GE::U]) {
      float sc[GE::U][G];
      chunk_scores<KF, HD, G, D>(q, sm.pro.kcen, qscale, kr, ok, sc);
#pragma unroll
      for (int u = 0; u < GE::U; ++u) {
        const int j = c + u * GE::P + r;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          mloc[h] = fmaxf(mloc[h], sc[u][h]);
          if (ok[u] && t == 0) sm.sc[(j - sp.pb) * G + h] = sc[u][h];
        }
      }
    };
    // The wave's chunks c, c + step, ...; chunk n sits in buffer n % NB and is
    // loaded NB - 1 chunks ahead of its use.  Every load is issued inside the
    // loop (the first NB - 1 uses are of empty, all-masked buffers), and the
    // loop runs whole rounds of NB chunks with one exit at the bottom; a chunk
    // past the end is all masked (its loads read the clamped last position, an
    // L2 hit).  With one loop entry state and no early exit the compiler keeps
    // NB - 1 chunks in flight across the back edge.
    constexpr int NB = KVQ_SCORE_BUFS;
    Raw<KF, D> kb[NB][GE::U];
    Raw<KVQ_BF16, D> vdummy[GE::U];
    bool ob[NB][GE::U];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int u = 0; u < GE::U; ++u) {
        zero_raw(kb[i][u]);
        ob[i][u] = false;
      }
    int c = cs + w * kChunk;  // next chunk to load; the one used trails by NB - 1
    if (c < sp.pe) {
      const int rounds = ((sp.pe - 1 - c) / step + 2 * NB - 1) / NB;  // covers chunks + NB - 1 uses
      for (int it = 0; it < rounds; ++it) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          load_chunk<KF, KVQ_BF16, HD, G, D, false>(a, sm.pro, first, c, sp.pb, sp.pe, tl.g, t, r,
                                                 kb[(i + NB - 1) % NB], vdummy, ob[(i + NB - 1) % NB]);
          consume(c - (NB - 1) * step, kb[i], ob[i]);
          c += step;
        }
      }
    }
  }
  // the wave's own scores: lane (sub, pos) visits position pos of every
  // kSubs-th chunk the wave scored
  wave_lds_sync();
  constexpr int kSubs = kWave / kChunk;
  constexpr int lap = kSubs * step;
  const int sub = lane / kChunk, pos = lane % kChunk;
  float mw[G], zl[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mw[h] = group_max<kWave>(mloc[h]);
    zl[h] = 0.0f;
  }
  for (int cw = cs + w * kChunk; cw < sp.pe; cw += lap) {
    const int j = cw + sub * step + pos;
    if (j >= sp.pb && j < sp.pe) {
#pragma unroll
      for (int h = 0; h < G; ++h) zl[h] += fast_exp2(sm.sc[(j - sp.pb) * G + h] - mw[h]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float zw = group_sum<kWave>(zl[h]);
    if (lane == 0) {
      sm.wm[w][h] = mw[h];
      sm.wz[w][h] = zw;
    }
  }
  __syncthreads();
  float M[G], cut[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float m = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) m = fmaxf(m, sm.wm[ww][h]);
    float z = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float mk = sm.wm[ww][h];
      if (mk > -INFINITY) z += fast_exp2(mk - m) * sm.wz[ww][h];
    }
    M[h] = m;
    cut[h] = a.thr * (1.0f - 1e-4f) * z;
    if (tid == h) {
      const uint64_t base = (uint64_t(tl.s) * a.num_kv_heads + tl.g) * a.nsplit + tl.split;
      a.ml[(base * G + h) * 2] = m;
      a.ml[(base * G + h) * 2 + 1] = z;
    }
  }
  // candidates of this wave, compacted in its own segment
  const uint64_t seg = ((uint64_t(tl.s) * a.num_kv_heads + tl.g) * a.nsplit + tl.split) * NW + w;
  uint32_t* rec = a.crec + seg * a.seg_cap * RS;
  int nw = 0;
  for (int cw = cs + w * kChunk; cw < sp.pe; cw += lap) {
    const int j = cw + sub * step + pos;
    bool cand = false;
    float sv[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sv[h] = 0.0f;
    if (j >= sp.pb && j < sp.pe) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        sv[h] = sm.sc[(j - sp.pb) * G + h];
        cand |= fast_exp2(sv[h] - M[h]) > cut[h];
      }
    }
    const uint64_t bal = __ballot(cand);
    if (cand) {
      const int k = nw + __popcll(bal & ((1ull << lane) - 1ull));
      uint32_t rw[RS];
      rw[0] = sm.pro.page[(j >> a.log2_bs) - first];
      rw[1] = uint32_t(j);
#pragma unroll
      for (int h = 0; h < G; ++h) rw[2 + h] = __float_as_uint(sv[h]);
#pragma unroll
      for (int i = 2 + G; i < RS; ++i) rw[i] = 0u;
      uint4* dst = reinterpret_cast<uint4*>(rec + uint64_t(k) * RS);
#pragma unroll
      for (int i = 0; i < RS / 4; ++i) dst[i] = make_uint4(rw[4 * i], rw[4 * i + 1], rw[4 * i + 2], rw[4 * i + 3]);
    }
    nw += __popcll(bal);
  }
  if (lane == 0) a.cnt[seg] = nw;
}

constexpr int kMaxStatSplits = 64;  // splits whose stats the V pass stages in LDS at once
constexpr int kVWaves = KVQ_VWAVES;  // waves of a V-pass workgroup
constexpr int kSegBatch = kWave;     // segments a V wave indexes at once (one per lane)
constexpr int kStageUnroll = 2;      // staged V rows a lane slot reads from LDS at once

// The V pass uses 8 dims per lane (more rows side by side, fewer registers).
template <int HD>
struct VGeo {
  static constexpr int D = 8;
  static constexpr int T = HD / D;
  static constexpr int P = kWave / T;
};

template <int G>
__device__ __forceinline__ void load_record(const uint32_t* src, uint32_t (&rw)[cand_record_words(G)]) {
  const uint4* p = reinterpret_cast<const uint4*>(src);
#pragma unroll
  for (int i = 0; i < int(cand_record_words(G)) / 4; ++i) {
    const uint4 v = p[i];
    rw[4 * i] = v.x;
    rw[4 * i + 1] = v.y;
    rw[4 * i + 2] = v.z;
    rw[4 * i + 3] = v.w;
  }
}

// Staging of kept V rows in LDS: each lane reads GPL granules of CK bytes of
// one row (LPR lanes per row), RPP rows per pass; rows sit CS bytes apart,
// followed by their scale bytes (turbo) SB bytes apart.
template <int VF, int HD>
struct VStage {
  static constexpr int RB = HD * Fmt<VF>::bits / 8;                 // code bytes per row
  static constexpr int SB = HD / 16 * Fmt<VF>::sgb;                // scale bytes per row
  static constexpr int CK = RB % 16 == 0 ? 16 : RB % 8 == 0 ? 8 : 4;  // load granule
  static constexpr int NCK = RB / CK;
  static constexpr int GPL = NCK < 4 ? NCK : 4;
  static constexpr int LPR = (NCK + GPL - 1) / GPL;
  static constexpr int RPP = kWave / LPR;
  static constexpr int CS = (RB + 15) / 16 * 16;
  static constexpr int WORDS = (RPP * CS + RPP * SB + 15) / 16 * 4 + 4;  // + slack for the 3-bit reads
};

template <int VF, int HD, int G>
struct SparseSmem {
  float vcen[16];
  float mz[G][2];                     // global (max, 1/sum) per head
  float st[kMaxStatSplits][G][2];     // split stats being reduced
  int pre[kVWaves][kSegBatch];        // per wave: inclusive prefix of its batch's segment counts
  struct Kept {
    uint64_t vb;   // byte offset of the V page
    uint32_t row;  // row (offset * Hkv + kv head) in the page
    float p[G];    // kept weights (0 for heads that drop the position)
  };
  union {
    struct {
      Kept kept[kVWaves][kWave];
      __attribute__((aligned(16))) uint32_t rows[kVWaves][VStage<VF, HD>::WORDS];
    } live;
    float red[kVWaves / 2][G][HD];
  } u;
};

// A lane's D dims of staged row q (LDS words `rw`), as load_lane would give them.
template <int F, int HD, int D>
__device__ __forceinline__ void staged_lane(const uint32_t* rw, int q, int t, Raw<F, D>& r) {
  using VS = VStage<F, HD>;
  constexpr int B = Raw<F, D>::bytes;
  const int byte = q * VS::CS + t * B;
  if constexpr (B % 4 == 0) {
#pragma unroll
    for (int i = 0; i < B / 4; ++i) r.w[i] = rw[byte / 4 + i];
  } else if constexpr (B == 2) {
    r.w[0] = (rw[byte / 4] >> ((byte & 3) * 8)) & 0xFFFFu;
  } else {
    // 3-bit codes: the two aligned words that cover them
    const uint64_t v = (uint64_t(rw[byte / 4 + 1]) << 32 | rw[byte / 4]) >> ((byte & 3) * 8);
    r.w[0] = uint32_t(v);
    if constexpr (Raw<F, D>::words > 1) r.w[1] = uint32_t(v >> 32) & 0xFFFFu;
  }
  if constexpr (Fmt<F>::turbo)
    r.sc = rw[(VS::RPP * VS::CS + q * VS::SB + ((((t * D) / 16) * Fmt<F>::sgb) & ~3)) / 4];
  else r.sc = 0;
}

// Lane `lane` copies its part of kept row (lane / LPR) of the pass into LDS.
template <int VF, int HD, typename KeptT>
__device__ __forceinline__ void stage_rows(const DecodeArgs& a, const KeptT* kept, int nrow, int lane, uint32_t* rw) {
  using VS = VStage<VF, HD>;
  const int qr = lane / VS::LPR, part = lane % VS::LPR;
  if (qr >= nrow) return;
  const uint8_t* blk = a.v_cache + kept[qr].vb;
  const uint32_t row = kept[qr].row;
  const uint8_t* src = blk + uint64_t(row) * VS::RB;
  uint32_t g[VS::GPL][VS::CK / 4];
  uint32_t sc[VS::SB > 0 ? VS::SB / 4 : 1];
#pragma unroll
  for (int j = 0; j < VS::GPL; ++j) {
    const int c = part * VS::GPL + j;
    if (c < VS::NCK) {
      const uint8_t* p = src + c * VS::CK;
      if constexpr (VS::CK == 16) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(p);
        g[j][0] = v.x; g[j][1] = v.y; g[j][2] = v.z; g[j][3] = v.w;
      } else if constexpr (VS::CK == 8) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(p);
        g[j][0] = v.x; g[j][1] = v.y;
      } else {
        g[j][0] = *reinterpret_cast<const uint32_t*>(p);
      }
    }
  }
  if constexpr (VS::SB > 0) {
    const uint8_t* p = blk + a.v_data + uint64_t(row) * VS::SB;
    if (part == 0) {
      if constexpr (VS::SB % 16 == 0) {
#pragma unroll
        for (int i = 0; i < VS::SB / 16; ++i) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(p + 16 * i);
          sc[4 * i] = v.x; sc[4 * i + 1] = v.y; sc[4 * i + 2] = v.z; sc[4 * i + 3] = v.w;
        }
      } else if constexpr (VS::SB == 8) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(p);
        sc[0] = v.x; sc[1] = v.y;
      } else {
        sc[0] = *reinterpret_cast<const uint32_t*>(p);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < VS::GPL; ++j) {
    const int c = part * VS::GPL + j;
    if (c < VS::NCK) {
      const int wo = (qr * VS::CS + c * VS::CK) / 4;
#pragma unroll
      for (int i = 0; i < VS::CK / 4; ++i) rw[wo + i] = g[j][i];
    }
  }
  if constexpr (VS::SB > 0) {
    if (part == 0) {
      const int wo = (VS::RPP * VS::CS + qr * VS::SB) / 4;
#pragma unroll
      for (int i = 0; i < VS::SB / 4; ++i) rw[wo + i] = sc[i];
    }
  }
}

// The kept rows of a wave's list (nk of them) into acc: their bytes go to
// LDS (every row of a pass requested at once), then each lane slot reads its
// dims of its rows from there.
template <int VF, int HD, int G, typename KeptT>
__device__ __forceinline__ void accumulate_kept(const DecodeArgs& a, const float* vcen, const KeptT* kept, int nk,
                                                uint32_t* rows, uint32_t vsh, float (&acc)[G][VGeo<HD>::D]) {
  using GE = VGeo<HD>;
  using VS = VStage<VF, HD>;
  constexpr int D = GE::D, T = GE::T, P = GE::P;
  const int lane = threadIdx.x & 63, t = lane % T, r = lane / T;
  for (int q0 = 0; q0 < nk; q0 += VS::RPP) {
    const int nrow = min(VS::RPP, nk - q0);
    stage_rows<VF, HD>(a, &kept[q0], nrow, lane, rows);
    wave_lds_sync();
    // kStageUnroll rows per lane slot at a time, their LDS reads issued together
    for (int q = r; q < nrow; q += P * kStageUnroll) {
      Raw<VF, D> vr[kStageUnroll];
#pragma unroll
      for (int u = 0; u < kStageUnroll; ++u) {
        const int qu = q + u * P;
        staged_lane<VF, HD, D>(rows, qu < nrow ? qu : q, t, vr[u]);
      }
#pragma unroll
      for (int u = 0; u < kStageUnroll; ++u) {
        const int qu = q + u * P;
        const bool ok = qu < nrow;
        float x[D], sq;
        v_values<VF, D>(vr[u], vcen, x, sq, vsh);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float pw = (ok ? kept[q0 + qu].p[h] : 0.0f) * sq;
#pragma unroll
          for (int i = 0; i < D; ++i) acc[h][i] = fmaf(pw, x[i], acc[h][i]);
        }
      }
    }
    wave_lds_sync();
  }
}

// The G output rows of (sequence s, kv head g) from their sums in LDS (o, G x
// HD): x v_scale, rotated back (a rotated V side) and stored.
template <int HD, int G, bool VROT, int NT>
__device__ __forceinline__ void store_sparse_rows(const DecodeArgs& a, float* o, uint32_t s, uint32_t g) {
  const int tid = threadIdx.x;
  if constexpr (VROT) {
    // inverse rotation of every head's row (the orthonormal WHT is its own inverse)
    for (int h2 = 1; h2 < HD; h2 <<= 1) {
      for (int i = tid; i < G * HD / 2; i += NT) {
        const int hh = i / (HD / 2), k = i % (HD / 2);
        const int lo = hh * HD + (k / h2) * 2 * h2 + (k % h2);
        const float x = o[lo], y = o[lo + h2];
        o[lo] = x + y;
        o[lo + h2] = x - y;
      }
      __syncthreads();
    }
  }
  float* dst = a.out + (uint64_t(s) * a.num_q_heads + uint64_t(g) * G) * HD;
  for (int i = tid; i < G * HD; i += NT) dst[i] = VROT ? o[i] * a.wht_scale : o[i];
}

// The end of a sparse-V workgroup (part `part` of sequence s, kv head g): the
// lane slots' and the waves' partial sums added in a fixed order.  With one
// part the result is scaled by the fp8 V scale, rotated back (turbo V) and
// stored; with several, each part stores its sum for sparse_v_merge_kernel.
template <int VF, int HD, int G, typename Smem>
__device__ __forceinline__ void sparse_v_finish(const DecodeArgs& a, Smem& sm, float (&acc)[G][VGeo<HD>::D],
                                                uint32_t s, uint32_t g, uint32_t part) {
  using GE = VGeo<HD>;
  constexpr int D = GE::D, T = GE::T;
  constexpr int NT = kVWaves * kWave;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = lane % T, r = lane / T;
  // lane slots of a wave hold the same dims: add them
#pragma unroll
  for (int off = T; off < kWave; off <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < D; ++i) acc[h][i] += __shfl_xor(acc[h][i], off);
  // waves, in a fixed order: the upper half stores, the lower half adds its own
  constexpr int HW = kVWaves / 2;
  __syncthreads();  // the reduction area overlays the kept lists
  if (w >= HW && r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < D; ++i) sm.u.red[w - HW][h][t * D + i] = acc[h][i];
  }
  __syncthreads();
  if (w < HW && r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < D; ++i) sm.u.red[w][h][t * D + i] += acc[h][i];
  }
  __syncthreads();
  float* o = &sm.u.red[0][0][0];  // row h of the result at o + h * HD
  if (a.vparts > 1) {
    float* mine = a.vpart + ((uint64_t(s) * a.num_kv_heads + g) * a.vparts + part) * (G * HD);
    for (int i = tid; i < G * HD; i += NT) {
      const int h = i / HD, d = i % HD;
      float v = 0.0f;
#pragma unroll
      for (int ww = 0; ww < HW; ++ww) v += sm.u.red[ww][h][d];
      mine[i] = v;
    }
    return;
  }
  for (int i = tid; i < G * HD; i += NT) {
    const int h = i / HD, d = i % HD;
    float v = 0.0f;
#pragma unroll
    for (int ww = 0; ww < HW; ++ww) v += sm.u.red[ww][h][d];
    o[i] = v * a.v_scale;
  }
  __syncthreads();
  store_sparse_rows<HD, G, Fmt<VF>::rot, NT>(a, o, s, g);
}

// The V parts' sums of one output row (sequence, q head) per wave, added in
// part order, x v_scale, rotated back (a rotated V side: butterflies inside
// the lane for the low index bits, then lane exchanges) and stored.  Lane l
// holds dims l * E ... l * E + E - 1.
template <int HD, bool VROT>
__global__ __launch_bounds__(256) void sparse_v_merge_kernel(const DecodeArgs a, uint32_t G) {
  constexpr int E = HD / kWave;
  constexpr int kMaxParts = int(kMaxVParts);
  const uint64_t row = uint64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);  // s * num_q_heads + q head
  if (row >= uint64_t(a.num_seqs) * a.num_q_heads) return;
  const int lane = threadIdx.x & 63;
  const uint64_t pair = row / G;
  const float* src = a.vpart + (pair * a.vparts * G + row % G) * HD + lane * E;
  // every part's values requested at once (parts past the last re-read it)
  float v[kMaxParts][E];
#pragma unroll
  for (int k = 0; k < kMaxParts; ++k) {
    const float* p = src + uint64_t(min(uint32_t(k), a.vparts - 1u)) * G * HD;
    if constexpr (E == 4) {
      const float4 f = *reinterpret_cast<const float4*>(p);
      v[k][0] = f.x; v[k][1] = f.y; v[k][2] = f.z; v[k][3] = f.w;
    } else if constexpr (E == 2) {
      const float2 f = *reinterpret_cast<const float2*>(p);
      v[k][0] = f.x; v[k][1] = f.y;
    } else {
      v[k][0] = *p;
    }
  }
  float x[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    x[i] = v[0][i];
#pragma unroll
    for (int k = 1; k < kMaxParts; ++k)
      if (uint32_t(k) < a.vparts) x[i] += v[k][i];
    x[i] *= a.v_scale;
  }
  if constexpr (VROT) wave_wht<E>(x, lane, a.wht_scale);
  float* dst = a.out + row * HD + lane * E;
  if constexpr (E == 4) *reinterpret_cast<float4*>(dst) = make_float4(x[0], x[1], x[2], x[3]);
  else if constexpr (E == 2) *reinterpret_cast<float2*>(dst) = make_float2(x[0], x[1]);
  else dst[0] = x[0];
}

// a.vparts workgroups of kVWaves waves per (sequence, kv head) do the V side
// of the sparse path and write the output.  The score kernel left one record
// segment per (split, wave); V wave v of part p (wave W = p * kVWaves + v of
// the NW = vparts * kVWaves) takes segments W, W + NW, ... (the score kernel's
// waves scored interleaved chunks, so the work is evenly spread).  The global softmax statistics come from the split statistics;
// each lane reads one record, keeps a position for head h when its exact
// global weight exceeds the threshold, and a ballot compacts the kept ones
// into LDS; the wave's lane slots then stream their V rows.  The segment
// counts, a first record per lane (read ahead of the counts) and the split
// statistics are all requested at once.  At the end the waves' partial sums
// are added in LDS in a fixed order, scaled by the fp8 V scale, rotated back
// (turbo V) and stored.
// At most 128 registers per lane: two workgroups per CU stay resident.
template <int VF, int HD, int G>
__global__ __launch_bounds__(kVWaves * kWave) __attribute__((amdgpu_waves_per_eu(4))) void sparse_v_kernel(
    const DecodeArgs a) {
  using GE = VGeo<HD>;
  constexpr int D = GE::D, T = GE::T, P = GE::P;
  constexpr int RS = cand_record_words(G);
  constexpr int NT = kVWaves * kWave;
  __shared__ SparseSmem<VF, HD, G> sm;
  uint32_t s, g;
  // the parts of a (sequence, kv head) run on one XCD
  const uint32_t part = (blockIdx.x >> 3) % a.vparts;
  const uint32_t tile = (blockIdx.x & 7u) | (((blockIdx.x >> 3) / a.vparts) << 3);
  if (!xcd_unit_tile(tile, a.num_seqs, a.num_kv_heads, s, g)) return;
  const SeqSpan sp = split_span(a, s, 0);
  const int span = sp.L - sp.j0;
  const int ns = span > 0 ? (span + int(a.split_len) - 1) / int(a.split_len) : 0;
  const uint64_t sbase = (uint64_t(s) * a.num_kv_heads + g) * a.nsplit;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = lane % T, r = lane / T;
  const int nseg_all = ns * int(a.segs);  // (split, score wave) segments
  const int NW = int(a.vparts) * kVWaves, W = int(part) * kVWaves + w;
  const int nseg = nseg_all > W ? (nseg_all - W + NW - 1) / NW : 0;  // this wave's
  // requests that do not depend on each other go out first: the counts of the
  // wave's first batch of segments, a first record per lane, the statistics
  const int myc0 = lane < nseg ? a.cnt[sbase * a.segs + W + NW * lane] : 0;
  uint32_t spec[RS];
  if (W < nseg_all) {  // the wave's first segment exists (the last head's would lie past the workspace)
    load_record<G>(a.crec + ((sbase * a.segs + W) * a.seg_cap + lane) * RS, spec);
  } else {
#pragma unroll
    for (int i = 0; i < RS; ++i) spec[i] = 0u;
  }
  if (tid < 16) {
    if constexpr (Fmt<VF>::cb) sm.vcen[tid] = tid < (1 << Fmt<VF>::bits) ? a.cb.centroid[VF - 2][tid] : 0.0f;
  }
  float runm = -INFINITY, runz = 0.0f;  // (threads < G) running stats of head tid
  for (int kb = 0; kb < ns; kb += kMaxStatSplits) {
    const int nk = min(kMaxStatSplits, ns - kb);
    for (int i = tid; i < nk * G; i += NT) {
      const int k = i / G, h = i % G;
      sm.st[k][h][0] = a.ml[((sbase + kb + k) * G + h) * 2];
      sm.st[k][h][1] = a.ml[((sbase + kb + k) * G + h) * 2 + 1];
    }
    __syncthreads();
    if (tid < G) {
      float mx = runm;
      for (int k = 0; k < nk; ++k) mx = fmaxf(mx, sm.st[k][tid][0]);
      float z = runm > -INFINITY ? runz * fast_exp2(runm - mx) : 0.0f;
      for (int k = 0; k < nk; ++k) {
        const float mk = sm.st[k][tid][0];
        if (mk > -INFINITY) z += fast_exp2(mk - mx) * sm.st[k][tid][1];
      }
      runm = mx;
      runz = z;
    }
    __syncthreads();
  }
  if (tid < G) {
    sm.mz[tid][0] = runm;
    sm.mz[tid][1] = runz > 0.0f ? 1.0f / runz : 0.0f;
  }
  __syncthreads();
  float M[G], iz[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    M[h] = sm.mz[h][0];
    iz[h] = sm.mz[h][1];
  }
  float acc[G][D];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < D; ++i) acc[h][i] = 0.0f;
  const uint32_t bmask = (1u << a.log2_bs) - 1u;
  const uint32_t vsh = scale_shift<D, Fmt<VF>::sgb == 2 ? 2 : 1>(t);
  using VS = VStage<VF, HD>;
  auto& kept = sm.u.live.kept[w];
  uint32_t* rows = sm.u.live.rows[w];
  // the wave's segments, kSegBatch at a time (segment i of the wave is
  // (split, score wave) number W + NW * i of the sequence and kv head)
  for (int sb = 0; sb < nseg; sb += kSegBatch) {
    const int nb = min(kSegBatch, nseg - sb);
    const int myc = sb == 0 ? myc0 : (lane < nb ? a.cnt[sbase * a.segs + W + NW * (sb + lane)] : 0);
    int pre = myc;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int v = __shfl_up(pre, off);
      if (lane >= off) pre += v;
    }
    wave_lds_sync();
    if (lane < nb) sm.pre[w][lane] = pre;
    wave_lds_sync();
    const int total = __shfl(pre, nb - 1);
    const int c0 = __shfl(myc, 0);
    // record gi of the batch (segment k: the number of segments whose
    // inclusive prefix is <= gi), or zeros past the end
    auto fetch = [&](int gi, uint32_t (&rw)[RS]) {
#pragma unroll
      for (int i = 0; i < RS; ++i) rw[i] = 0u;
      if (gi < total) {
        int k = 0;
#pragma unroll
        for (int bb = kSegBatch / 2; bb > 0; bb >>= 1)
          if (k + bb < nb && sm.pre[w][k + bb - 1] <= gi) k += bb;
        const int off = gi - (k > 0 ? sm.pre[w][k - 1] : 0);
        const uint64_t seg = sbase * a.segs + W + NW * (sb + k);
        load_record<G>(a.crec + (seg * a.seg_cap + off) * RS, rw);
      }
    };
    // rounds of 64 records; the next round's records are requested before
    // the current round's V rows, so the two latencies overlap
    uint32_t rw[RS];
    if (sb == 0 && lane < c0) {
#pragma unroll
      for (int i = 0; i < RS; ++i) rw[i] = spec[i];
    } else {
      fetch(lane, rw);
    }
    for (int i0 = 0; i0 < total; i0 += kWave) {
      // 1. one record per lane -> keep decisions, compacted into the wave's LDS list
      const bool ok = i0 + lane < total;
      float p[G];
      bool any = false;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pv = fast_exp2(__uint_as_float(rw[2 + h]) - M[h]) * iz[h];
        p[h] = (ok && pv > a.thr) ? pv : 0.0f;
        any |= p[h] > 0.0f;
      }
      const uint64_t bal = __ballot(any);
      if (any) {
        const int kk = __popcll(bal & ((1ull << lane) - 1ull));
        kept[kk].vb = uint64_t(rw[0]) * a.v_stride;
        kept[kk].row = (rw[1] & bmask) * a.num_kv_heads + g;
#pragma unroll
        for (int h = 0; h < G; ++h) kept[kk].p[h] = p[h];
      }
      fetch(i0 + kWave + lane, rw);
      const int nk = __popcll(bal);
      wave_lds_sync();
      // 2. the kept rows' V values into acc
      accumulate_kept<VF, HD, G>(a, sm.vcen, kept, nk, rows, vsh, acc);
    }
  }
  sparse_v_finish<VF, HD, G>(a, sm, acc, s, g, part);
}


// ------------------------------------------------------------------ dispatch

// Dense split kernel of a (K, V, head_dim, G) instance: the matrix-core one
// where its operand sizes allow it and a 16-position chunk lies in one page,
// else the VALU one.
template <int KF, int VF, int HD, int G>
hipError_t launch_split_one(const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  if constexpr (KVQ_DENSE_MFMA && MfmaGeo<KF, VF, HD, G>::ok) {
    if (a.log2_bs >= 4) {
      const uint32_t nw = mfma_unit_waves(a.num_kv_heads, mfma_waves_cap<KF, G>());
      const uint64_t n = mfma_grid(uint64_t(a.num_seqs) * a.nsplit, a.num_kv_heads / nw);
      hipLaunchKernelGGL((split_mfma_kernel<KF, VF, HD, G>), dim3(uint32_t(n)), dim3(nw * kWave), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((split_kernel<KF, VF, HD, G>), dim3(nwg), dim3(kWaves * kWave), 0, st, a);
  return hipGetLastError();
}

template <int KF, int VF, int HD>
hipError_t launch_split_g(int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  switch (g) {
    case 1: return launch_split_one<KF, VF, HD, 1>(a, nwg, st);
    case 2: return launch_split_one<KF, VF, HD, 2>(a, nwg, st);
    case 4: return launch_split_one<KF, VF, HD, 4>(a, nwg, st);
    case 8: return launch_split_one<KF, VF, HD, 8>(a, nwg, st);
    default: return hipErrorInvalidValue;
  }
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
    case KVQ_TURBO8: return launch_split_hd<KF, KVQ_TURBO8>(hd, g, a, nwg, st);
    case KVQ_NVFP4: return launch_split_hd<KF, KVQ_NVFP4>(hd, g, a, nwg, st);
    default: return hipErrorInvalidValue;
  }
}

// The score kernel of a (K, head_dim, G) instance: the matrix-core scores
// where they apply (block_size >= 16), else the VALU ones.
template <int KF, int HD, int G>
void launch_scores_one(const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  if constexpr (KVQ_SCORE_MFMA && mfma_scores_ok(KF, HD, G)) {
    if (scores_on_mfma(KF, HD, G, 1u << a.log2_bs)) {
      hipLaunchKernelGGL((scores_kernel<KF, HD, G, true>), dim3(nwg), dim3(score_waves(true) * kWave), 0, st, a);
      return;
    }
  }
  hipLaunchKernelGGL((scores_kernel<KF, HD, G, false>), dim3(nwg), dim3(score_waves(false) * kWave), 0, st, a);
}

template <int KF, int HD>
hipError_t launch_scores_g(int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  switch (g) {
    case 1: launch_scores_one<KF, HD, 1>(a, nwg, st); break;
    case 2: launch_scores_one<KF, HD, 2>(a, nwg, st); break;
    case 4: launch_scores_one<KF, HD, 4>(a, nwg, st); break;
    case 8: launch_scores_one<KF, HD, 8>(a, nwg, st); break;
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
