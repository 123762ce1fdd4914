// Chunked prefill on the bf16 matrix cores (kernel template; instantiated in
// kvq_prefill.hip and kvq_prefill_rot.hip): tiles of many (query, head) rows
// share every K/V chunk they stage.
//
// "combs_models/kv.rs", attend: the chunk's queries attend the cached
// positions with the causal mask aligned to the bottom right (query p sees
// keys 0 .. p), softmax(q K^T * scale) V, GQA by repeating each kv head for
// its G query heads.  "spark_runtime/kv_cache.rs": chunked-prefill coverage
// of the quantized formats, and is_wht_rotated: a rotated V side gives the
// rotated output, rotated back here.  A sliding window W keeps keys
// p - W < j <= p of query p.
//
// Work decomposition (MI355X):
//   * A workgroup takes one (sequence, kv head) and a tile of ROWS (query,
//     head) rows: ROWS / G consecutive queries with all G heads of the kv
//     head (row r = query r / G, head r % G).  It walks the tile's whole key
//     range in chunks of NK positions and writes the finished output rows:
//     no partials, no merge pass.
//   * Each chunk is dequantized once, by all 256 threads, into LDS: K
//     row-major in bf16, V transposed (dim-major) in bf16, with a second
//     "lo" plane (the bf16 rounding of value - hi) where a V value is not a
//     bf16 value (turbo2/3/4 centroids and turbo8 values times their group
//     scale).  A thread takes 4 consecutive keys x 8 consecutive dims, so
//     the global reads of 16 neighbouring threads cover a whole row.
//   * The four waves then each run 32 rows (16 at head_dim 256):
//       S^T = K Q^T on v_mfma_f32_16x16x32_bf16: K from LDS (operand A),
//             the queries in registers (operand B, loaded once);
//       online softmax in the instruction's output layout (lane = query
//             row, registers = keys); the maximum over the four lane groups
//             by lane swaps;
//       O^T += V^T P^T on the same instruction: V^T from LDS (operand A),
//             P^T straight from the softmax registers (operand B) as a
//             bf16 hi + lo pair.  The products hi*hi + hi*lo (+ lo*hi for
//             a V side with a lo plane) carry about 16 significant bits of
//             each operand into fp32 accumulators.
//     K from bf16, fp8 and NVFP4 sides is exact in bf16, so their scores
//     are those of fp32 arithmetic on the stored values.  A rotated K side
//     (turbo2/3/4, turbo8) is scored against the unnormalized WHT of the
//     query, which is not a bf16 value: both operands are fp32 (keys staged
//     as fp32 rows, the rotated query in registers) on
//     v_mfma_f32_16x16x4_f32.  Split into bf16 pieces, the rounding of the
//     keys and query (about 2^-18 of each product) times the sum of the
//     products' magnitudes, some 80 times a typical score, is amplified by
//     large V values past the parity bar.  Those waves take 16 rows.
//   * The bf16 MFMA pairs its A and B operands' k elements lane by lane,
//     so the order of keys inside a 32-key step only has to agree between
//     P^T and V^T: lane group j holds keys 4j .. 4j + 3 and 16 + 4j ..
//     16 + 4j + 3 of the step, the V^T rows store keys in that order, and
//     P^T needs no lane exchange.
//   * LDS rows are XOR-swizzled in 16-byte units so that the operand reads
//     of 16 lanes (16 keys of one K unit, 16 dims of one V^T unit) fall on
//     distinct banks.
//   * Raw bytes of chunk n + 1 are loaded into registers while chunk n is
//     on the matrix cores; two barriers per chunk.
#pragma once

#include "kvq_decode.h"

namespace kvq {
namespace prefill {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

template <int KF, int HD>
struct TGeo {
  static constexpr bool KROT = Fmt<KF>::rot;       // rotated K: fp32 keys and rotated query
  static constexpr int NK = 8192 / HD;             // keys per chunk
  static constexpr int RW = HD <= 128 && !KROT ? 32 : 16;  // rows per wave
  static constexpr int QB = RW / 16;               // 16-row blocks per wave
  static constexpr int NW = 4;                     // waves
  static constexpr int ROWS = NW * RW;             // rows per workgroup
  static constexpr int DB = HD / 8;                // 8-dim blocks of a row
  static constexpr int KT = NK / 16;               // 16-key tiles of S^T
  static constexpr int KS = NK / 32;               // 32-key steps of P.V
  static constexpr int DS = HD / 32;               // 32-dim steps of Q.K
  static constexpr int OD = HD / 16;               // 16-dim blocks of O^T
  static_assert((NK / 4) * DB == NW * kWave, "one key quad x 8 dims per thread");
};

// Formats whose stored values (times their group scale) are bf16 values:
// bf16, fp8 (the per-tensor scale is applied to scores or outputs), NVFP4
// (E2M1 x E4M3: at most 6 significant bits).
template <int F>
struct Bf16Exact {
  static constexpr bool value = F == KVQ_BF16 || F == KVQ_FP8_E4M3 || F == KVQ_NVFP4;
};

template <int KF, int VF, int HD>
struct TileSmem {
  static constexpr int NK = TGeo<KF, HD>::NK;
  static constexpr int VP = Bf16Exact<VF>::value ? 1 : 2;
  // K rows: bf16 pairs, or fp32 values for a rotated K side
  __attribute__((aligned(16))) uint32_t kt[Fmt<KF>::rot ? NK * HD : NK * HD / 2];
  __attribute__((aligned(16))) uint32_t vt[VP][HD * NK / 2];
  f32x2 kpair[Fmt<KF>::cb ? 1 << (2 * Fmt<KF>::bits) : 1];
  f32x2 vpair[Fmt<VF>::cb ? 1 << (2 * Fmt<VF>::bits) : 1];
};

// Physical 16-byte unit of logical unit u in K row kappa / V^T row d.
// (fp32 K rows have HD / 4 >= 16 units: the key's low bits spread them)
__device__ __forceinline__ int kf_unit(int kappa, int u) { return u ^ (kappa & 15); }
template <int HD>
__device__ __forceinline__ int kt_unit(int kappa, int u) {
  if constexpr (HD / 8 >= 16) return u ^ (kappa & 15);
  else return u ^ ((kappa >> 1) & 7);
}
template <int HD>
__device__ __forceinline__ int vt_unit(int d, int u) {
  constexpr int UPR = 8192 / HD / 8;
  if constexpr (UPR >= 16) return u ^ ((d ^ (d >> 4)) & 15);
  else if constexpr (UPR == 8) return u ^ (((d >> 1) ^ (d >> 4)) & 7);
  else return u ^ (((d >> 2) ^ (d >> 4)) & 3);
}

// Column of key kappa of a chunk in the V^T rows (see the file comment).
__device__ __forceinline__ int vt_col(int kappa) {
  const int r = kappa & 31;
  return (kappa & ~31) + 8 * ((r & 15) >> 2) + 4 * (r >> 4) + (r & 3);
}

// One thread's raw bytes of one key: 8 dims of its K row and of its V row
// (+ the word holding the V group scale).  The words stay as loaded (a 2- or
// 3-bit piece inside its aligned words, a scale byte inside its word) and
// are shifted into place only where they are used: a shift right after the
// load would make the wave wait for the next chunk's bytes before working on
// the current one.
template <int F>
struct PieceWords {
  static constexpr int n = (8 * Fmt<F>::bits + 31) / 32;     // words of the piece
  static constexpr int raw = Fmt<F>::bits == 3 ? 2 : n;     // words as loaded
};

template <int F>
__device__ __forceinline__ void load_piece(const uint8_t* row, int b, uint32_t* w) {
  constexpr int bits = Fmt<F>::bits;
  if constexpr (bits == 16) {
    const u32x4 x = load16(row + 16 * b);
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else if constexpr (bits == 8) {
    const u32x2 x = load8(row + 8 * b);
    w[0] = x.x; w[1] = x.y;
  } else if constexpr (bits == 4) {
    w[0] = load4(row + 4 * b);
  } else if constexpr (bits == 2) {
    w[0] = load4(row + 4 * (b >> 1));
  } else {
    // 3 bytes at byte 3b: the two aligned words that cover them (at most 5
    // bytes past the row, still inside the block: rows, then the scales)
    const int base = (3 * b) & ~3;
    w[0] = load4(row + base);
    w[1] = load4(row + base + 4);
  }
}

// Bit offset of the piece inside its loaded words (2- and 3-bit codes).
template <int F>
__device__ __forceinline__ uint32_t piece_shift(int b) {
  constexpr int bits = Fmt<F>::bits;
  return bits == 2 ? 16u * uint32_t(b & 1) : bits == 3 ? 8u * uint32_t((3 * b) & 3) : 0u;
}

// The piece's words from the loaded ones.
template <int F>
__device__ __forceinline__ void piece_words(const uint32_t* r, uint32_t sh, uint32_t* w) {
  constexpr int bits = Fmt<F>::bits;
  if constexpr (bits == 2) {
    w[0] = (r[0] >> sh) & 0xFFFFu;
  } else if constexpr (bits == 3) {
    w[0] = uint32_t(((uint64_t(r[1]) << 32) | r[0]) >> sh) & 0xFFFFFFu;
  } else {
#pragma unroll
    for (int i = 0; i < PieceWords<F>::n; ++i) w[i] = r[i];
  }
}

// The word holding the group scale of dims 8b .. 8b + 7 of a row whose
// scales start at srow (turbo8: a bf16 word, else an E4M3 byte), as loaded;
// scale_shift gives the scale's bit offset in it.
template <int F, int HD>
__device__ __forceinline__ uint32_t load_scale(const uint8_t* srow, int b) {
  if constexpr (Fmt<F>::sgb == 0) {
    return 0u;
  } else {
    const int o = (b >> 1) * Fmt<F>::sgb;
    return load4(srow + (o & ~3));
  }
}
template <int F>
__device__ __forceinline__ uint32_t scale_shift(int b) {
  return 8u * uint32_t(((b >> 1) * Fmt<F>::sgb) & 3);
}

// The 8 values of a piece in fp32 (exact: products of at most 12
// significant bits).
template <int VF>
__device__ __forceinline__ void piece_values(const uint32_t* w, uint32_t sw, const f32x2* vpair, float (&x)[8]) {
  if constexpr (VF == KVQ_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else if constexpr (VF == KVQ_FP8_E4M3 || VF == KVQ_TURBO8) {
    const float sq = VF == KVQ_TURBO8 ? __uint_as_float(sw << 16) : 1.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(w[i]), false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(w[i]), true);
      x[4 * i] = lo.x * sq; x[4 * i + 1] = lo.y * sq; x[4 * i + 2] = hi.x * sq; x[4 * i + 3] = hi.y * sq;
    }
  } else {
    constexpr int B2 = 2 * Fmt<VF>::bits;
    const float sq = __builtin_amdgcn_cvt_f32_fp8(int(sw), 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x2 c = vpair[(w[0] >> (B2 * k)) & ((1u << B2) - 1u)];
      x[2 * k] = c.x * sq;
      x[2 * k + 1] = c.y * sq;
    }
  }
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}
__device__ __forceinline__ float lo_half(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float hi_half(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }

// max / sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (every lane active)
__device__ __forceinline__ float lanegroup_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float lanegroup_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Butterfly with the lane l ^ 16 (X = 16) or l ^ 32 (X = 32): the lane
// without the bit gets own + partner, the lane with it partner - own.
template <int X>
__device__ __forceinline__ float lane_butterfly(float x, int lane) {
  const auto p = X == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                         : __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const bool up = (lane & X) != 0;
  const float partner = __uint_as_float(up ? p[0] : p[1]);
  return up ? partner - x : x + partner;
}

__device__ __forceinline__ f32x4v mfma_bf16(u32x4 a, u32x4 b, f32x4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}

// Workgroup -> (sequence, kv head, split of the key range, tile).  The
// tiles of one (sequence, kv head, split) read the same keys at about the
// same time: they go to one XCD (workgroup i runs on XCD i % 8), and groups
// of 8 such units rotate over the XCDs.  With a.order the units come longest
// first, and a unit's tiles start from its last (longest key range), so
// short tiles fill the end of the launch.
struct TileId {
  uint32_t s, g, split, tile;
  bool valid;
};
__device__ __forceinline__ TileId tile_id(const DecodeArgs& a) {
  const uint32_t i = blockIdx.x, x = i & 7u, rest = i >> 3;
  uint32_t unit = (rest / a.ntiles) * 8u + x;
  if (a.order && unit < a.num_seqs * a.num_kv_heads * a.nsplit) unit = a.order[unit];  // longest units first
  const uint32_t sg = unit / a.nsplit;
  TileId t;
#if KVQ_PREFILL_TILE_DESC
  t.tile = a.ntiles - 1u - rest % a.ntiles;
#else
  t.tile = rest % a.ntiles;
#endif
  t.split = unit % a.nsplit;
  t.s = sg / a.num_kv_heads;
  t.g = sg % a.num_kv_heads;
  t.valid = sg < a.num_seqs * a.num_kv_heads;
  return t;
}

// Chunks of NK keys of a tile's range [lo, hi), aligned to NK; with splits
// (small grids), split k takes chunks [k cps, (k + 1) cps) of them.
template <int NK>
__device__ __forceinline__ int tile_chunks(const PrefillTile& pt) {
  return (pt.hi - (pt.lo / NK) * NK + NK - 1) / NK;
}

template <int KF, int VF, int HD>
__global__ __launch_bounds__(256, HD <= 128 ? 2 : 1) void prefill_tile_kernel(const DecodeArgs a, int G) {
  using TG = TGeo<KF, HD>;
  constexpr int NK = TG::NK, QB = TG::QB, KT = TG::KT, KS = TG::KS, DS = TG::DS, OD = TG::OD;
  constexpr bool KROT = TG::KROT;                   // rotated K: fp32 scores
  constexpr bool VLO = !Bf16Exact<VF>::value;       // a lo plane of V
  constexpr int KW = PieceWords<KF>::n, VW = PieceWords<VF>::n;
  constexpr int KRB = HD * Fmt<KF>::bits / 8, VRB = HD * Fmt<VF>::bits / 8;  // row bytes
  static_assert(KROT || Bf16Exact<KF>::value, "a K side is exact in bf16 unless rotated");
  static_assert(TG::NW * kWave == 256, "the launch bound");
  __shared__ TileSmem<KF, VF, HD> sm;

  const TileId id = tile_id(a);
  if (!id.valid) return;
  const PrefillTile pt = prefill_tile(a, id.s, id.tile);
  if (pt.nq <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, jg = lane >> 4;
  const uint32_t nkv = a.num_kv_heads, g = id.g;
  const uint32_t bs = 1u << a.log2_bs;

  // code-pair tables (index lo | hi << bits) of the table formats
  if constexpr (Fmt<VF>::cb) {
    constexpr int BITS = Fmt<VF>::bits;
    for (int e = tid; e < (1 << (2 * BITS)); e += TG::NW * kWave) {
      sm.vpair[e].x = a.cb.centroid[VF - 2][e & ((1 << BITS) - 1)];
      sm.vpair[e].y = a.cb.centroid[VF - 2][e >> BITS];
    }
  }
  if constexpr (Fmt<KF>::cb) {
    constexpr int BITS = Fmt<KF>::bits;
    for (int e = tid; e < (1 << (2 * BITS)); e += TG::NW * kWave) {
      sm.kpair[e].x = a.cb.centroid[KF - 2][e & ((1 << BITS) - 1)];
      sm.kpair[e].y = a.cb.centroid[KF - 2][e >> BITS];
    }
  }

  // the wave's query rows (operand B of S^T): row 16 qb + n16 of the wave;
  // rows past the tile's queries are zero.  bf16 operands: dims 32 st + 8 jg
  // .. + 7.  A rotated K side is scored on the fp32 matrix cores against the
  // unnormalized WHT of the query (its 1/sqrt(d) joins the score scale):
  // operand B of instruction (u, i) is dim 16 u + 4 jg + i, and the WHT runs
  // in registers (dim bits 0-1 in a lane, 2-3 across its lane groups, 4..
  // across registers).
  constexpr int QU = HD / 16;
  int rpos[QB];    // position of the row's query (valid rows)
  bool rok[QB];
  u32x4 qv[KROT ? 1 : QB][KROT ? 1 : DS];
  float qf[KROT ? QB : 1][KROT ? QU : 1][4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = TG::RW * wave + 16 * qb + n16;
    const int t = r / G, h = r % G;
    rok[qb] = t < pt.nq;
    rpos[qb] = pt.p0 + t;
    const uint16_t* qrow = a.q + uint64_t(pt.qrow0 + (rok[qb] ? t : 0)) * a.q_stride + (g * G + h) * HD;
    if constexpr (!KROT) {
#pragma unroll
      for (int st = 0; st < DS; ++st) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        qv[qb][st] = rok[qb] ? *reinterpret_cast<const u32x4*>(qrow + 32 * st + 8 * jg) : z;
      }
    } else {
      float (&x)[QU][4] = qf[KROT ? qb : 0];
#pragma unroll
      for (int u = 0; u < QU; ++u) {
        const u32x2 w = rok[qb] ? *reinterpret_cast<const u32x2*>(qrow + 16 * u + 4 * jg) : u32x2{0u, 0u};
        x[u][0] = lo_half(w.x); x[u][1] = hi_half(w.x); x[u][2] = lo_half(w.y); x[u][3] = hi_half(w.y);
        const float a0 = x[u][0] + x[u][1], a1 = x[u][0] - x[u][1], a2 = x[u][2] + x[u][3], a3 = x[u][2] - x[u][3];
        x[u][0] = a0 + a2; x[u][2] = a0 - a2; x[u][1] = a1 + a3; x[u][3] = a1 - a3;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[u][i] = lane_butterfly<16>(x[u][i], lane);
          x[u][i] = lane_butterfly<32>(x[u][i], lane);
        }
      }
#pragma unroll
      for (int hb = 1; hb < QU; hb <<= 1)
#pragma unroll
        for (int u = 0; u < QU; ++u)
          if ((u & hb) == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float y0 = x[u][i], y1 = x[u + hb][i];
              x[u][i] = y0 + y1;
              x[u + hb][i] = y0 - y1;
            }
          }
    }
  }

  // this thread's share of every chunk: keys 4 kq .. 4 kq + 3, dims 8 db ..
  const int kq = tid / TG::DB, db = tid % TG::DB;
  const int c_first = (pt.lo / NK) * NK;
  const int nch = tile_chunks<NK>(pt);
  const int cps = int(a.split_len) / NK;                         // chunks per split
  const int cbeg = a.nsplit > 1 ? int(id.split) * cps : 0;
  const int cend = a.nsplit > 1 ? min(nch, cbeg + cps) : nch;
  if (cbeg >= cend) return;  // a split past the tile's keys (uniform)
  const int32_t* table = a.block_tables + uint64_t(id.s) * a.max_blocks;
  auto page_of = [&](int c) -> uint32_t {  // page of the thread's key quad in chunk c (0: none)
    const int j = c_first + c * NK + 4 * kq;
    return (c < cend && j < pt.hi) ? uint32_t(table[j >> a.log2_bs]) : 0u;
  };
  uint32_t kr[4][PieceWords<KF>::raw], ks[4], vr[4][PieceWords<VF>::raw], vs[4];
  const uint32_t kpsh = piece_shift<KF>(db), vpsh = piece_shift<VF>(db);
  const uint32_t kssh = scale_shift<KF>(db), vssh = scale_shift<VF>(db);
  // the thread's four keys are consecutive rows of one page, nkv rows
  // apart: one 64-bit base per side and chunk, then 32-bit row steps
  constexpr uint32_t KSR = (HD / 16) * Fmt<KF>::sgb, VSR = (HD / 16) * Fmt<VF>::sgb;  // scale bytes per row
  const uint32_t kstep = nkv * KRB, vstep = nkv * VRB, ksstep = nkv * KSR, vsstep = nkv * VSR;
  auto load_chunk = [&](int c, uint32_t pid) {
    const uint32_t prow = (uint32_t(c_first + c * NK + 4 * kq) & (bs - 1u)) * nkv + g;
    const uint8_t* kb = a.k_cache + uint64_t(pid) * a.k_stride;
    const uint8_t* vb = a.v_cache + uint64_t(pid) * a.v_stride;
    const uint32_t ko = prow * KRB, vo = prow * VRB, kso = prow * KSR, vso = prow * VSR;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      load_piece<KF>(kb + (ko + t * kstep), db, kr[t]);
      ks[t] = load_scale<KF, HD>(kb + a.k_data + (kso + t * ksstep), db);
      load_piece<VF>(vb + (vo + t * vstep), db, vr[t]);
      vs[t] = load_scale<VF, HD>(vb + a.v_data + (vso + t * vsstep), db);
    }
  };

  uint32_t pid_next = page_of(cbeg + 1);
  load_chunk(cbeg, page_of(cbeg));

  // running reference m (log2 units) and the lane's share of the sum of
  // 2^(score - m) for query row n16 of each block.  The reference moves only
  // when a score exceeds it by more than 8 (weights stay below 2^8 before
  // normalization), so the accumulators are rescaled in the first chunks
  // and rarely after.  It starts finite: a chunk with every key masked
  // leaves everything unchanged.
  const float neg = -1.0e30f;
  float m[QB], lsum[QB];
  f32x4v acc[OD][QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = neg;
    lsum[qb] = 0.0f;
#pragma unroll
    for (int d = 0; d < OD; ++d) acc[d][qb] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const int lo_all = a.window ? pt.p0 + pt.nq - int(a.window) : 0;  // every row sees keys >= this
  const float qk = KROT ? a.qk_scale * a.wht_scale : a.qk_scale;

  __syncthreads();  // the code-pair tables are in LDS before any thread looks one up
  for (int c = cbeg; c < cend; ++c) {
    const int c0 = c_first + c * NK;
    __syncthreads();  // every wave is done with the previous chunk's LDS
    // dequantize this thread's share straight into LDS (nothing is held
    // across a barrier); keys outside [lo, hi) become zeros (only chunks at
    // the ends of the range hold such keys)
    const bool ends = c0 < pt.lo || c0 + NK > pt.hi;
    uint32_t vh[8][2], vl[VLO ? 8 : 1][2];
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {  // keys 2 pr, 2 pr + 1
      float x[2][8];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = 2 * pr + u, kappa = 4 * kq + t, j = c0 + kappa;
        const bool ok = !ends || (j >= pt.lo && j < pt.hi);
        uint32_t kp[KW], vp[VW];
        piece_words<KF>(kr[t], kpsh, kp);
        piece_words<VF>(vr[t], vpsh, vp);
        uint32_t ksw = ks[t] >> kssh, vsw = vs[t] >> vssh;
        if (ends) {
#pragma unroll
          for (int i = 0; i < KW; ++i) kp[i] = ok ? kp[i] : 0u;
#pragma unroll
          for (int i = 0; i < VW; ++i) vp[i] = ok ? vp[i] : 0u;
          ksw = ok ? ksw : 0u;
          vsw = ok ? vsw : 0u;
        }
        // the key's K row piece, straight to LDS
        if constexpr (KF == KVQ_BF16) {
          *reinterpret_cast<u32x4*>(&sm.kt[kappa * (HD / 2) + 4 * kt_unit<HD>(kappa, db)]) =
              u32x4{kp[0], kp[1], kp[2], kp[3]};
        } else if constexpr (KF == KVQ_FP8_E4M3) {
          *reinterpret_cast<u32x4*>(&sm.kt[kappa * (HD / 2) + 4 * kt_unit<HD>(kappa, db)]) =
              u32x4{fp8x2_to_bf16x2<false>(kp[0]), fp8x2_to_bf16x2<true>(kp[0]), fp8x2_to_bf16x2<false>(kp[1]),
                    fp8x2_to_bf16x2<true>(kp[1])};
        } else {
          float y[8];
          piece_values<KF>(kp, ksw, sm.kpair, y);
          if constexpr (KROT) {
#pragma unroll
            for (int v = 0; v < 2; ++v)
              *reinterpret_cast<u32x4*>(&sm.kt[kappa * HD + 4 * kf_unit(kappa, 2 * db + v)]) =
                  u32x4{__float_as_uint(y[4 * v]), __float_as_uint(y[4 * v + 1]), __float_as_uint(y[4 * v + 2]),
                        __float_as_uint(y[4 * v + 3])};
          } else {  // exact in bf16 (NVFP4)
            *reinterpret_cast<u32x4*>(&sm.kt[kappa * (HD / 2) + 4 * kt_unit<HD>(kappa, db)]) =
                u32x4{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7])};
          }
        }
        piece_values<VF>(vp, vsw, sm.vpair, x[u]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        vh[e][pr] = pack_bf16(x[0][e], x[1][e]);
        if constexpr (VLO) vl[e][pr] = pack_bf16(x[0][e] - lo_half(vh[e][pr]), x[1][e] - hi_half(vh[e][pr]));
      }
    }
    {
      const int col = vt_col(4 * kq);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * db + e;
        const int wi = d * (NK / 2) + 4 * vt_unit<HD>(d, col >> 3) + ((col & 7) >> 1);
        *reinterpret_cast<u32x2*>(&sm.vt[0][wi]) = u32x2{vh[e][0], vh[e][1]};
        if constexpr (VLO) *reinterpret_cast<u32x2*>(&sm.vt[VLO ? 1 : 0][wi]) = u32x2{vl[e][0], vl[e][1]};
      }
    }
    // the next chunk's raw bytes travel while this one is on the matrix cores
    if (c + 1 < cend) {
      load_chunk(c + 1, pid_next);
      pid_next = page_of(c + 2);  // after the loads that read the old value: no copy, no early wait
    }
    __syncthreads();

    // S^T = K Q^T (one K operand read serves every row block)
    f32x4v sc[KT][QB];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sc[kt][qb] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (!KROT) {
#pragma unroll
      for (int st = 0; st < DS; ++st)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const int kappa = 16 * kt + n16;
          const u32x4 ka =
              *reinterpret_cast<const u32x4*>(&sm.kt[kappa * (HD / 2) + 4 * kt_unit<HD>(kappa, 4 * st + jg)]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) sc[kt][qb] = mfma_bf16(ka, qv[KROT ? 0 : qb][KROT ? 0 : st], sc[kt][qb]);
        }
    } else {
      // fp32: one read gives the K operands of instructions (u, 0..3)
#pragma unroll
      for (int u = 0; u < QU; ++u)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const int kappa = 16 * kt + n16;
          const u32x4 ka = *reinterpret_cast<const u32x4*>(&sm.kt[kappa * HD + 4 * kf_unit(kappa, 4 * u + jg)]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              sc[kt][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(ka[i]), qf[KROT ? qb : 0][KROT ? u : 0][i],
                                                                sc[kt][qb], 0, 0, 0);
        }
    }
    // masks: only chunks that cross a row's causal limit or window start
    if (c0 + NK - 1 > pt.p0 || c0 < lo_all) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = c0 + 16 * kt + 4 * jg + i;
            const bool in = j <= rpos[qb] && (a.window == 0u || j > rpos[qb] - int(a.window));
            sc[kt][qb][i] = in ? sc[kt][qb][i] : -INFINITY;
          }
    }
    // the reference of each row moves if the chunk's maximum passes it by 8
    bool grow = false;
    float mc[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[kt][qb][i]);
      mc[qb] = lanegroup_max(mx) * qk;
      grow |= mc[qb] > m[qb] + 8.0f;
    }
    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float mn = mc[qb] > m[qb] + 8.0f ? mc[qb] : m[qb];
        const float alpha = fast_exp2(m[qb] - mn);
        m[qb] = mn;
        lsum[qb] *= alpha;
#pragma unroll
        for (int d = 0; d < OD; ++d) acc[d][qb] *= alpha;
      }
    }
    // O^T += V^T P^T, one 32-key step at a time: its weights as bf16 hi + lo
    // pairs (operand B), then the step's products
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 ph[QB], pl[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        uint32_t h[4], l[4];
        float rs = 0.0f;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[i] = fast_exp2(__builtin_fmaf(sc[2 * ks + u][qb][i], qk, -m[qb]));
            rs += p[i];
          }
          h[2 * u] = pack_bf16(p[0], p[1]);
          h[2 * u + 1] = pack_bf16(p[2], p[3]);
          l[2 * u] = pack_bf16(p[0] - lo_half(h[2 * u]), p[1] - hi_half(h[2 * u]));
          l[2 * u + 1] = pack_bf16(p[2] - lo_half(h[2 * u + 1]), p[3] - hi_half(h[2 * u + 1]));
        }
        lsum[qb] += rs;
        ph[qb] = u32x4{h[0], h[1], h[2], h[3]};
        pl[qb] = u32x4{l[0], l[1], l[2], l[3]};
      }
#pragma unroll
      for (int d = 0; d < OD; ++d) {
        const int row = 16 * d + n16;
        const int wi = row * (NK / 2) + 4 * vt_unit<HD>(row, 4 * ks + jg);
        const u32x4 va = *reinterpret_cast<const u32x4*>(&sm.vt[0][wi]);
        u32x4 vb = va;
        if constexpr (VLO) vb = *reinterpret_cast<const u32x4*>(&sm.vt[VLO ? 1 : 0][wi]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          acc[d][qb] = mfma_bf16(va, ph[qb], acc[d][qb]);
          acc[d][qb] = mfma_bf16(va, pl[qb], acc[d][qb]);
          if constexpr (VLO) acc[d][qb] = mfma_bf16(vb, ph[qb], acc[d][qb]);
        }
      }
    }
  }

  // epilogue.  Lane holds dims 16 d + 4 jg + i of query row n16 of each
  // block.  With splits: the row's reference m, its sum and unnormalized
  // output (rotated basis) for the merge.  Else: normalize, fp8 V scale,
  // inverse rotation, store.
  if (a.nsplit > 1) {
    const uint64_t unit = ((uint64_t(id.s) * a.ntiles + id.tile) * nkv + g) * a.nsplit + id.split;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l = lanegroup_sum(lsum[qb]);
      const uint64_t row = unit * TG::ROWS + uint64_t(TG::RW * wave + 16 * qb + n16);
      float* dst = a.part + row * HD + 4 * jg;
#pragma unroll
      for (int d = 0; d < OD; ++d) *reinterpret_cast<f32x4v*>(dst + 16 * d) = acc[d][qb];
      if (jg == 0) *reinterpret_cast<f32x2*>(a.ml + row * 2) = f32x2{m[qb], l};
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = lanegroup_sum(lsum[qb]);
    const float inv = a.v_scale / l;
#pragma unroll
    for (int d = 0; d < OD; ++d) acc[d][qb] *= inv;
    if constexpr (Fmt<VF>::rot) {
      // unnormalized WHT over dim bits 0-1 (registers), 2-3 (lane groups),
      // 4.. (blocks), then the orthonormal scale
#pragma unroll
      for (int d = 0; d < OD; ++d) {
        f32x4v& o = acc[d][qb];
        const float a0 = o[0] + o[1], a1 = o[0] - o[1], a2 = o[2] + o[3], a3 = o[2] - o[3];
        o[0] = a0 + a2; o[2] = a0 - a2; o[1] = a1 + a3; o[3] = a1 - a3;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[i] = lane_butterfly<16>(o[i], lane);
          o[i] = lane_butterfly<32>(o[i], lane);
        }
      }
#pragma unroll
      for (int hb = 1; hb < OD; hb <<= 1)
#pragma unroll
        for (int d = 0; d < OD; ++d)
          if ((d & hb) == 0) {
            const f32x4v u = acc[d][qb], v = acc[d + hb][qb];
            acc[d][qb] = u + v;
            acc[d + hb][qb] = u - v;
          }
#pragma unroll
      for (int d = 0; d < OD; ++d) acc[d][qb] *= a.wht_scale;
    }
    if (rok[qb]) {
      const int r = TG::RW * wave + 16 * qb + n16;
      const int t = r / G, h = r % G;
      float* dst = a.out + (uint64_t(pt.qrow0 + t) * a.num_q_heads + g * G + h) * HD + 4 * jg;
#pragma unroll
      for (int d = 0; d < OD; ++d) *reinterpret_cast<f32x4v*>(dst + 16 * d) = acc[d][qb];
    }
  }
}

template <int KF, int VF>
hipError_t launch_hd(int hd, const DecodeArgs& a, int G, uint32_t nwg, hipStream_t st) {
  switch (hd) {
    case 64: prefill_tile_kernel<KF, VF, 64><<<nwg, TGeo<KF, 64>::NW * kWave, 0, st>>>(a, G); break;
    case 128: prefill_tile_kernel<KF, VF, 128><<<nwg, TGeo<KF, 128>::NW * kWave, 0, st>>>(a, G); break;
    default: prefill_tile_kernel<KF, VF, 256><<<nwg, TGeo<KF, 256>::NW * kWave, 0, st>>>(a, G); break;
  }
  return hipGetLastError();
}

// Every V format and head size of one K format.
template <int KF>
hipError_t launch_kf(int vf, int hd, const DecodeArgs& a, int G, uint32_t nwg, hipStream_t st) {
  switch (vf) {
    case KVQ_BF16: return launch_hd<KF, KVQ_BF16>(hd, a, G, nwg, st);
    case KVQ_FP8_E4M3: return launch_hd<KF, KVQ_FP8_E4M3>(hd, a, G, nwg, st);
    case KVQ_TURBO2: return launch_hd<KF, KVQ_TURBO2>(hd, a, G, nwg, st);
    case KVQ_TURBO3: return launch_hd<KF, KVQ_TURBO3>(hd, a, G, nwg, st);
    case KVQ_TURBO4: return launch_hd<KF, KVQ_TURBO4>(hd, a, G, nwg, st);
    case KVQ_NVFP4: return launch_hd<KF, KVQ_NVFP4>(hd, a, G, nwg, st);
    default: return launch_hd<KF, KVQ_TURBO8>(hd, a, G, nwg, st);
  }
}

// Split partials of one output row per wave: row r of tile `tile` of
// (sequence, kv head) is query r / G, head r % G.  Log-sum-exp over the
// splits that hold keys (in split order), the fp8 V scale, the inverse
// rotation of a rotated V side (dims lane * HD/64 + e: bits below in
// registers, the rest across lanes), then the row.
template <int HD, bool VROT>
__global__ __launch_bounds__(256) void tile_merge_kernel(const DecodeArgs a, int G) {
  constexpr int NK = 8192 / HD, DPL = HD / kWave;
  const int lane = threadIdx.x & 63;
  const int rows = int(a.qt) * G;
  const uint64_t wrow = uint64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);  // over (s, tile, g, r)
  const int r = int(wrow % uint64_t(rows));
  const uint64_t stg = wrow / uint64_t(rows);
  const uint32_t g = uint32_t(stg % a.num_kv_heads), tile = uint32_t((stg / a.num_kv_heads) % a.ntiles);
  const uint32_t s = uint32_t(stg / (uint64_t(a.num_kv_heads) * a.ntiles));
  if (s >= a.num_seqs) return;
  const PrefillTile pt = prefill_tile(a, s, tile);
  const int t = r / G, h = r % G;
  if (t >= pt.nq) return;
  const int ns = (tile_chunks<NK>(pt) + int(a.split_len) / NK - 1) / (int(a.split_len) / NK);
  const uint64_t row0 = (uint64_t(stg) * a.nsplit) * uint64_t(rows) + uint64_t(r);  // split 0's row
  const uint64_t sstride = uint64_t(rows);
  float M = -INFINITY;
  for (int k = 0; k < ns; ++k) M = fmaxf(M, a.ml[(row0 + k * sstride) * 2]);
  float z = 0.0f, o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.0f;
  for (int k = 0; k < ns; ++k) {
    const uint64_t row = row0 + k * sstride;
    const float w = fast_exp2(a.ml[row * 2] - M);
    z += w * a.ml[row * 2 + 1];
    const float* src = a.part + row * HD + lane * DPL;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] += w * src[e];
  }
  const float inv = a.v_scale / z;
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] *= inv;
  if constexpr (VROT) wave_wht<DPL>(o, lane, a.wht_scale);
  float* dst = a.out + (uint64_t(pt.qrow0 + t) * a.num_q_heads + g * G + h) * HD + lane * DPL;
#pragma unroll
  for (int e = 0; e < DPL; ++e) dst[e] = o[e];
}

// The rotated K formats' instances (kvq_prefill_rot.hip).
hipError_t launch_rot(int kf, int vf, int hd, int G, const DecodeArgs& a, uint32_t nwg, hipStream_t st);

}  // namespace prefill
}  // namespace kvq
