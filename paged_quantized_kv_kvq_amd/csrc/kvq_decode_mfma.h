// Dense split pass on the matrix cores.
//
// Same contract as split_kernel ("metrale_model_layers/layers/ops/
// kv_cache_bf16k_turbov.rs", paged_decode_attn_bf16k_turbo{2,3,4}v: block
// tables, GQA, inv_sqrt_d, sliding window; "combs_models/kv.rs", attend;
// "spark_runtime/kv_cache.rs", is_wht_rotated: a rotated K side is scored
// against the rotated query): for every (sequence, kv head, split) the partial
// (max, sum, unnormalized output) of each query head of the group, in the
// layout merge_kernel reads.  The work is laid out for the memory system and
// the matrix cores:
//
//   * One workgroup per (sequence, split) and group of up to eight kv heads;
//     wave w serves kv head g0 + w and walks every 16-position chunk of the
//     split by itself.  A block row holds the kv heads of one position side
//     by side, so the waves of a workgroup read neighbouring bytes of the
//     same pages at about the same time and the workgroup streams whole
//     pages.  (One workgroup per kv head reads one head's short rows at a
//     stride; on MI355X that pattern reached about 60% of the bandwidth of
//     the page-wide one for 128-byte K and 32-byte V rows.)
//   * block_size >= 16, so that a chunk lies in one page: its page base is
//     uniform (read from LDS into scalar registers once per chunk) and every
//     lane's byte offset inside the page is fixed for the whole split.
//     Positions of a chunk outside the split lie in the same page and are
//     read too, then masked: their scores become -inf, their V words and
//     group scales zero, so that no value of an unwritten slot reaches an
//     accumulator.
//   * Q.K^T, bf16 / fp8 K: v_mfma_f32_4x4x4_16b_bf16.  Block b = lane/4 takes
//     the four positions 4(b%4).. and the quarter b/4 of head_dim; lane l
//     supplies four dims of query head l%4 (operand A) and four dims of the K
//     row of position l%16 (operand B).  bf16 x bf16 products are exact in
//     fp32, and fp8 K widens exactly to bf16, so this is the arithmetic of
//     the VALU dot products.
//   * Q.K^T, K with per-16 group scales (turbo, NVFP4):
//     v_mfma_f32_4x4x1_16b_f32 over the same blocks, one dim per instruction:
//     the query in fp32 (rotated for a turbo side) in A, the table value of
//     the lane's code (Lloyd-Max centroid or E2M1 value; adjacent codes looked
//     up as pairs) or turbo8's E4M3 value in B.  One accumulator per 16-dim
//     scale group; the lane's own position's group scales multiply the group
//     sums afterwards.
//   * Either way two lane swaps then sum the quarters so that row k of 16
//     lanes holds query head 4 hg + k for the chunk's 16 positions, and the
//     softmax runs on one value per lane.
//   * P.V on v_mfma_f32_4x4x1_16b_f32, one instruction per position and per
//     block of 64 dims.  Lane l supplies p x (group scale) of head l%4 (A)
//     and the centroid (or value) of dim l*DV + v (B); register r of its
//     accumulator is head r's output for that dim.  fp32 operands: the
//     products are exact.
//
// The VALU keeps the K widening and lookups, the V dequantization (the
// chunk's V rows are staged transposed in LDS by the wave, adjacent turbo
// codes looked up as pairs), the softmax and the masks.
#pragma once

#include "kvq_decode.h"

namespace kvq {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kUnitWaves = 8;  // most kv heads (waves) per workgroup

// Waves (kv heads) per workgroup of one instance.  Decode with a grouped-scale
// K side is bound by its arithmetic and latency chain (144 VGPRs at G = 4,
// three waves per SIMD; 194 at G = 8, two): workgroups of four kv heads let
// more of them share a CU than of eight (turbo8 / turbo8 and turbo4 / turbo8,
// G = 4: 0.51 -> 0.46 ms and 0.57 -> 0.54 ms; turbo4 / turbo3, G = 8, once
// its units are taken longest first: 0.310 -> 0.277 ms).  bf16 and fp8 K keep
// whole pages to one workgroup.
template <int KF, int G>
constexpr int mfma_waves_cap() {
  static_assert(mfma_waves_cap_of(KF, G) == (Fmt<KF>::turbo ? 4 : kUnitWaves), "host and device caps");
  return mfma_waves_cap_of(KF, G);
}

template <int KF, int VF, int HD, int G>
struct MfmaGeo {
  static constexpr int NG = (G + 3) / 4;                    // head groups of four
  static constexpr bool KT = Fmt<KF>::turbo;                // rotated K (codebook codes or E4M3 values)
  static constexpr int KQ = HD / 4;                         // K dims per lane (one quarter)
  static constexpr int KSTEPS = HD / 16;                    // 4-dim steps per quarter (bf16 / fp8 K)
  static constexpr int RBK = HD * Fmt<KF>::bits / 8;        // K code bytes per row
  static constexpr int KQB = RBK / 4;                       // K bytes per lane per chunk
  static constexpr int KGQ = KT ? KQ / 16 : 1;              // turbo K: scale groups per quarter
  static constexpr int KSG = Fmt<KF>::sgb;                  // ... bytes per group scale
  static constexpr int KSW = KT ? (KGQ * KSG + 3) / 4 : 1;  // ... words holding the quarter's scales
  static constexpr int DV = HD / 64;                        // V dims per lane
  static constexpr int RBC = HD * Fmt<VF>::bits / 8;        // V code bytes per row
  static constexpr int WR = RBC / 4;                        // ... in words
  static constexpr int NGS = Fmt<VF>::turbo ? HD / 16 : 1;  // V scale groups per row (1: no scales)
  static constexpr int SWL = HD / 16 * Fmt<VF>::sgb / 4;    // V scale words of a row
  static constexpr int NSD = (kChunk * WR + kWave - 1) / kWave;  // staged code words per lane
  static constexpr bool ok = mfma_split_ok(KF, VF, HD);
};

// One wave's staging area: the chunk's V rows transposed (word w of position
// j at [w][j], plus one zero row of slack for 3-bit fields that cross a
// word); operand A of P.V for every scale group (p of head r at position j
// times the group's E4M3 scale at [group][r][j]; without scales a single
// group of plain p); and the heads' rescale factors.
template <int KF, int VF, int HD, int G>
struct MfmaWave {
  using MG = MfmaGeo<KF, VF, HD, G>;
  __attribute__((aligned(16))) uint32_t vcode[MG::WR + 1][kChunk];
  __attribute__((aligned(16))) float pt[MG::NG][MG::NGS][4][kChunk];
  __attribute__((aligned(16))) float alpha[MG::NG][4];
};

template <int KF, int VF, int HD, int G, int NW = kUnitWaves, int NP = kMaxPages>
struct MfmaSmem {
  uint64_t kbase[NP];  // byte offset of each page of the split in the K pool
  uint64_t vbase[NP];  // ... and in the V pool
  float vcen[16];
  // turbo sides: centroids of every pair of adjacent codes (index lo | hi << bits)
  f32x2 vpair[Fmt<VF>::cb && MfmaGeo<KF, VF, HD, G>::DV >= 2 ? 1 << (2 * Fmt<VF>::bits) : 1];
  f32x2 kpair[Fmt<KF>::cb ? 1 << (2 * Fmt<KF>::bits) : 1];
  union {
    MfmaWave<KF, VF, HD, G> wv[NW];
    // turbo K, before the chunk loop: each wave's query rows, rotated in place
    float qrot[Fmt<KF>::turbo ? NW : 1][Fmt<KF>::turbo ? G : 1][Fmt<KF>::turbo ? HD : 1];
  } u;
};

// Column of position j in a wave's p x scale row of scale group grp.  The
// 4-position blocks of the row are XOR-swizzled by the group: the rows of the
// groups are 64 words apart, so unswizzled the 16-byte operand-A reads of
// lanes in different groups all start on the same bank (an 8-way conflict);
// swizzled, the blocks the lanes read spread over 16 bank offsets.
__device__ __forceinline__ int pt_col(int grp, int j) { return j ^ ((grp & 3) << 2); }

// One chunk's raw bytes in a lane's registers: its K quarter (turbo K: and
// the words that hold its quarter's scales), its share of the chunk's V code
// words, and the V scale words of position lane % 16.
template <int KF, int VF, int HD, int G>
struct MfmaChunk {
  using MG = MfmaGeo<KF, VF, HD, G>;
  uint32_t k[MG::KQB / 4];
  uint32_t ks[MG::KSW];
  uint32_t v[MG::NSD];
  uint32_t s[MG::SWL > 0 ? MG::SWL : 1];
};

// Sum of the four head_dim quarters of a 4x4 score tile.  Lane l holds
// partial scores of heads 0..3 (registers) for quarter l / 16; the result is
// the full score of head l / 16.  permlane32_swap exchanges the upper half of
// its first operand with the lower half of its second, permlane16_swap the
// odd rows of the first with the even rows of the second.
__device__ __forceinline__ float quarter_sum(const f32x4 d) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(d[0]), __float_as_uint(d[2]), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(d[1]), __float_as_uint(d[3]), false, false);
  const float y0 = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // low half: head 0, high: head 2
  const float y1 = __uint_as_float(b[0]) + __uint_as_float(b[1]);  // low half: head 1, high: head 3
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(y0), __float_as_uint(y1), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

__device__ __forceinline__ uint64_t uniform_u64(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(x >> 32));
  return uint64_t(hi) << 32 | lo;
}

// `n` bytes (a multiple of 4) from p into consecutive words, in the widest
// loads that fit.
template <int N>
__device__ __forceinline__ void load_words(const uint8_t* p, uint32_t* w) {
  int o = 0;
#pragma unroll
  for (; o + 16 <= N; o += 16) {
    const u32x4 x = load16(p + o);
    w[o / 4] = x.x; w[o / 4 + 1] = x.y; w[o / 4 + 2] = x.z; w[o / 4 + 3] = x.w;
  }
  if constexpr (N % 16 >= 8) {
    const u32x2 x = load8(p + o);
    w[o / 4] = x.x; w[o / 4 + 1] = x.y;
    o += 8;
  }
  if constexpr (N % 8 == 4) w[o / 4] = load4(p + o);
}

// Q.K^T partials of a grouped-scale K side on the matrix cores: lane l holds
// the raw bytes of its quarter (lane / 16) of position l % 16's row (k), the
// words that hold the quarter's group scales (ks, the first group at bit
// ksh) and operand A, the rotated query of head l % 4 over the quarter's dims
// (qf).  Returns the four heads' partial scores of position l % 16 over the
// quarter (the MFMA 4x4 layout).  One accumulator per scale group, the groups
// interleaved for independent chains; each group's scale multiplies its sum
// once.
//
// Codebook K sides look their code pairs up in LDS NL at a time, each batch
// requested before its products, so that NL lookups share one wait (the
// additions into each group's accumulator keep the same order for any NL).
template <int KF, int HD, int NL = MfmaGeo<KF, KVQ_BF16, HD, 4>::KGQ>
__device__ __forceinline__ f32x4 mfma_qk_turbo(const uint32_t* k, const uint32_t* ks, int ksh, const float* qf,
                                               const f32x2* kpair) {
  using MG = MfmaGeo<KF, KVQ_BF16, HD, 4>;
  f32x4 dg[MG::KGQ];
#pragma unroll
  for (int gq = 0; gq < MG::KGQ; ++gq) dg[gq] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (!Fmt<KF>::cb) {
    // turbo8: E4M3 values of the quarter
#pragma unroll
    for (int i = 0; i < 4; ++i)  // word i of each group's 16 bytes
#pragma unroll
      for (int gq = 0; gq < MG::KGQ; ++gq) {
        const uint32_t wd = k[gq * 4 + i];
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(wd), false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(wd), true);
        const int d0 = gq * 16 + 4 * i;
        dg[gq] = __builtin_amdgcn_mfma_f32_4x4x1f32(qf[d0], lo.x, dg[gq], 0, 0, 0);
        dg[gq] = __builtin_amdgcn_mfma_f32_4x4x1f32(qf[d0 + 1], lo.y, dg[gq], 0, 0, 0);
        dg[gq] = __builtin_amdgcn_mfma_f32_4x4x1f32(qf[d0 + 2], hi.x, dg[gq], 0, 0, 0);
        dg[gq] = __builtin_amdgcn_mfma_f32_4x4x1f32(qf[d0 + 3], hi.y, dg[gq], 0, 0, 0);
      }
    f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int gq = 0; gq < MG::KGQ; ++gq) {
      const int bit = ksh + 16 * gq;  // BF16 scale of group gq
      const float sc = __uint_as_float(((ks[bit / 32] >> (bit % 32)) & 0xFFFFu) << 16);
      d += sc * dg[gq];
    }
    return d;
  } else {
    // code pair p (dims 2p, 2p + 1 of the quarter) sits at bits 2 BITS p of
    // the quarter's little-endian bit stream, looked up as a pair of centroids
    constexpr int BITS = Fmt<KF>::bits, PB = 2 * BITS, PPG = 8;  // pairs per 16-dim group
    constexpr int NP = MG::KGQ * PPG;  // pairs of the quarter, visited q = pp * KGQ + gq
    constexpr int NB = NL < NP ? NL : NP;
    static_assert(NP % NB == 0, "whole batches");
#pragma unroll
    for (int q0 = 0; q0 < NP; q0 += NB) {
      f32x2 cv[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int q = q0 + b, p = (q % MG::KGQ) * PPG + q / MG::KGQ;
        const int bit = p * PB, wd = bit / 32, sh = bit % 32;
        uint32_t field;
        if constexpr (32 % PB == 0) {
          field = (k[wd] >> sh) & ((1u << PB) - 1u);
        } else {
          const uint32_t hi = wd + 1 < MG::KQB / 4 ? k[wd + 1] : 0u;
          field = uint32_t((uint64_t(hi) << 32 | k[wd]) >> sh) & ((1u << PB) - 1u);
        }
        cv[b] = kpair[field];
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int q = q0 + b, gq = q % MG::KGQ, p = gq * PPG + q / MG::KGQ;
        dg[gq] = __builtin_amdgcn_mfma_f32_4x4x1f32(qf[2 * p], cv[b].x, dg[gq], 0, 0, 0);
        dg[gq] = __builtin_amdgcn_mfma_f32_4x4x1f32(qf[2 * p + 1], cv[b].y, dg[gq], 0, 0, 0);
      }
    }
    // the groups' E4M3 scales (of this lane's position) on the group sums
    f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int gq = 0; gq < MG::KGQ; ++gq) {
      const int bit = ksh + 8 * gq;
      const float sc = __builtin_amdgcn_cvt_f32_fp8(int(ks[bit / 32] >> (bit % 32)), 0);
      d += sc * dg[gq];
    }
    return d;
  }
}

// One query per sequence; the rows of a wave are the G query heads of its
// kv head.
template <int KF, int VF, int HD, int G>
__global__ __launch_bounds__(kUnitWaves * kWave) void split_mfma_kernel(const DecodeArgs a) {
  constexpr int R = G;  // rows: the query heads
  using MG = MfmaGeo<KF, VF, HD, R>;
  constexpr int NG = MG::NG, DV = MG::DV;
  __shared__ MfmaSmem<KF, VF, HD, R, mfma_waves_cap<KF, G>(), dense_max_pages(KF)> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = __builtin_amdgcn_readfirstlane(int(blockDim.x) >> 6);
  // workgroup -> (unit, group of kv heads).  Workgroups are dealt to the 8
  // XCDs in turn; when a unit spans several workgroups (hblocks > 1) they are
  // the consecutive workgroups k, k + 1, ... of one XCD (k = blockIdx / 8), so
  // the 128-byte lines that hold several heads' scale rows of a position are
  // fetched into one L2.  The grid is padded to whole rounds of 8 units.
  const uint32_t hblocks = a.num_kv_heads / uint32_t(nw);
  uint32_t unit = blockIdx.x, hb = 0;
  if (hblocks > 1) {
    const uint32_t k = blockIdx.x / 8u;
    unit = (k / hblocks) * 8u + blockIdx.x % 8u;
    hb = k % hblocks;
  }
  const uint32_t g = hb * uint32_t(nw) + uint32_t(w);
  const uint32_t nkv = a.num_kv_heads;
  if (unit >= a.num_seqs * a.nsplit) return;
  if (a.order) unit = a.order[unit];
  const uint32_t s = unit % a.num_seqs, split = unit / a.num_seqs;
  const SeqSpan sp = split_span(a, s, split);
  if (sp.pb >= sp.L) return;  // uniform over the workgroup
  const uint16_t* qg = a.q + uint64_t(row_query(a, s)) * a.q_stride + uint64_t(g) * G * HD;  // the group's rows

  // bf16 / fp8 K, query operand A: head 4 hg + lane % 4, dims (lane / 16) * KQ + 4 k .. + 4
  i16x4 qa[MG::KT ? 1 : NG][MG::KT ? 1 : MG::KSTEPS];
  if constexpr (!MG::KT) {
#pragma unroll
    for (int hg = 0; hg < NG; ++hg) {
      const int h = 4 * hg + (lane & 3);
#pragma unroll
      for (int k = 0; k < MG::KSTEPS; ++k) {
        const int d = (lane >> 4) * MG::KQ + 4 * k;
        if (h < G) {
          const u32x2 x = *reinterpret_cast<const u32x2*>(qg + h * HD + d);
          qa[hg][k] = __builtin_bit_cast(i16x4, x);
        } else {
          qa[hg][k] = i16x4{0, 0, 0, 0};
        }
      }
    }
  }
  // page offsets of the split and the codebooks, shared by the waves
  const int first = sp.pb >> a.log2_bs;
  {
    const int n = ((sp.pe - 1) >> a.log2_bs) - first + 1;
    const int32_t* bt = a.block_tables + uint64_t(row_table(a, s)) * a.max_blocks + first;
    for (int i = tid; i < n; i += int(blockDim.x)) {
      const uint64_t page = uint64_t(uint32_t(bt[i]));
      sm.kbase[i] = page * a.k_stride;
      sm.vbase[i] = page * a.v_stride;
    }
    if constexpr (Fmt<VF>::cb) {
      constexpr int BITS = Fmt<VF>::bits;
      if (tid < 16) sm.vcen[tid] = tid < (1 << BITS) ? a.cb.centroid[VF - 2][tid] : 0.0f;
      if constexpr (DV >= 2) {
        for (int e = tid; e < (1 << (2 * BITS)); e += int(blockDim.x)) {
          sm.vpair[e].x = a.cb.centroid[VF - 2][e & ((1 << BITS) - 1)];
          sm.vpair[e].y = a.cb.centroid[VF - 2][e >> BITS];
        }
      }
    }
    if constexpr (Fmt<KF>::cb) {
      constexpr int BITS = Fmt<KF>::bits;
      for (int e = tid; e < (1 << (2 * BITS)); e += int(blockDim.x)) {
        sm.kpair[e].x = a.cb.centroid[KF - 2][e & ((1 << BITS) - 1)];
        sm.kpair[e].y = a.cb.centroid[KF - 2][e >> BITS];
      }
    }
  }
  // turbo K, query operand A: the rotated query (unnormalized: 1/sqrt(d)
  // goes into the score scale), head 4 hg + lane % 4, dim (lane / 16) * KQ + k
  float qf[MG::KT ? NG : 1][MG::KT ? MG::KQ : 1];
  if constexpr (MG::KT) {
    auto& qr = sm.u.qrot[w];
    for (int i = lane; i < G * HD; i += kWave) qr[i / HD][i % HD] = bf16_bits_to_float(qg[i]);
    wave_lds_sync();
    if constexpr (Fmt<KF>::rot) {  // NVFP4 K: the query as it is
      for (int h2 = 1; h2 < HD; h2 <<= 1) {
        for (int i = lane; i < R * HD / 2; i += kWave) {
          const int hh = i / (HD / 2), k = i % (HD / 2);
          const int lo = (k / h2) * 2 * h2 + (k % h2);
          const float x = qr[hh][lo], y = qr[hh][lo + h2];
          qr[hh][lo] = x + y;
          qr[hh][lo + h2] = x - y;
        }
        wave_lds_sync();
      }
    }
#pragma unroll
    for (int hg = 0; hg < NG; ++hg) {
      const int h = 4 * hg + (lane & 3);
#pragma unroll
      for (int k = 0; k < MG::KQ; ++k) qf[hg][k] = h < R ? qr[h][(lane >> 4) * MG::KQ + k] : 0.0f;
    }
  }
  // every load so far completes before the chunk loop, whose wait counts
  // then only ever cover chunk loads; the staging areas overlay the rotated
  // queries, so the slack rows are cleared after the barrier
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  auto& wv = sm.u.wv[w];
  if (lane < kChunk) wv.vcode[MG::WR][lane] = 0u;  // the slack row stays zero

  // the lane's byte offsets inside a chunk's page, fixed for the split:
  // K quarter lane/16 of position lane%16 (turbo K: and the word of that
  // row's scale bytes that holds the quarter's groups); code word i%WR of
  // row i/WR for i = lane + 64 n; the V scale words of row lane%16
  const uint32_t bmask = (1u << a.log2_bs) - 1u;
  const uint32_t koff = ((uint32_t(lane) & 15u) * nkv + g) * MG::RBK + (uint32_t(lane) >> 4) * MG::KQB;
  // (the quarter's scales start at byte (lane/16) * KGQ * KSG of the row's scales)
  const uint32_t ksb = (uint32_t(lane) >> 4) * MG::KGQ * MG::KSG;
  const uint32_t ksoff = a.k_data + ((uint32_t(lane) & 15u) * nkv + g) * (HD / 16 * MG::KSG) + (ksb & ~3u);
  const int ksh = int(ksb & 3u) * 8;  // bit offset of the first group's scale in ks[0]
  uint32_t voff[MG::NSD];
  int vrow[MG::NSD];
#pragma unroll
  for (int n = 0; n < MG::NSD; ++n) {
    const int i = lane + n * kWave;
    vrow[n] = min(i / MG::WR, kChunk - 1);
    voff[n] = (uint32_t(vrow[n]) * nkv + g) * MG::RBC + uint32_t(i % MG::WR) * 4u;
  }
  const uint32_t soff = a.v_data + ((uint32_t(lane) & 15u) * nkv + g) * (HD / 16 * Fmt<VF>::sgb);
  const int cs = sp.pb & ~(kChunk - 1);
  const int clast = (sp.pe - 1) & ~(kChunk - 1);
  auto load = [&](int c, MfmaChunk<KF, VF, HD, R>& ck) {
    const int cl = min(c, clast);  // past the end: reread the last chunk (all masked)
    const int pg = (cl >> a.log2_bs) - first;
    const uint32_t within = uint32_t(cl) & bmask;
    const uint64_t kpage = uniform_u64(sm.kbase[pg]);
    const uint64_t vb = uniform_u64(sm.vbase[pg]);
    load_words<MG::KQB>(a.k_cache + kpage + uint64_t(within) * nkv * MG::RBK + koff, ck.k);
    if constexpr (MG::KT) {
#pragma unroll
      for (int i = 0; i < MG::KSW; ++i)
        ck.ks[i] = load4(a.k_cache + kpage + uint64_t(within) * nkv * (HD / 16 * MG::KSG) + ksoff + 4 * i);
    } else {
      ck.ks[0] = 0u;
    }
    const uint8_t* vp = a.v_cache + vb + uint64_t(within) * nkv * MG::RBC;
#pragma unroll
    for (int n = 0; n < MG::NSD; ++n) ck.v[n] = load4(vp + voff[n]);
    if constexpr (MG::SWL > 0)
      load_words<4 * MG::SWL>(a.v_cache + vb + uint64_t(within) * nkv * (HD / 16 * Fmt<VF>::sgb) + soff, ck.s);
    else ck.s[0] = 0u;
  };

  const float qscale = a.qk_scale * (Fmt<KF>::rot ? a.wht_scale : 1.0f);
  // running state.  Lane l follows head 4 hg + l / 16 (its row of 16 lanes):
  // m is that head's running max (uniform in the row; finite at the start so
  // that a chunk with every position masked rescales by exactly 1), lsum the
  // lane's share of its sum (position l % 16 of every chunk).  Accumulators
  // are in the MFMA layout: register r holds head 4 hg + r.
  constexpr float kNoMax = -3.0e38f;
  float m[NG], lsum[NG];
  // two chains (even and odd positions), or one where four or more row
  // groups already give independent chains
  constexpr int NCH = NG >= 4 ? 1 : 2;
  f32x4 acc[NG][NCH][DV];
#pragma unroll
  for (int hg = 0; hg < NG; ++hg) {
    m[hg] = kNoMax;
    lsum[hg] = 0.0f;
#pragma unroll
    for (int v = 0; v < DV; ++v) {
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) acc[hg][ch][v] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }
  auto& vcode = wv.vcode;
  auto& pt = wv.pt;

  // the lane's Q.K^T partial over its quarter for heads 4 hg + r (registers)
  // at position c + lane % 16
  auto qk = [&](const MfmaChunk<KF, VF, HD, R>& ck, int hg) -> f32x4 {
    if constexpr (!MG::KT) {
      i16x4 kb[MG::KSTEPS];
#pragma unroll
      for (int k = 0; k < MG::KSTEPS; ++k) {
        if constexpr (KF == KVQ_BF16) {
          const u32x2 x = {ck.k[2 * k], ck.k[2 * k + 1]};
          kb[k] = __builtin_bit_cast(i16x4, x);
        } else {
          const u32x2 x = {fp8x2_to_bf16x2<false>(ck.k[k]), fp8x2_to_bf16x2<true>(ck.k[k])};
          kb[k] = __builtin_bit_cast(i16x4, x);
        }
      }
      f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < MG::KSTEPS; ++k) d = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(qa[hg][k], kb[k], d, 0, 0, 0);
      return d;
    } else {
      return mfma_qk_turbo<KF, HD>(ck.k, ck.ks, ksh, qf[hg], sm.kpair);
    }
  };

  auto consume = [&](int c, const MfmaChunk<KF, VF, HD, R>& ck) {
    // 1. stage the chunk's V codes in LDS (bf16 / fp8 / turbo8 V: rows
    //    outside the split as zeros, whatever bytes they hold)
#pragma unroll
    for (int n = 0; n < MG::NSD; ++n) {
      const int i = lane + n * kWave;
      if (i < kChunk * MG::WR) {
        uint32_t word = ck.v[n];
        if constexpr (!Fmt<VF>::cb) {  // values (not codes) may be NaN bytes
          const int j = c + vrow[n];
          word = (j >= sp.pb && j < sp.pe) ? word : 0u;
        }
        vcode[i % MG::WR][vrow[n]] = word;
      }
    }
    // 2. scores: position c + lane % 16, heads 4 hg + r
    const int j = c + (lane & 15);
    const bool in_split = j >= sp.pb && j < sp.pe;
    bool grew = false;
#pragma unroll
    for (int hg = 0; hg < NG; ++hg) {
      const bool ok = in_split;
      const f32x4 d = qk(ck, hg);
      // 3. the row's head: full score (masked positions: -inf, whatever
      //    bytes they hold), then its online softmax over the chunk.  The
      //    lane swaps exchange values between the rows of one position, which
      //    share the mask: a swap never reads an inactive lane.
      const float sc = ok ? quarter_sum(d) * qscale : -INFINITY;
      const float mn = fmaxf(m[hg], group_max<16>(sc));
      const float al = fast_exp2(m[hg] - mn);
      grew |= mn > m[hg];
      m[hg] = mn;
      const float p = fast_exp2(sc - mn);  // 0 where masked
      lsum[hg] = fmaf(lsum[hg], al, p);
      if constexpr (MG::SWL > 0 && Fmt<VF>::cb) {
        // operand A per scale group: p x the group's scale (outside the
        // split the scale words are zeroed: p = 0 times a garbage NaN
        // scale would not be 0)
#pragma unroll
        for (int sw = 0; sw < MG::SWL; ++sw) {
          const int sword = ok ? int(ck.s[sw]) : 0;
          const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(sword, false);
          const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(sword, true);
          pt[hg][4 * sw][lane >> 4][pt_col(4 * sw, lane & 15)] = p * lo.x;
          pt[hg][4 * sw + 1][lane >> 4][pt_col(4 * sw + 1, lane & 15)] = p * lo.y;
          pt[hg][4 * sw + 2][lane >> 4][pt_col(4 * sw + 2, lane & 15)] = p * hi.x;
          pt[hg][4 * sw + 3][lane >> 4][pt_col(4 * sw + 3, lane & 15)] = p * hi.y;
        }
      } else if constexpr (MG::SWL > 0) {
        // turbo8: two BF16 scales per word
#pragma unroll
        for (int sw = 0; sw < MG::SWL; ++sw) {
          const uint32_t sword = ok ? ck.s[sw] : 0u;
          pt[hg][2 * sw][lane >> 4][pt_col(2 * sw, lane & 15)] = p * __uint_as_float(sword << 16);
          pt[hg][2 * sw + 1][lane >> 4][pt_col(2 * sw + 1, lane & 15)] = p * __uint_as_float(sword & 0xFFFF0000u);
        }
      } else {
        pt[hg][0][lane >> 4][pt_col(0, lane & 15)] = p;
      }
      wv.alpha[hg][lane >> 4] = al;
    }
    wave_lds_sync();
    if (__builtin_amdgcn_ballot_w64(grew)) {  // rare after the first chunks
#pragma unroll
      for (int hg = 0; hg < NG; ++hg) {
        const f32x4 al = *reinterpret_cast<const f32x4*>(&wv.alpha[hg][0]);
#pragma unroll
        for (int v = 0; v < DV; ++v) {
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch) acc[hg][ch][v] *= al;
        }
      }
    }
    // 4. P.V: the lane's operands for 8 positions at a time come from LDS in
    //    16-byte reads; even and odd positions feed two accumulator chains
#pragma unroll
    for (int h8 = 0; h8 < kChunk; h8 += 8) {
      // the lane's scale group (a block of four lanes covers 4 DV dims, all in one group)
      const int grp = MG::SWL > 0 ? (lane * DV) / 16 : 0;
      float pa[NG][8];
#pragma unroll
      for (int hg = 0; hg < NG; ++hg) {
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(&pt[hg][grp][lane & 3][pt_col(grp, h8)]);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(&pt[hg][grp][lane & 3][pt_col(grp, h8 + 4)]);
        pa[hg][0] = x0.x; pa[hg][1] = x0.y; pa[hg][2] = x0.z; pa[hg][3] = x0.w;
        pa[hg][4] = x1.x; pa[hg][5] = x1.y; pa[hg][6] = x1.z; pa[hg][7] = x1.w;
      }
      float b[8][DV];
      if constexpr (Fmt<VF>::cb) {
        constexpr int BITS = Fmt<VF>::bits;
        const int bit = lane * DV * BITS;
        const int wd = bit / 32, sh = bit % 32;
        const u32x4 c00 = *reinterpret_cast<const u32x4*>(&vcode[wd][h8]);
        const u32x4 c01 = *reinterpret_cast<const u32x4*>(&vcode[wd][h8 + 4]);
        uint32_t cw[8] = {c00.x, c00.y, c00.z, c00.w, c01.x, c01.y, c01.z, c01.w};
        if constexpr (32 % (DV * BITS) != 0) {  // fields may cross into the next word
          const u32x4 c10 = *reinterpret_cast<const u32x4*>(&vcode[wd + 1][h8]);
          const u32x4 c11 = *reinterpret_cast<const u32x4*>(&vcode[wd + 1][h8 + 4]);
          const uint32_t hi[8] = {c10.x, c10.y, c10.z, c10.w, c11.x, c11.y, c11.z, c11.w};
#pragma unroll
          for (int q = 0; q < 8; ++q) cw[q] = uint32_t((uint64_t(hi[q]) << 32 | cw[q]) >> sh);
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) cw[q] >>= sh;
        }
        // the centroids go into operand B
        if constexpr (DV >= 2) {
#pragma unroll
          for (int q = 0; q < 8; ++q)
#pragma unroll
            for (int v2 = 0; v2 < DV / 2; ++v2) {
              const f32x2 pr = sm.vpair[(cw[q] >> (2 * BITS * v2)) & ((1u << (2 * BITS)) - 1u)];
              b[q][2 * v2] = pr.x;
              b[q][2 * v2 + 1] = pr.y;
            }
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) b[q][0] = sm.vcen[cw[q] & ((1u << BITS) - 1u)];
        }
      } else {
        constexpr int EB = Fmt<VF>::bits / 8;
        const int byte = lane * DV * EB;
        const u32x4 c00 = *reinterpret_cast<const u32x4*>(&vcode[byte / 4][h8]);
        const u32x4 c01 = *reinterpret_cast<const u32x4*>(&vcode[byte / 4][h8 + 4]);
        const uint32_t cw0[8] = {c00.x, c00.y, c00.z, c00.w, c01.x, c01.y, c01.z, c01.w};
        uint32_t cw1[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if constexpr (DV * EB > 4) {
          const u32x4 c10 = *reinterpret_cast<const u32x4*>(&vcode[byte / 4 + 1][h8]);
          const u32x4 c11 = *reinterpret_cast<const u32x4*>(&vcode[byte / 4 + 1][h8 + 4]);
          const uint32_t t1[8] = {c10.x, c10.y, c10.z, c10.w, c11.x, c11.y, c11.z, c11.w};
#pragma unroll
          for (int q = 0; q < 8; ++q) cw1[q] = t1[q];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint64_t all = (uint64_t(cw1[q]) << 32 | cw0[q]) >> ((byte % 4) * 8);
#pragma unroll
          for (int v = 0; v < DV; ++v) {
            if constexpr (Fmt<VF>::bits == 8) {  // fp8, turbo8: E4M3 values
              const f32x2 x = __builtin_amdgcn_cvt_pk_f32_fp8(int(uint32_t(all >> (8 * (v & ~1)))), false);
              b[q][v] = (v & 1) ? x.y : x.x;
            } else {
              b[q][v] = __uint_as_float(uint32_t(all >> (16 * v)) << 16);
            }
          }
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int hg = 0; hg < NG; ++hg)
#pragma unroll
          for (int v = 0; v < DV; ++v)
            acc[hg][q % NCH][v] = __builtin_amdgcn_mfma_f32_4x4x1f32(pa[hg][q], b[q][v], acc[hg][q % NCH][v], 0, 0, 0);
    }
    wave_lds_sync();
  };

  // chunk loop: chunk n sits in buffer n % NB and is loaded NB - 1 chunks
  // ahead of its use; every load is issued inside the loop, whose rounds of
  // NB chunks have one exit, at the bottom (the first NB - 1 uses are of
  // zeroed buffers before the split, all masked)
  constexpr int NB = KVQ_DENSE_BUFS;
  MfmaChunk<KF, VF, HD, R> cb[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
#pragma unroll
    for (int k = 0; k < MG::KQB / 4; ++k) cb[i].k[k] = 0u;
#pragma unroll
    for (int k = 0; k < MG::KSW; ++k) cb[i].ks[k] = 0u;
#pragma unroll
    for (int k = 0; k < MG::NSD; ++k) cb[i].v[k] = 0u;
#pragma unroll
    for (int k = 0; k < (MG::SWL > 0 ? MG::SWL : 1); ++k) cb[i].s[k] = 0u;
  }
  {
    const int nch = (clast - cs) / kChunk + 1;
    const int rounds = (nch + 2 * NB - 2) / NB;  // covers the chunks and the NB - 1 leading uses
    int c = cs;  // next chunk to load
    for (int it = 0; it < rounds; ++it) {
      // every other round the waves meet (no memory fence: loads stay in
      // flight), so that none runs more than a few chunks ahead of the
      // others.  Their heads' V rows (32 bytes) and scale rows (8 bytes)
      // share 128-byte lines; with the waves this close, a line is still in
      // L2 when the last of them reads it (apart, the kernel fetched 1.11 to
      // 1.17 times its bytes from beyond L2).
      if ((it & 1) == 0) __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        load(c, cb[(i + NB - 1) % NB]);
        consume(c - (NB - 1) * kChunk, cb[i]);
        c += kChunk;
      }
    }
  }

  // the wave's partials for its kv head: sums over the row's 16 lanes, one
  // output dim pair per lane and head
  const uint64_t base = (uint64_t(s) * nkv + g) * a.nsplit + split;
#pragma unroll
  for (int hg = 0; hg < NG; ++hg) {
    const float z = group_sum<16>(lsum[hg]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * hg + r;
      if (h < R) {
        float* dst = a.part + (base * R + h) * HD + lane * DV;
#pragma unroll
        for (int v = 0; v < DV; ++v) {
          float o = acc[hg][0][v][r];
#pragma unroll
          for (int ch = 1; ch < NCH; ++ch) o += acc[hg][ch][v][r];
          dst[v] = o;
        }
      }
    }
    const int h = 4 * hg + (lane >> 4);
    if ((lane & 15) == 0 && h < R) {  // a split that saw no position reports -inf
      a.ml[(base * R + h) * 2] = z > 0.0f ? m[hg] : -INFINITY;
      a.ml[(base * R + h) * 2 + 1] = z;
    }
  }
}

// Workgroups of split_mfma_kernel for `units` units of `hblocks` workgroups
// each (whole rounds of 8 units when a unit spans several workgroups; see the
// mapping in the kernel).
inline uint64_t mfma_grid(uint64_t units, uint32_t hblocks) {
  return hblocks > 1 ? (units + 7) / 8 * 8 * hblocks : units;
}


}  // namespace kvq
