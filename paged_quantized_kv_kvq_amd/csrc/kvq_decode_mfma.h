// Dense split pass on the matrix cores, for bf16 and fp8 K sides.
//
// Same contract as split_kernel ("metrale_model_layers/layers/ops/
// kv_cache_bf16k_turbov.rs", paged_decode_attn_bf16k_turbo{2,3,4}v: block
// tables, GQA, inv_sqrt_d, sliding window; "combs_models/kv.rs", attend): one
// workgroup per (sequence, kv head, split), four waves on interleaved
// 16-position chunks, online softmax, and the same per-split partials for
// merge_kernel.  What moves to the matrix cores is the arithmetic:
//
//   * Q.K^T on v_mfma_f32_4x4x4_16b_bf16.  Block b = lane/4 takes the four
//     positions 4(b%4).. and the quarter b/4 of head_dim; lane l supplies
//     four dims of query head l%4 (operand A) and four dims of the K row of
//     position l%16 (operand B).  Over the quarter's head_dim/16 steps each
//     block accumulates partial scores; two cross-lane sums over the quarters
//     leave every lane with the scores of position l%16 for its head group.
//     bf16 x bf16 products are exact in fp32, and fp8 K widens exactly to
//     bf16, so this is the same arithmetic as the VALU dot products.
//   * P.V on v_mfma_f32_4x4x1_16b_f32, one instruction per position and per
//     block of 64 dims.  Lane l supplies p of head l%4 (A) and the dequantized
//     V value of dim l*DV + v (B); register r of its accumulator is head r's
//     output for that dim.  All operands are fp32: the products are exact.
//
// The VALU keeps the K widening, the V dequantization (V rows of a chunk are
// staged in LDS by all lanes, their E4M3 group scales decoded once), the
// softmax and the index arithmetic.
#pragma once

#include "kvq_decode.h"

namespace kvq {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <int KF, int VF, int HD, int G>
struct MfmaGeo {
  static constexpr int NG = (G + 3) / 4;                    // head groups of four
  static constexpr int KQ = HD / 4;                         // K dims per lane (one quarter)
  static constexpr int KSTEPS = HD / 16;                    // 4-dim steps per quarter
  static constexpr int KQB = KQ * Fmt<KF>::bits / 8;        // K bytes per lane per chunk
  static constexpr int DV = HD / 64;                        // V dims per lane
  static constexpr int RBC = HD * Fmt<VF>::bits / 8;        // V code bytes per row
  static constexpr int WR = RBC / 4;                        // ... in words
  static constexpr int SW = Fmt<VF>::turbo ? HD / 64 : 0;   // V scale words per row (4 bytes each)
  static constexpr int NSD = (kChunk * WR + kWave - 1) / kWave;  // staged code words per lane
  static constexpr bool ok = (KF == KVQ_BF16 || KF == KVQ_FP8_E4M3) && KQB <= 64 && RBC <= 128 &&
                             (KQB % 16 == 0);
};

template <int KF, int VF, int HD, int G>
struct MfmaSmem {
  using MG = MfmaGeo<KF, VF, HD, G>;
  PrologueSmem<KF, HD, G> pro;
  // the chunk's V rows, transposed (word w of position j at [w][j]; one
  // zero row of slack for 3-bit fields that cross a word), and their group
  // scales, decoded, transposed the same way
  __attribute__((aligned(16))) uint32_t vcode[kWaves][MG::WR + 1][kChunk];
  __attribute__((aligned(16))) float vscale[kWaves][Fmt<VF>::turbo ? HD / 16 : 1][kChunk];
  __attribute__((aligned(16))) float pt[kWaves][MG::NG][4][kChunk];  // p, transposed for operand A
  __attribute__((aligned(16))) float alpha[kWaves][MG::NG][4];        // rescale factors of a chunk
  // turbo V: centroids of every pair of adjacent codes (index lo | hi << bits)
  f32x2 vpair[Fmt<VF>::turbo && MG::DV >= 2 ? 1 << (2 * Fmt<VF>::bits) : 1];
  float red[kWaves][G][HD + 2];
};

// One chunk's raw data in a lane's registers: its K quarter, and its share of
// the chunk's V rows (code words and scale words).
template <int KF, int VF, int HD, int G>
struct MfmaChunk {
  using MG = MfmaGeo<KF, VF, HD, G>;
  uint32_t k[MG::KQB / 4];
  uint32_t v[MG::NSD];
  uint32_t s;
};

template <int KF, int VF, int HD, int G>
__device__ __forceinline__ void mfma_load(const DecodeArgs& a, const PrologueSmem<KF, HD, G>& sm, int first, int c,
                                          int pb, int pe, uint32_t g, int lane, MfmaChunk<KF, VF, HD, G>& ck) {
  using MG = MfmaGeo<KF, VF, HD, G>;
  const uint32_t bmask = (1u << a.log2_bs) - 1u;
  // K: position c + lane%16, quarter lane/16 (clamped into the split; masked later)
  {
    const int j = min(max(c + (lane & 15), pb), pe - 1);
    const int bi = (j >> a.log2_bs) - first;
    const uint32_t row = (uint32_t(j) & bmask) * a.num_kv_heads + g;
    const uint8_t* p = a.k_cache + sm.kbase[bi] + uint64_t(row) * (HD * Fmt<KF>::bits / 8) + (lane >> 4) * MG::KQB;
#pragma unroll
    for (int i = 0; i < MG::KQB / 16; ++i) {
      const u32x4 x = load16(p + 16 * i);
      ck.k[4 * i] = x.x; ck.k[4 * i + 1] = x.y; ck.k[4 * i + 2] = x.z; ck.k[4 * i + 3] = x.w;
    }
  }
  // V codes: word i of the chunk's rows is word i % WR of row i / WR
#pragma unroll
  for (int n = 0; n < MG::NSD; ++n) {
    const int i = lane + n * kWave;
    const int rr = min(i / MG::WR, kChunk - 1);
    const int j = min(max(c + rr, pb), pe - 1);
    const int bi = (j >> a.log2_bs) - first;
    const uint32_t row = (uint32_t(j) & bmask) * a.num_kv_heads + g;
    const uint8_t* p = a.v_cache + sm.vbase[bi] + uint64_t(row) * MG::RBC + (i % MG::WR) * 4;
    ck.v[n] = *reinterpret_cast<const uint32_t*>(p);
  }
  // V scales: word lane % SW of row lane / SW (lanes < 16 * SW)
  if constexpr (MG::SW > 0) {
    const int rr = min(lane / MG::SW, kChunk - 1);
    const int j = min(max(c + rr, pb), pe - 1);
    const int bi = (j >> a.log2_bs) - first;
    const uint32_t row = (uint32_t(j) & bmask) * a.num_kv_heads + g;
    const uint8_t* p = a.v_cache + sm.vbase[bi] + a.v_data + uint64_t(row) * (HD / 16) + (lane % MG::SW) * 4;
    ck.s = *reinterpret_cast<const uint32_t*>(p);
  } else {
    ck.s = 0;
  }
}

// Sum of the four head_dim quarters of a 4x4x4 score tile.  Lane l holds
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

template <int KF, int VF, int HD, int G>
__global__ __launch_bounds__(kWaves * kWave) void split_mfma_kernel(const DecodeArgs a) {
  using MG = MfmaGeo<KF, VF, HD, G>;
  constexpr int NG = MG::NG, DV = MG::DV;
  __shared__ MfmaSmem<KF, VF, HD, G> sm;
  const Tile tl = unit_tile<KVQ_TILE_DENSE>(a, a.nsplit);
  if (!tl.valid) return;
  const SeqSpan sp = split_span(a, tl.s, tl.split);
  if (sp.pb >= sp.L) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // query operand A: head 4 * hg + lane % 4, dims (lane / 16) * KQ + 4 s .. + 4
  i16x4 qa[NG][MG::KSTEPS];
  {
    const uint16_t* qg = a.q + uint64_t(tl.s) * a.q_stride + uint64_t(tl.g) * G * HD;
#pragma unroll
    for (int hg = 0; hg < NG; ++hg) {
      const int h = 4 * hg + (lane & 3);
#pragma unroll
      for (int s = 0; s < MG::KSTEPS; ++s) {
        const int d = (lane >> 4) * MG::KQ + 4 * s;
        if (h < G) {
          const u32x2 x = *reinterpret_cast<const u32x2*>(qg + h * HD + d);
          qa[hg][s] = __builtin_bit_cast(i16x4, x);
        } else {
          qa[hg][s] = i16x4{0, 0, 0, 0};
        }
      }
    }
  }
  // page offsets and codebook (the QReg argument of the shared prologue is unused here)
  {
    QReg<KF, 16, G> unused;
    prologue<KF, VF, HD, G, 16>(a, sm.pro, tl.s, tl.g, sp.pb, sp.pe, 0, unused);
  }
  if constexpr (Fmt<VF>::turbo && DV >= 2) {
    constexpr int BITS = Fmt<VF>::bits;
    for (int e = tid; e < (1 << (2 * BITS)); e += kWaves * kWave) {
      sm.vpair[e].x = a.cb.centroid[VF - 2][e & ((1 << BITS) - 1)];
      sm.vpair[e].y = a.cb.centroid[VF - 2][e >> BITS];
    }
    __syncthreads();
  }
  const int first = sp.pb >> a.log2_bs;
  const float qscale = a.qk_scale;
  // running state.  Lane l follows head 4 hg + l / 16 (its row of 16 lanes):
  // m is that head's running max (uniform in the row; finite at the start so
  // that a chunk with every position masked rescales by exactly 1), lsum the
  // lane's share of its sum (position l % 16 of every chunk).  Accumulators
  // are in the MFMA layout: register r holds head 4 hg + r.
  constexpr float kNoMax = -3.0e38f;
  float m[NG], lsum[NG];
  f32x4 acc[NG][2][DV];  // two chains: even and odd positions
#pragma unroll
  for (int hg = 0; hg < NG; ++hg) {
    m[hg] = kNoMax;
    lsum[hg] = 0.0f;
#pragma unroll
    for (int v = 0; v < DV; ++v) {
      acc[hg][0][v] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      acc[hg][1][v] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }
  auto& vcode = sm.vcode[w];
  auto& vscale = sm.vscale[w];
  auto& pt = sm.pt[w];

  if (lane < kChunk) vcode[MG::WR][lane] = 0u;  // the slack row stays zero

  auto consume = [&](int c, const MfmaChunk<KF, VF, HD, G>& ck) {
    // 1. stage the chunk's V rows (codes as loaded, scales decoded) in LDS
#pragma unroll
    for (int n = 0; n < MG::NSD; ++n) {
      const int i = lane + n * kWave;
      if (i < kChunk * MG::WR) vcode[i % MG::WR][i / MG::WR] = ck.v[n];
    }
    if constexpr (MG::SW > 0) {
      if (lane < kChunk * MG::SW) {
        const int rr = lane / MG::SW, q4 = (lane % MG::SW) * 4;
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(ck.s), false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(ck.s), true);
        vscale[q4][rr] = lo.x;
        vscale[q4 + 1][rr] = lo.y;
        vscale[q4 + 2][rr] = hi.x;
        vscale[q4 + 3][rr] = hi.y;
      }
    }
    // 2. scores: position c + lane % 16, heads 4 hg + r
    i16x4 kb[MG::KSTEPS];
#pragma unroll
    for (int s = 0; s < MG::KSTEPS; ++s) {
      if constexpr (KF == KVQ_BF16) {
        const u32x2 x = {ck.k[2 * s], ck.k[2 * s + 1]};
        kb[s] = __builtin_bit_cast(i16x4, x);
      } else {
        const u32x2 x = {fp8x2_to_bf16x2<false>(ck.k[s]), fp8x2_to_bf16x2<true>(ck.k[s])};
        kb[s] = __builtin_bit_cast(i16x4, x);
      }
    }
    const int j = c + (lane & 15);
    const bool ok = j >= sp.pb && j < sp.pe;
    bool grew = false;
#pragma unroll
    for (int hg = 0; hg < NG; ++hg) {
      f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < MG::KSTEPS; ++s) d = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(qa[hg][s], kb[s], d, 0, 0, 0);
      // 3. sum the four quarters so that row k of 16 lanes ends with head
      //    4 hg + k: the half-wave swap pairs rows (0,1) with (2,3) and keeps
      //    heads {0,1} in the low half, the row swap then pairs rows 0-1, 2-3
      const float s = ok ? quarter_sum(d) * qscale : -INFINITY;
      // 4. online softmax of the row's head over the chunk's 16 positions
      const float mn = fmaxf(m[hg], group_max<16>(s));
      const float al = fast_exp2(m[hg] - mn);
      grew |= mn > m[hg];
      m[hg] = mn;
      const float p = fast_exp2(s - mn);  // 0 where masked
      lsum[hg] = fmaf(lsum[hg], al, p);
      pt[hg][lane >> 4][lane & 15] = p;
      sm.alpha[w][hg][lane >> 4] = al;
    }
    wave_lds_sync();
    if (__builtin_amdgcn_ballot_w64(grew)) {  // rare after the first chunks
#pragma unroll
      for (int hg = 0; hg < NG; ++hg) {
        const f32x4 al = *reinterpret_cast<const f32x4*>(&sm.alpha[w][hg][0]);
#pragma unroll
        for (int v = 0; v < DV; ++v) {
          acc[hg][0][v] *= al;
          acc[hg][1][v] *= al;
        }
      }
    }
    // 5. P.V: the lane's operands for 8 positions at a time come from LDS in
    //    16-byte reads; even and odd positions feed two accumulator chains
#pragma unroll
    for (int h8 = 0; h8 < kChunk; h8 += 8) {
      float pa[NG][8];
#pragma unroll
      for (int hg = 0; hg < NG; ++hg) {
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(&pt[hg][lane & 3][h8]);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(&pt[hg][lane & 3][h8 + 4]);
        pa[hg][0] = x0.x; pa[hg][1] = x0.y; pa[hg][2] = x0.z; pa[hg][3] = x0.w;
        pa[hg][4] = x1.x; pa[hg][5] = x1.y; pa[hg][6] = x1.z; pa[hg][7] = x1.w;
      }
      float b[8][DV];
      if constexpr (Fmt<VF>::turbo) {
        constexpr int BITS = Fmt<VF>::bits;
        const int bit = lane * DV * BITS;
        const int wd = bit / 32, sh = bit % 32;
        const u32x4 c00 = *reinterpret_cast<const u32x4*>(&vcode[wd][h8]);
        const u32x4 c01 = *reinterpret_cast<const u32x4*>(&vcode[wd][h8 + 4]);
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(&vscale[(lane * DV) / 16][h8]);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(&vscale[(lane * DV) / 16][h8 + 4]);
        uint32_t cw[8] = {c00.x, c00.y, c00.z, c00.w, c01.x, c01.y, c01.z, c01.w};
        const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
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
        // the group scale goes into operand A (one block = four lanes = one
        // 16-dim group), the centroids into operand B
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int hg = 0; hg < NG; ++hg) pa[hg][q] *= ss[q];
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
          for (int q = 0; q < 8; ++q) b[q][0] = sm.pro.vcen[cw[q] & ((1u << BITS) - 1u)];
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
            if constexpr (VF == KVQ_FP8_E4M3) {
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
            acc[hg][q & 1][v] = __builtin_amdgcn_mfma_f32_4x4x1f32(pa[hg][q], b[q][v], acc[hg][q & 1][v], 0, 0, 0);
    }
    wave_lds_sync();
  };

  // chunk loop: every load issued inside the loop, one chunk ahead
  constexpr int NB = KVQ_DENSE_BUFS;
  MfmaChunk<KF, VF, HD, G> cb[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
#pragma unroll
    for (int k = 0; k < MG::KQB / 4; ++k) cb[i].k[k] = 0u;
#pragma unroll
    for (int k = 0; k < MG::NSD; ++k) cb[i].v[k] = 0u;
    cb[i].s = 0u;
  }
  constexpr int step = kWaves * kChunk;
  int c = (sp.pb & ~(kChunk - 1)) + w * kChunk;  // next chunk to load; the one used trails by NB - 1
  if (c < sp.pe) {
    const int rounds = ((sp.pe - 1 - c) / step + 2 * NB - 1) / NB;
    for (int it = 0; it < rounds; ++it) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        mfma_load<KF, VF, HD, G>(a, sm.pro, first, c, sp.pb, sp.pe, tl.g, lane, cb[(i + NB - 1) % NB]);
        consume(c - (NB - 1) * step, cb[i]);
        c += step;
      }
    }
  }

  // the wave's state: sums over its 16 positions (lanes < 16), outputs by dim
  const uint64_t base = (uint64_t(tl.s) * a.num_kv_heads + tl.g) * a.nsplit + tl.split;
#pragma unroll
  for (int hg = 0; hg < NG; ++hg) {
    lsum[hg] = group_sum<16>(lsum[hg]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * hg + r;
      if (h < G) {
#pragma unroll
        for (int v = 0; v < DV; ++v) sm.red[w][h][lane * DV + v] = acc[hg][0][v][r] + acc[hg][1][v][r];
      }
    }
    const int h = 4 * hg + (lane >> 4);
    if ((lane & 15) == 0 && h < G) {  // a wave that saw no position reports -inf
      sm.red[w][h][HD] = lsum[hg] > 0.0f ? m[hg] : -INFINITY;
      sm.red[w][h][HD + 1] = lsum[hg];
    }
  }
  __syncthreads();
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

}  // namespace kvq
