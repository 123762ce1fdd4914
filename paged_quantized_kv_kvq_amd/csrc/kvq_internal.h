// Internal interface between the exported C-ABI (kvq_api.hip) and the kernel
// translation units.  Plain structs passed by value as kernel arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvq.h"

// Tuning constants (compile-time; the defaults are the measured best on MI355X).
#ifndef KVQ_WAVES
#define KVQ_WAVES 4              // waves per decode workgroup
#endif
#ifndef KVQ_TARGET_WORKGROUPS
#define KVQ_TARGET_WORKGROUPS 2048  // the split length is chosen to give about this many (kv head, split) units
#endif
#ifndef KVQ_MAX_PAGES
#define KVQ_MAX_PAGES 160        // page offsets of one decode split staged in LDS
#endif
#ifndef KVQ_MFMA_MAX_PAGES
#define KVQ_MFMA_MAX_PAGES 260   // ... for the matrix-core split kernel with a bf16 / fp8 K side
#endif
#ifndef KVQ_MAX_SPLIT
#define KVQ_MAX_SPLIT 4096       // longest decode split (positions)
#endif
#ifndef KVQ_MIN_WORKGROUPS
#define KVQ_MIN_WORKGROUPS 1024  // ... and dense splits are shortened until the split kernel gets this many workgroups
#endif
#ifndef KVQ_SPARSE_TARGET_WORKGROUPS
#define KVQ_SPARSE_TARGET_WORKGROUPS 512  // ... on the sparse path (its score kernel runs one workgroup per unit)
#endif
#ifndef KVQ_MAX_SPARSE_SPLIT
#define KVQ_MAX_SPARSE_SPLIT 2048  // positions per split on the sparse path (scores kept in LDS)
#endif
#ifndef KVQ_VWAVES
#define KVQ_VWAVES 8             // waves of a sparse-V workgroup
#endif
#ifndef KVQ_V_TARGET_WORKGROUPS
#define KVQ_V_TARGET_WORKGROUPS 512  // the sparse V pass splits each (sequence, kv head) into parts up to about this many
#endif
#ifndef KVQ_SCORE_DIMS
#define KVQ_SCORE_DIMS 0         // dims per lane in the sparse score kernel (0: as the dense kernel)
#endif
#ifndef KVQ_SCORE_ORDER
#define KVQ_SCORE_ORDER 1        // 1: the sparse score kernel takes its units longest first
#endif
#ifndef KVQ_EQ_SPLITS
#define KVQ_EQ_SPLITS 1          // 1: on the dense path a sequence's splits share its span equally
#endif
#ifndef KVQ_DENSE_ORDER
#define KVQ_DENSE_ORDER 1        // 1: the dense split kernel takes its units longest first
#endif
#ifndef KVQ_SCORE_MFMA
#define KVQ_SCORE_MFMA 1         // 1: the sparse score kernel scores a grouped-scale K side on the matrix cores
#endif
#ifndef KVQ_SCORE_ORDER_INLINE
#define KVQ_SCORE_ORDER_INLINE 1  // 1: small sparse launches order their units inside the score kernel
#endif
#ifndef KVQ_SCORE_MFMA_BUFS
#define KVQ_SCORE_MFMA_BUFS 2    // ... its chunk buffers per wave
#endif
#ifndef KVQ_SCORE_LOOKUPS
#define KVQ_SCORE_LOOKUPS 16     // ... its code-pair lookups requested at once
#endif
#ifndef KVQ_SCORE_WAVES
#define KVQ_SCORE_WAVES 8        // waves of the sparse score kernel's VALU form (its matrix-core form: 4)
#endif
#ifndef KVQ_SCORE_BUFS
#define KVQ_SCORE_BUFS 2         // chunk buffers per wave in the sparse score kernel (loads run this - 1 ahead)
#endif
#ifndef KVQ_DENSE_MFMA
#define KVQ_DENSE_MFMA 1         // 1: dense split pass on the matrix cores where the operands allow
#endif
#ifndef KVQ_DENSE_BUFS
#define KVQ_DENSE_BUFS 2         // chunk buffers per wave in the dense split kernel
#endif
#ifndef KVQ_TILE_DENSE
#define KVQ_TILE_DENSE 1         // workgroup -> (unit, kv head) map of the dense split kernel (see unit_tile)
#endif
#ifndef KVQ_TILE_SCORES
#define KVQ_TILE_SCORES 1        // ... of the sparse score kernel
#endif
#ifndef KVQ_TILE_SPARSE_V
#define KVQ_TILE_SPARSE_V 1      // ... of the sparse V pass
#endif
#ifndef KVQ_PREFILL_TILES
#define KVQ_PREFILL_TILES 1      // 1: chunked prefill on the tile kernel (kvq_prefill.h) where block_size >= 4
#endif
#ifndef KVQ_PREFILL_ORDER
#define KVQ_PREFILL_ORDER 1      // 1: prefill units (sequence, kv head, split) start longest first
#endif
#ifndef KVQ_PREFILL_TILE_DESC
#define KVQ_PREFILL_TILE_DESC 1  // 1: a unit's prefill tiles start from the last (longest key range)
#endif
#ifndef KVQ_NT_LOADS
#define KVQ_NT_LOADS 0           // 1: K/V chunk loads carry the non-temporal hint
#endif

namespace kvq {

// Whether the dense split pass runs on the matrix cores for these formats and
// head_dim (bf16 / fp8 K: bf16 MFMA for Q.K^T; turbo K: fp32 MFMA over the
// rotated query; V rows of at most 128 bytes); it also needs block_size >= 16.
// Page offsets one split of the dense decode pass may stage: the matrix-core
// kernel with a bf16 / fp8 K side takes longer splits (fewer partials to
// write and merge; workload 3: 16 -> 8 splits per sequence, 2% faster), the
// grouped-scale K paths keep shorter ones (longer ones measured 6% slower on
// workloads 6 and 7).
__host__ __device__ constexpr int dense_max_pages(int kf) {
  return kf == KVQ_BF16 || kf == KVQ_FP8_E4M3 ? KVQ_MFMA_MAX_PAGES : KVQ_MAX_PAGES;
}

// Most kv heads (waves) per workgroup of the matrix-core split kernel: four
// with a grouped-scale K side, else eight; and the heads per workgroup for
// nkv kv heads (the largest divisor of nkv up to that cap).
__host__ __device__ constexpr int mfma_waves_cap_of(int kf, int g) { return (kf >= KVQ_TURBO2 && g <= 8) ? 4 : 8; }
__host__ __device__ constexpr uint32_t mfma_unit_waves(uint32_t nkv, uint32_t cap) {
  for (uint32_t d = cap; d > 1; --d)
    if (nkv % d == 0) return d;
  return 1;
}

// The sparse score kernel scores a grouped-scale K side on the matrix cores
// (the dense kernel's turbo-K operand layout) where its quarter rows fit and
// G <= 4, and block_size >= 16 (a 16-position chunk in one page).
__host__ __device__ constexpr bool mfma_scores_ok(int kf, int hd, int g) {
  const int kqb = hd * (kf == KVQ_NVFP4 ? 4 : kf) / 32;  // K bytes per lane and chunk (a quarter of a row)
  return kf >= KVQ_TURBO2 && g <= 4 && kqb % 4 == 0 && kqb <= 32 && hd / 4 >= 16;
}

// Waves of the sparse score kernel, one record segment each: four for the
// matrix-core form, KVQ_SCORE_WAVES for the VALU one.
__host__ __device__ constexpr bool scores_on_mfma(int kf, int hd, int g, uint32_t bs) {
  return KVQ_SCORE_MFMA && mfma_scores_ok(kf, hd, g) && bs >= 16;
}
__host__ __device__ constexpr uint32_t score_waves(bool mfma) { return mfma ? 4u : uint32_t(KVQ_SCORE_WAVES); }

__host__ __device__ constexpr bool mfma_split_ok(int kf, int vf, int hd) {
  const int kbits = kf == KVQ_BF16 ? 16 : kf == KVQ_FP8_E4M3 ? 8 : kf == KVQ_NVFP4 ? 4 : kf;
  const int vbits = vf == KVQ_BF16 ? 16 : vf == KVQ_FP8_E4M3 ? 8 : vf == KVQ_NVFP4 ? 4 : vf;
  const int kqb = hd * kbits / 32;  // K bytes per lane and chunk (a quarter of a row)
  const bool kturbo = kf >= KVQ_TURBO2;  // grouped-scale K (codes through a table or turbo8's E4M3 values)
  return hd * vbits / 8 <= 128 &&
         (kturbo ? (kqb % 4 == 0 && kqb <= 32 && hd / 4 >= 16) : (kqb <= 64 && kqb % 16 == 0));
}

// fp32 Lloyd-Max tables for 2/3/4-bit codes, indexed [bits - 2], and NVFP4's
// E2M1 values (row KVQ_NVFP4 - 2, in nibble order); a 4-bit-or-smaller format
// F reads its table at row F - 2.
struct Codebooks {
  float centroid[4][16];   // Lloyd-Max rows ascending
  float threshold[3][16];  // [k] = midpoint of centroids k-1 and k; [0] unused
  float inv_cmax[3];       // 1 / largest centroid
};

const Codebooks& codebooks();  // built once per process (host)

struct WriteArgs {
  const uint16_t* key;
  const uint16_t* value;
  uint8_t* k_cache;
  uint8_t* v_cache;
  const int64_t* slots;
  uint32_t num_tokens;
  uint32_t num_kv_heads;
  uint32_t log2_bs;
  uint32_t key_stride;
  uint32_t value_stride;
  int32_t k_format;
  int32_t v_format;
  uint32_t pad0;
  uint64_t k_stride;
  uint64_t k_data;
  uint64_t v_stride;
  uint64_t v_data;
  float k_scale;
  float v_scale;
  float wht_scale;  // RN32(1/sqrt(head_dim))
  float pad1;
  Codebooks cb;
};

// Sparse-V candidate lists hold one segment per (split, wave of the score
// kernel).  With `segs` waves, a wave scores every segs-th chunk of 16
// positions of its split, so a segment never holds more than
// cand_segment_cap records (at least 64: the V pass reads one record per
// lane ahead of the counts).
__host__ __device__ constexpr uint32_t cand_segment_cap(uint32_t split_len, uint32_t segs) {
  return ((split_len + 15u) / (16u * segs) + 1u) * 16u < 64u ? 64u : ((split_len + 15u) / (16u * segs) + 1u) * 16u;
}
// Words per candidate record: page id, position, G scores, padded to 16 bytes.
__host__ __device__ constexpr uint32_t cand_record_words(uint32_t g) { return (2u + g + 3u) / 4u * 4u; }

// Most workgroups the sparse V pass gives one (sequence, kv head).
constexpr uint32_t kMaxVParts = 8;

struct DecodeArgs {
  const uint16_t* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  float* out;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* part;     // dense: [S][Hkv][nsplit][G][hd] unnormalized partial
                   // outputs of each split (relative to the split max)
  float* ml;       // [S][Hkv][nsplit][G][2] (max in log2 units, sum of exp2)
  int32_t* cnt;    // sparse: [S][Hkv][nsplit][KVQ_WAVES] candidate counts per segment
  uint32_t* crec;  // sparse: [S][Hkv][nsplit][KVQ_WAVES][seg_cap] candidate records
                   // of cand_record_words(G) words: page id, position, G log2 scores
  float* vpart;    // sparse, vparts > 1: [S][Hkv][vparts][G][hd] the V parts' sums
  uint32_t* order;  // [S * nsplit] units (split * S + sequence), longest first (null: in that order)
  uint32_t lpt_inline;  // sparse VALU score kernel: each workgroup finds its unit of the longest-first order
  uint32_t max_blocks;
  uint32_t num_seqs;
  uint32_t num_q_heads;
  uint32_t num_kv_heads;
  uint32_t log2_bs;
  uint32_t q_stride;
  uint32_t window;
  uint32_t split_len;
  uint32_t nsplit;
  uint32_t seg_cap;  // sparse: records per segment, cand_segment_cap(split_len, segs)
  uint32_t segs;     // sparse: record segments per split (the score kernel's waves)
  uint32_t vparts;   // sparse: V-pass workgroups per (sequence, kv head)
  uint32_t eq_split;  // 1: a sequence's splits share its span equally (split_span)
  uint64_t k_stride;
  uint64_t k_data;
  uint64_t v_stride;
  uint64_t v_data;
  float qk_scale;   // inv_sqrt_d * log2(e) (* k_scale for an fp8 K side)
  float v_scale;    // fp8 V side's scale, else 1
  float thr;        // sparse-V threshold (0: dense)
  float wht_scale;  // RN32(1/sqrt(head_dim))
  // chunked prefill run as decode rows (block sizes the prefill tiles do
  // not take): row s of the call is query row vrow[2 s + 1] of sequence
  // vrow[2 s] (-1: no query), its length that query's position + 1; null in
  // a plain decode call (row s is sequence s)
  const int32_t* vrow;
  const int32_t* query_start;  // chunked prefill: [S + 1] first query row of each sequence
  uint32_t ntiles;             // ... tiles of qt queries per sequence (of the longest chunk)
  uint32_t qt;                 // ... queries per tile
  Codebooks cb;
};

// Launchers (return the HIP launch status).  Template instances live in one
// translation unit per K format (split / score kernels) and per V format.
hipError_t launch_write(int head_dim, const WriteArgs& a, hipStream_t st);

hipError_t launch_split_bf16(int vf, int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
hipError_t launch_split_fp8(int vf, int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
hipError_t launch_split_turbo2(int vf, int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
hipError_t launch_split_turbo3(int vf, int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
hipError_t launch_split_turbo4(int vf, int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
hipError_t launch_split_turbo8(int vf, int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
hipError_t launch_split_nvfp4(int vf, int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);

hipError_t launch_scores_bf16(int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
hipError_t launch_scores_fp8(int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
hipError_t launch_scores_turbo2(int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
hipError_t launch_scores_turbo3(int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
hipError_t launch_scores_turbo4(int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
hipError_t launch_scores_turbo8(int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
hipError_t launch_scores_nvfp4(int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
// Chunked prefill as decode rows: vrow / vlen of the num_seqs * max_query_len
// rows (row s * max_query_len + i is query i of sequence s).
hipError_t launch_prefill_rows(const int32_t* query_start, const int32_t* seq_lens, uint32_t num_seqs,
                               uint32_t max_query_len, int32_t* vrow, int32_t* vlen, hipStream_t st);
// Chunked prefill on the tile kernel: (query, head) rows per workgroup for a
// K format and head_dim, and the launcher (grid of nwg workgroups).
int prefill_tile_rows(int kf, int hd);
hipError_t launch_prefill_tiles(int kf, int vf, int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
// ... and the merge of its key splits (a.nsplit > 1)
hipError_t launch_prefill_tile_merge(bool v_rotated, int hd, int g, const DecodeArgs& a, hipStream_t st);
// The order in which a split kernel takes its units (a.order): decode units
// (mode 0) or prefill tile units (mode 1), lengths bucketed by `width`
hipError_t launch_unit_order(const DecodeArgs& a, hipStream_t st, int mode = 0, int width = 16);
hipError_t launch_sparse_v(int vf, int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
// ... and the sum of its parts (a.vparts > 1), one workgroup per (sequence, kv head)
hipError_t launch_sparse_v_merge(bool v_rotated, int hd, int g, const DecodeArgs& a, hipStream_t st);
hipError_t launch_merge(bool v_rotated, int hd, int g, const DecodeArgs& a, hipStream_t st);

}  // namespace kvq
