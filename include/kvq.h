/*
 * kvq.h -- paged quantized KV cache for AMD Instinct MI355X (gfx950).
 *
 * Two steps of LLM decoding over a paged KV cache whose K and V sides are each
 * stored in one of seven formats (any K/V pairing):
 *   1. kvq_reshape_and_cache: write new K/V rows into the paged pools;
 *   2. kvq_paged_decode:      one query token per sequence attends to its pages
 *      (kvq_paged_prefill:    a chunk of query tokens per sequence, causally).
 * kvq_pool_layout gives the byte layout the caller allocates the pools with.
 *
 * Sources (web pages, cited by title and item):
 *   [kv_cache.rs]  "spark_runtime/kv_cache.rs" -- KvCacheDtype catalogue,
 *                  kv_pair / is_wht_rotated, KvCacheConfig::block_bytes_dims,
 *                  LayerPool (separate K / V block strides).
 *   [bf16k_turbov] "metrale_model_layers/layers/ops/kv_cache_bf16k_turbov.rs" --
 *                  module invariants (pool layout, code section then scales)
 *                  and the reshape_and_cache_* / paged_decode_attn_* launchers.
 *   [kv.rs]        "combs_models/kv.rs" -- repeat_kv (GQA), attend (scaled
 *                  softmax attention; decode needs no mask), paged gather.
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are HIP device pointers; "host" ones are host
 *     memory read before the call returns.  The entry points of this header
 *     allocate nothing, keep no state between calls (apart from constant
 *     tables built once per process) and never synchronize the host: work is
 *     queued on `stream` (a hipStream_t, NULL = the default stream) in call
 *     order.  (The host block manager of kvq_blocks.h keeps host bookkeeping
 *     of its own.)
 *   - Every argument is checked on the host before anything is launched; a
 *     failed check returns a negative kvq_status and launches nothing.  The
 *     checks cannot see device memory: slot ids, block ids and sequence
 *     lengths must lie in range (caller contract; an out-of-range id is a
 *     memory fault).  kvq_check_slots / kvq_check_tables validate host
 *     copies of those arrays for a debug mode.
 *   - Functions are thread-safe.  Concurrent calls that write the same pool
 *     slots or the same workspace race.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage format of one side (K or V) of the cache.  [kv_cache.rs] KvCacheDtype:
 *   KVQ_BF16      2 bytes per element, the bf16 bit pattern.
 *   KVQ_FP8_E4M3  1 byte per element: OCP E4M3FN of x / scale, one fp32 scale
 *                 per tensor supplied by the caller (clamped to +-448, round
 *                 to nearest even).
 *   KVQ_TURBO{2,3,4}  TurboQuant: the row (head_dim values) is rotated by the
 *                 orthonormal Walsh-Hadamard transform, re-rounded to bf16, and
 *                 every group of 16 elements is stored as 2/3/4-bit indices into
 *                 the Lloyd-Max codebook of a standard Gaussian, with one E4M3
 *                 scale byte (group absmax / largest centroid) per group.
 *   KVQ_TURBO8    [kv_cache.rs] KvCacheDtype::Turbo8, turbo8_data_bytes /
 *                 turbo8_scale_bytes: the row rotated and re-rounded as for
 *                 turbo, then one OCP E4M3FN byte per element (value / group
 *                 scale) and one BF16 scale per group of 16 (group absmax /
 *                 448, round to nearest even), 2 bytes, little-endian, in the
 *                 scale section.  An all-zero group stores zero bytes.
 *   KVQ_NVFP4     [kv_cache.rs] KvCacheDtype::Nvfp4, nvfp4_data_bytes /
 *                 nvfp4_scale_bytes (turbo4's byte layout): not rotated; per
 *                 group of 16 one E4M3 scale byte (group absmax / 6) and one
 *                 OCP E2M1 nibble per element (value / scale, saturated to +-6,
 *                 round to nearest even, sign kept; element 2k in the low
 *                 nibble of byte k).  A group whose scale encodes to 0 stores
 *                 zero nibbles.
 * Rotated sides (turbo2/3/4/8) make decode rotate the query (K side) and
 * rotate the output back (V side) -- [kv_cache.rs] is_wht_rotated. */
typedef enum kvq_format {
  KVQ_BF16 = 0,
  KVQ_FP8_E4M3 = 1,
  KVQ_TURBO2 = 2,
  KVQ_TURBO3 = 3,
  KVQ_TURBO4 = 4,
  KVQ_NVFP4 = 5,
  KVQ_TURBO8 = 8
} kvq_format;

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = -1,  /* a size, count, scale or pointer is invalid  */
  KVQ_ERR_UNSUPPORTED = -2,  /* valid, but outside what the kernels handle  */
  KVQ_ERR_ALIGNMENT = -3,    /* a pointer or stride is not 16-byte aligned  */
  KVQ_ERR_WORKSPACE = -4,    /* workspace missing or smaller than required  */
  KVQ_ERR_LAUNCH = -5,       /* the HIP runtime rejected a kernel launch    */
  KVQ_ERR_EXHAUSTED = -6,    /* the block manager has too few free blocks   */
  KVQ_ERR_HOST_MEMORY = -7   /* a host allocation failed; nothing changed   */
} kvq_status;

/* Byte layout of the two pools of one attention layer.
 * Pool element order [bf16k_turbov, module invariants]:
 *   [num_blocks, block_size, num_kv_heads, head_dim]; inside a block the flat
 *   element index of (offset, head, d) is e = (offset*num_kv_heads + head)*head_dim + d.
 * A block of one side is its code section (data_section_bytes) followed, for
 * turbo sides, by one E4M3 scale byte per group of 16 elements (byte e/16 of
 * the scale section).  Codes of b bits occupy bits [e*b, e*b+b) of the code
 * section read as a little-endian bit stream.  Blocks are block_stride_bytes
 * apart: the block's size [kv_cache.rs block_bytes_dims] rounded up to 16.
 * K and V have separate strides [kv_cache.rs LayerPool]. */
typedef struct kvq_layout {
  int32_t k_format;            /* kvq_format of the K side                     */
  int32_t v_format;            /* kvq_format of the V side                     */
  uint32_t block_size;         /* token positions per block                    */
  uint32_t num_kv_heads;
  uint32_t head_dim;
  uint32_t k_rotated;          /* 1 if the K side is stored WHT-rotated         */
  uint32_t v_rotated;          /* 1 if the V side is stored WHT-rotated         */
  uint32_t reserved;           /* 0                                            */
  uint64_t k_data_section_bytes;
  uint64_t k_block_stride_bytes;
  uint64_t v_data_section_bytes;
  uint64_t v_block_stride_bytes;
} kvq_layout;

/* Fill *out (host) with the pool layout for a (K format, V format) pair.
 * [kv_cache.rs] block_bytes_dims, k/v_block_bytes_for_layer.
 * Supported: block_size a power of two in [1, 1024]; num_kv_heads in [1, 256];
 * head_dim in {64, 128, 256}.  Pools hold num_blocks * *_block_stride_bytes
 * bytes; their base pointers must be 16-byte aligned.
 * Returns KVQ_OK, KVQ_ERR_INVALID_ARG (unknown format, zero size, out == NULL)
 * or KVQ_ERR_UNSUPPORTED (a size outside the supported set). */
int kvq_pool_layout(int32_t k_format, int32_t v_format, uint32_t block_size,
                    uint32_t num_kv_heads, uint32_t head_dim, kvq_layout* out);

/* Write num_tokens new K/V rows into the pools.
 * [bf16k_turbov] reshape_and_cache_bf16k_turbo{2,3,4}v; [kv_cache.rs] write path
 * (turbo sides rotated by wht before quantizing).
 *   layout        host; as filled by kvq_pool_layout (re-checked here).
 *   key, value    device bf16 [num_tokens, num_kv_heads, head_dim]; token t's
 *                 row of head h starts at element t*key_stride + h*head_dim
 *                 (value_stride for value).  16-byte aligned; strides are
 *                 multiples of 8 and >= num_kv_heads*head_dim.
 *   k_cache, v_cache  device pools (see kvq_layout).
 *   slot_mapping  device int64 [num_tokens]: slot = block*block_size + offset;
 *                 a negative slot skips the token.  Slots must be distinct.
 *   k_scale, v_scale  per-tensor scales of fp8 sides (finite, > 0); ignored
 *                 for other formats.
 * num_tokens == 0 returns KVQ_OK with nothing launched. */
int kvq_reshape_and_cache(const kvq_layout* layout, const void* key, const void* value,
                          void* k_cache, void* v_cache, const int64_t* slot_mapping,
                          uint32_t num_tokens, uint32_t key_stride, uint32_t value_stride,
                          float k_scale, float v_scale, void* stream);

/* Paged decode attention: for every sequence s and query head h (kv head
 * g = h / (num_q_heads/num_kv_heads), [kv.rs] repeat_kv):
 *   L = seq_lens[s] (counts the token just written); window start
 *   j0 = sliding_window ? max(0, L - sliding_window) : 0;
 *   score_j = inv_sqrt_d * <q, K_j> over j in [j0, L), K_j read from page
 *   block_tables[s][j / block_size] at offset j % block_size;
 *   p = softmax(score) over the window;
 *   out[s][h] = sum over j with p_j > sparse_v_threshold of p_j * V_j
 *   (no renormalization; threshold 0 = dense).
 * [bf16k_turbov] paged_decode_attn_bf16k_turbo{2,3,4}v (argument list, sparse-V
 * skip of a position's V "when its attention weight is at most" the threshold);
 * [kv.rs] attend.  Rotated K: the query is rotated first; rotated V: the
 * output is rotated back ([kv_cache.rs] is_wht_rotated).  An empty sequence
 * (L == 0) gives a zero row.
 *   q             device bf16 [num_seqs, num_q_heads, head_dim]; sequence s
 *                 starts at element s*q_stride (multiple of 8, >= Hq*head_dim).
 *   out           device fp32 [num_seqs, num_q_heads, head_dim], contiguous.
 *   block_tables  device int32 [num_seqs, max_blocks_per_seq]; entries past a
 *                 sequence's last page are never read.
 *   seq_lens      device int32 [num_seqs], each <= max_blocks_per_seq*block_size.
 *   num_q_heads   a multiple of num_kv_heads; the group size
 *                 num_q_heads/num_kv_heads must be 1, 2, 4 or 8.
 *   inv_sqrt_d    the score scale (finite, > 0), used as given.
 *   k_scale, v_scale  fp8 per-tensor scales (as passed to the write).
 *   workspace     device scratch of *workspace_bytes bytes (16-byte aligned),
 *                 overwritten by the call.  With workspace == NULL the call
 *                 only stores the required size in *workspace_bytes (host)
 *                 and returns KVQ_OK without launching; the size depends on
 *                 every size argument and on whether the threshold is 0.
 * Returns KVQ_OK or a negative kvq_status (nothing launched on error). */
int kvq_paged_decode(const kvq_layout* layout, const void* q, const void* k_cache,
                     const void* v_cache, float* out, const int32_t* block_tables,
                     const int32_t* seq_lens, uint32_t max_blocks_per_seq, uint32_t num_seqs,
                     uint32_t num_q_heads, float inv_sqrt_d, uint32_t q_stride,
                     uint32_t sliding_window, float sparse_v_threshold, float k_scale,
                     float v_scale, void* workspace, size_t* workspace_bytes, void* stream);

/* kvq_paged_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, results and errors are those
 * of kvq_paged_decode (same kernels, same plan; the outputs are bit-identical).
 * The scratch it needs lives in a device array inside the library of at most
 * 64 MiB per GPU, held from the first call on a GPU until the process ends;
 * a call whose kvq_paged_decode workspace size exceeds that returns
 * KVQ_ERR_WORKSPACE (nothing launched).  The call allocates nothing: no
 * hipMalloc, no allocating library routine.
 *   stream  must belong to the current device (else KVQ_ERR_INVALID_ARG); the
 *           first call on a device looks up that device's scratch address.
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one
 * GPU (other streams, other threads) race.  Nothing in the scratch needs to
 * start at zero; each call writes everything it reads. */
int kvq_paged_decode_noalloc(const kvq_layout* layout, const void* q, const void* k_cache,
                             const void* v_cache, float* out, const int32_t* block_tables,
                             const int32_t* seq_lens, uint32_t max_blocks_per_seq, uint32_t num_seqs,
                             uint32_t num_q_heads, float inv_sqrt_d, uint32_t q_stride,
                             uint32_t sliding_window, float sparse_v_threshold, float k_scale,
                             float v_scale, void* stream);

/* Chunked prefill attention over the same pools -- [kv.rs] attend with its
 * bottom-right causal mask (query at position p sees keys 0 .. p), after the
 * chunk's own K/V were written with kvq_reshape_and_cache; [kv_cache.rs]
 * names chunked prefill among the kernels every format covers.
 *   q            device, bf16 [T][num_q_heads][head_dim] with row stride
 *                q_stride elements: the queries of sequence s are rows
 *                query_start[s] .. query_start[s + 1] - 1, for positions
 *                seq_lens[s] - C_s .. seq_lens[s] - 1 (C_s = its row count,
 *                C_s <= seq_lens[s]; rows of positions below 0 are not written).
 *   out          device, fp32 [T][num_q_heads][head_dim], one row per query.
 *   query_start  device, int32 [num_seqs + 1], non-decreasing, query_start[0] = 0.
 *   max_query_len  host: the largest C_s (sizes the grid; larger chunks are a
 *                caller error: their later queries are not computed).
 *   block_tables, seq_lens, max_blocks_per_seq, inv_sqrt_d, sliding_window
 *                (per query: keys p - W < j <= p), k_scale, v_scale, workspace,
 *                workspace_bytes, stream: as for kvq_paged_decode.  No sparse-V
 *                threshold: the skip is a decode feature.
 * With block_size >= 4, tiles of queries run on the matrix cores: tiles of
 * 128 (query, head) rows (64 at head_dim 256 or with a rotated K side) share
 * each dequantized K/V chunk and write their rows directly; the workspace
 * holds the order in which the (sequence, kv head) units run, 4 bytes each
 * (longest first), and, when a small grid splits the key ranges, the
 * per-split partial rows that a second kernel merges.  With block_size < 4
 * every query runs as its own decode row through the decode kernels, which
 * reads the keys once per query; the workspace covers num_seqs *
 * max_query_len rows there. */
int kvq_paged_prefill(const kvq_layout* layout, const void* q, const void* k_cache, const void* v_cache, float* out,
                      const int32_t* block_tables, const int32_t* seq_lens, const int32_t* query_start,
                      uint32_t max_blocks_per_seq, uint32_t num_seqs, uint32_t num_q_heads, uint32_t max_query_len,
                      float inv_sqrt_d, uint32_t q_stride, uint32_t sliding_window, float k_scale, float v_scale,
                      void* workspace, size_t* workspace_bytes, void* stream);

/* Debug validation of index arrays (host only; nothing is launched).  The
 * entry points above cannot see device memory, so an out-of-range slot or
 * page id there is a memory fault.  A caller in a debug mode copies its index
 * arrays to the host and calls these first; each returns KVQ_OK, or
 * KVQ_ERR_INVALID_ARG with the first offending token / sequence in
 * *first_bad (host, may be NULL).  num_blocks is the number of blocks the
 * pools hold.  Sources as for the calls they guard: [bf16k_turbov] slot =
 * block*block_size + offset, block_tables / seq_lens; [kv.rs] the paged
 * gather (position j in page table[j / block_size]).
 *
 * kvq_check_slots: every slot_mapping[t] (host int64 [num_tokens]) is
 *   negative (skipped) or < num_blocks*block_size, and the non-negative ones
 *   are distinct (two writes of one slot in one call race). */
int kvq_check_slots(const kvq_layout* layout, const int64_t* slot_mapping, uint32_t num_tokens,
                    uint64_t num_blocks, uint32_t* first_bad);

/* kvq_check_tables: for every sequence s, 0 <= seq_lens[s] <=
 *   max_blocks_per_seq*block_size, and every block_tables[s][i] (host int32
 *   [num_seqs][max_blocks_per_seq]) that a decode (query_start == NULL) or a
 *   chunked prefill (query_start: host int32 [num_seqs + 1]) reads lies in
 *   [0, num_blocks): the pages of positions [j0, L) with the window start j0
 *   of the call.  For prefill also query_start[0] == 0, non-decreasing, and
 *   query_start[s + 1] - query_start[s] <= seq_lens[s]. */
int kvq_check_tables(const kvq_layout* layout, const int32_t* block_tables, const int32_t* seq_lens,
                     const int32_t* query_start, uint32_t max_blocks_per_seq, uint32_t num_seqs,
                     uint32_t sliding_window, uint64_t num_blocks, uint32_t* first_bad);

/* Introspection (host only): the fp32 Lloyd-Max tables the turbo format uses.
 * centroids[0..L-1] ascending, thresholds[1..L-1] (midpoints; [0] = 0),
 * *inv_cmax = 1/largest centroid, *levels = L = 2^bits.  Buffers hold 16 floats.
 * Returns KVQ_ERR_INVALID_ARG for a format without a Lloyd-Max codebook (bf16,
 * fp8, turbo8, nvfp4) or a NULL pointer. */
int kvq_codebook(int32_t format, float* centroids, float* thresholds, float* inv_cmax,
                 uint32_t* levels);

/* Static, human-readable name of a kvq_status value. */
const char* kvq_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
