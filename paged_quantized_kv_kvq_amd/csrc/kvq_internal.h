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
#define KVQ_TARGET_WORKGROUPS 2048  // the split length is chosen to give about this many
#endif
#ifndef KVQ_MAX_SPARSE_SPLIT
#define KVQ_MAX_SPARSE_SPLIT 2048  // positions per split on the sparse path (scores kept in LDS)
#endif
#ifndef KVQ_VPART_POSITIONS
#define KVQ_VPART_POSITIONS 2048  // positions whose candidates one sparse-V workgroup takes
#endif
#ifndef KVQ_SCORE_DIMS
#define KVQ_SCORE_DIMS 0         // dims per lane in the sparse score kernel (0: as the dense kernel)
#endif
#ifndef KVQ_NT_LOADS
#define KVQ_NT_LOADS 0           // 1: K/V chunk loads carry the non-temporal hint
#endif

namespace kvq {

// fp32 Lloyd-Max tables for 2/3/4-bit codes, indexed [bits - 2].
struct Codebooks {
  float centroid[3][16];   // ascending
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
  int32_t* cnt;    // sparse: [S][Hkv][nsplit] candidate counts
  int32_t* cidx;   // sparse: [S][Hkv][nsplit][split_len] candidate positions
  uint64_t* cvbase; // sparse: [S][Hkv][nsplit][split_len] byte offset of their V page
  float* cscore;   // sparse: [S][Hkv][nsplit][split_len][G] their log2 scores
  float* vpart;    // sparse: [S][Hkv][nparts][G][hd] output partials of the V-pass parts
  uint32_t max_blocks;
  uint32_t num_seqs;
  uint32_t num_q_heads;
  uint32_t num_kv_heads;
  uint32_t log2_bs;
  uint32_t q_stride;
  uint32_t window;
  uint32_t split_len;
  uint32_t nsplit;
  uint32_t vsplits;  // sparse: splits per V-pass part
  uint32_t nparts;   // sparse: V-pass parts per (sequence, kv head) = ceil(nsplit / vsplits)
  uint64_t k_stride;
  uint64_t k_data;
  uint64_t v_stride;
  uint64_t v_data;
  float qk_scale;   // inv_sqrt_d * log2(e) (* k_scale for an fp8 K side)
  float v_scale;    // fp8 V side's scale, else 1
  float thr;        // sparse-V threshold (0: dense)
  float wht_scale;  // RN32(1/sqrt(head_dim))
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

hipError_t launch_scores_bf16(int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
hipError_t launch_scores_fp8(int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
hipError_t launch_scores_turbo2(int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
hipError_t launch_scores_turbo3(int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
hipError_t launch_scores_turbo4(int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
hipError_t launch_sparse_v(int vf, int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);
hipError_t launch_merge(bool sparse, bool v_rotated, int hd, int g, const DecodeArgs& a, hipStream_t st);

}  // namespace kvq
