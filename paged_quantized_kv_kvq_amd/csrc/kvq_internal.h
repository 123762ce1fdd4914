// Internal interface between the exported C-ABI (kvq_api.hip) and the kernel
// translation units.  Plain structs passed by value as kernel arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/kvq.h"

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
  uint32_t max_blocks;
  uint32_t num_seqs;
  uint32_t num_q_heads;
  uint32_t num_kv_heads;
  uint32_t log2_bs;
  uint32_t q_stride;
  uint32_t window;
  uint32_t split_len;
  uint32_t nsplit;
  uint32_t pad0;
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
hipError_t launch_sparse_v(int vf, int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st);  // one workgroup per (seq, kv head)
hipError_t launch_merge(bool v_rotated, int hd, int g, const DecodeArgs& a, hipStream_t st);

}  // namespace kvq
