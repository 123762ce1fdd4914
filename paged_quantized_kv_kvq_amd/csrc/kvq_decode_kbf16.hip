// Decode kernels with a bf16 K side: the dense split kernel for every V format,
// head_dim and group size, and the score kernel of the sparse-V path.
#include "kvq_decode.h"

namespace kvq {

hipError_t launch_split_bf16(int vf, int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  return launch_split_k<KVQ_BF16>(vf, hd, g, a, nwg, st);
}

hipError_t launch_scores_bf16(int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  return launch_scores_k<KVQ_BF16>(hd, g, a, nwg, st);
}

}  // namespace kvq
