// Decode kernels with a turbo8 K side: the dense split kernel for every V format,
// head_dim and group size, and the score kernel of the sparse-V path.
#include "kvq_decode.h"

namespace kvq {

hipError_t launch_split_turbo8(int vf, int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  return launch_split_k<KVQ_TURBO8>(vf, hd, g, a, nwg, st);
}

hipError_t launch_scores_turbo8(int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  return launch_scores_k<KVQ_TURBO8>(hd, g, a, nwg, st);
}

}  // namespace kvq
