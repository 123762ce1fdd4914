// Decode kernels with a turbo3 K side: the dense split kernel for every V format,
// head_dim and group size, and the score kernel of the sparse-V path.
#include "kvq_decode.h"

namespace kvq {

hipError_t launch_split_turbo3(int vf, int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  return launch_split_k<KVQ_TURBO3>(vf, hd, g, a, nwg, st);
}

hipError_t launch_scores_turbo3(int hd, int g, const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  return launch_scores_k<KVQ_TURBO3>(hd, g, a, nwg, st);
}

}  // namespace kvq
