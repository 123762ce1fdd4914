// Chunked prefill tile kernel: instances for the rotated K formats
// (turbo2/3/4, turbo8), compiled apart from the others.
#include "kvq_prefill.h"

namespace kvq {
namespace prefill {

hipError_t launch_rot(int kf, int vf, int hd, int G, const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  switch (kf) {
    case KVQ_TURBO2: return launch_kf<KVQ_TURBO2>(vf, hd, a, G, nwg, st);
    case KVQ_TURBO3: return launch_kf<KVQ_TURBO3>(vf, hd, a, G, nwg, st);
    case KVQ_TURBO4: return launch_kf<KVQ_TURBO4>(vf, hd, a, G, nwg, st);
    default: return launch_kf<KVQ_TURBO8>(vf, hd, a, G, nwg, st);
  }
}

}  // namespace prefill
}  // namespace kvq
