// Chunked prefill tile kernel: the K formats exact in bf16 (bf16, fp8,
// NVFP4), and the entry points the C ABI calls.
#include "kvq_prefill.h"

namespace kvq {

int prefill_tile_rows(int kf, int hd) {
  using prefill::TGeo;
  static_assert(TGeo<KVQ_BF16, 128>::ROWS == 128 && TGeo<KVQ_BF16, 256>::ROWS == 64 &&
                    TGeo<KVQ_NVFP4, 128>::ROWS == 128 && TGeo<KVQ_TURBO4, 128>::ROWS == 64,
                "rows per tile");
  const bool rot = kf == KVQ_TURBO2 || kf == KVQ_TURBO3 || kf == KVQ_TURBO4 || kf == KVQ_TURBO8;
  return rot || hd > 128 ? 64 : 128;
}

hipError_t launch_prefill_tiles(int kf, int vf, int hd, int G, const DecodeArgs& a, uint32_t nwg, hipStream_t st) {
  switch (kf) {
    case KVQ_BF16: return prefill::launch_kf<KVQ_BF16>(vf, hd, a, G, nwg, st);
    case KVQ_FP8_E4M3: return prefill::launch_kf<KVQ_FP8_E4M3>(vf, hd, a, G, nwg, st);
    case KVQ_NVFP4: return prefill::launch_kf<KVQ_NVFP4>(vf, hd, a, G, nwg, st);
    default: return prefill::launch_rot(kf, vf, hd, G, a, nwg, st);
  }
}

}  // namespace kvq
