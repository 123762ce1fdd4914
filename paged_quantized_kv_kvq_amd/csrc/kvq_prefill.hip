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

hipError_t launch_prefill_tile_merge(bool v_rotated, int hd, int G, const DecodeArgs& a, hipStream_t st) {
  const uint64_t waves = uint64_t(a.num_seqs) * a.ntiles * a.num_kv_heads * a.qt * uint32_t(G);
  const dim3 grid(uint32_t((waves + 3) / 4)), block(256);
  switch (hd) {
    case 64:
      if (v_rotated) prefill::tile_merge_kernel<64, true><<<grid, block, 0, st>>>(a, G);
      else prefill::tile_merge_kernel<64, false><<<grid, block, 0, st>>>(a, G);
      break;
    case 128:
      if (v_rotated) prefill::tile_merge_kernel<128, true><<<grid, block, 0, st>>>(a, G);
      else prefill::tile_merge_kernel<128, false><<<grid, block, 0, st>>>(a, G);
      break;
    default:
      if (v_rotated) prefill::tile_merge_kernel<256, true><<<grid, block, 0, st>>>(a, G);
      else prefill::tile_merge_kernel<256, false><<<grid, block, 0, st>>>(a, G);
      break;
  }
  return hipGetLastError();
}

}  // namespace kvq
