// The exported C ABI: argument checks, pool layout, Lloyd-Max tables, decode
// planning and kernel dispatch.  Device memory is only reached through the
// kernels; the one device object defined here is the scratch array of the
// allocation-free decode.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr uint32_t kMaxSplitLen = KVQ_MAX_SPLIT;
constexpr uint32_t kMaxSparseSplitLen = KVQ_MAX_SPARSE_SPLIT;  // scores of a split live in LDS
constexpr uint32_t kPagesPerSplit = KVQ_MAX_PAGES;             // page offsets of a split live in LDS
constexpr uint64_t kTargetWorkgroups = KVQ_TARGET_WORKGROUPS;
constexpr uint64_t kSparseTargetWorkgroups = KVQ_SPARSE_TARGET_WORKGROUPS;
constexpr uint64_t kMinWorkgroups = KVQ_MIN_WORKGROUPS;
constexpr uint64_t kVTargetWorkgroups = KVQ_V_TARGET_WORKGROUPS;
// chunked prefill on the tile kernel: a grid of fewer workgroups than this
// splits the tiles' key ranges (two per CU fill the GPU), into splits of at
// least kTileSplitChunks chunks
constexpr uint64_t kTilePrefillWorkgroups = 512;
constexpr uint64_t kTileSplitChunks = 16;

bool valid_format(int32_t f) { return (f >= KVQ_BF16 && f <= KVQ_NVFP4) || f == KVQ_TURBO8; }
bool is_rotated(int32_t f) { return f >= KVQ_TURBO2 && f != KVQ_NVFP4; }  // is_wht_rotated
bool has_codebook(int32_t f) { return f >= KVQ_TURBO2 && f <= KVQ_TURBO4; }  // Lloyd-Max books
// scale bytes per group of 16 elements: E4M3 for the 2/3/4-bit formats, BF16 for turbo8
uint64_t scale_bytes_per_group(int32_t f) {
  return (has_codebook(f) || f == KVQ_NVFP4) ? 1u : f == KVQ_TURBO8 ? 2u : 0u;
}
uint32_t format_bits(int32_t f) {
  return f == KVQ_BF16 ? 16u : f == KVQ_FP8_E4M3 ? 8u : f == KVQ_NVFP4 ? 4u : uint32_t(f);
}
bool pow2(uint64_t x) { return x && !(x & (x - 1)); }
uint32_t log2u(uint64_t x) {
  uint32_t r = 0;
  while ((1ull << r) < x) ++r;
  return r;
}
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Lloyd-Max quantizer of N(0,1) with L levels: iterate the two optimality
// conditions (thresholds at centroid midpoints; centroids at the conditional
// mean (pdf(a) - pdf(b)) / (cdf(b) - cdf(a)) of their cell) over all L cells,
// mirroring the result after every sweep to keep it exactly symmetric.
double gauss_pdf(double x) { return std::isinf(x) ? 0.0 : std::exp(-0.5 * x * x) * 0.3989422804014327; }

// cdf(b) - cdf(a) without cancellation in either tail
double gauss_mass(double a, double b) {
  const double r = 0.7071067811865476;
  if (a >= 0.0) return 0.5 * (std::erfc(a * r) - std::erfc(b * r));
  if (b <= 0.0) return 0.5 * (std::erfc(-b * r) - std::erfc(-a * r));
  return 1.0 - 0.5 * std::erfc(-a * r) - 0.5 * std::erfc(b * r);
}

void lloyd_max(int L, double* c) {
  for (int k = 0; k < L; ++k) c[k] = -3.0 + 6.0 * (k + 0.5) / L;
  int settle = 2000;
  for (int it = 0; it < 100000; ++it) {
    double t[17];
    t[0] = -INFINITY;
    t[L] = INFINITY;
    for (int k = 1; k < L; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
    double nc[16], delta = 0.0;
    for (int k = 0; k < L; ++k) nc[k] = (gauss_pdf(t[k]) - gauss_pdf(t[k + 1])) / gauss_mass(t[k], t[k + 1]);
    for (int k = 0; k < L / 2; ++k) {
      const double v = 0.5 * (nc[L - 1 - k] - nc[k]);
      nc[k] = -v;
      nc[L - 1 - k] = v;
    }
    for (int k = 0; k < L; ++k) {
      delta = std::fmax(delta, std::fabs(nc[k] - c[k]));
      c[k] = nc[k];
    }
    if (delta <= 1e-15 && (--settle < 0 || delta == 0.0)) break;
  }
}

Codebooks build_codebooks() {
  Codebooks cb;
  std::memset(&cb, 0, sizeof(cb));
  for (int bits = 2; bits <= 4; ++bits) {
    const int L = 1 << bits;
    double c[16];
    lloyd_max(L, c);
    for (int k = 0; k < L; ++k) cb.centroid[bits - 2][k] = float(c[k]);
    for (int k = 1; k < L; ++k) cb.threshold[bits - 2][k] = float(0.5 * (c[k - 1] + c[k]));
    cb.inv_cmax[bits - 2] = float(1.0 / c[L - 1]);
  }
  // NVFP4's table: the value of every E2M1 nibble (sign in bit 3, two
  // exponent bits with bias 1, one mantissa bit; exponent 0 is subnormal)
  for (int code = 0; code < 16; ++code) {
    const int e = (code >> 1) & 3, m = code & 1;
    const float mag = e == 0 ? 0.5f * float(m) : (1.0f + 0.5f * float(m)) * float(1 << e) * 0.5f;
    cb.centroid[KVQ_NVFP4 - 2][code] = (code & 8) ? -mag : mag;
  }
  return cb;
}

int layout_impl(int32_t kf, int32_t vf, uint32_t bs, uint32_t nkv, uint32_t hd, kvq_layout* out) {
  if (!out || !valid_format(kf) || !valid_format(vf) || bs == 0 || nkv == 0 || hd == 0)
    return KVQ_ERR_INVALID_ARG;
  if (!pow2(bs) || bs > 1024 || nkv > 256 || (hd != 64 && hd != 128 && hd != 256)) return KVQ_ERR_UNSUPPORTED;
  const uint64_t e = uint64_t(bs) * nkv * hd;
  kvq_layout l;
  std::memset(&l, 0, sizeof(l));
  l.k_format = kf;
  l.v_format = vf;
  l.block_size = bs;
  l.num_kv_heads = nkv;
  l.head_dim = hd;
  l.k_rotated = is_rotated(kf) ? 1u : 0u;
  l.v_rotated = is_rotated(vf) ? 1u : 0u;
  const int32_t fmts[2] = {kf, vf};
  uint64_t data[2], stride[2];
  for (int i = 0; i < 2; ++i) {
    data[i] = e * format_bits(fmts[i]) / 8;
    const uint64_t bytes = data[i] + e / 16 * scale_bytes_per_group(fmts[i]);
    stride[i] = (bytes + 15) / 16 * 16;
  }
  l.k_data_section_bytes = data[0];
  l.k_block_stride_bytes = stride[0];
  l.v_data_section_bytes = data[1];
  l.v_block_stride_bytes = stride[1];
  *out = l;
  return KVQ_OK;
}

// A layout handed back by the caller must be exactly one this library made.
int check_layout(const kvq_layout* l) {
  if (!l) return KVQ_ERR_INVALID_ARG;
  kvq_layout ref;
  const int st = layout_impl(l->k_format, l->v_format, l->block_size, l->num_kv_heads, l->head_dim, &ref);
  if (st != KVQ_OK) return st;
  return std::memcmp(&ref, l, sizeof(ref)) == 0 ? KVQ_OK : KVQ_ERR_INVALID_ARG;
}

bool good_scale(float s) { return std::isfinite(s) && s > 0.0f; }

struct Plan {
  uint32_t split_len, nsplit, seg_cap, segs, vparts;
  uint64_t off_part, off_ml, off_cnt, off_crec, off_vpart, off_order, bytes;
};

uint64_t up256(uint64_t x) { return (x + 255) / 256 * 256; }

// Page offsets a split may stage for the kernel that will run: the
// matrix-core split kernel (KVQ_DENSE_MFMA, operands it takes, block_size
// >= 16) by its K format, everything else the common limit.
bool dense_on_mfma(const kvq_layout* layout, bool sparse) {
  return KVQ_DENSE_MFMA && !sparse && layout->block_size >= 16 &&
         mfma_split_ok(layout->k_format, layout->v_format, int(layout->head_dim));
}
uint32_t dense_pages(const kvq_layout* layout, bool sparse) {
  return dense_on_mfma(layout, sparse) ? uint32_t(dense_max_pages(layout->k_format)) : kPagesPerSplit;
}

// Workgroups of the split kernel per (sequence, split): one per kv head, or
// one per group of kv heads on the matrix-core kernel.
uint32_t wg_per_unit(const kvq_layout* layout, uint32_t G, bool sparse) {
  const uint32_t nkv = layout->num_kv_heads;
  if (!dense_on_mfma(layout, sparse)) return nkv;
  return nkv / mfma_unit_waves(nkv, uint32_t(mfma_waves_cap_of(layout->k_format, int(G))));
}

// Split length: the smallest power of two >= 256 giving about
// kTargetWorkgroups (kv head, split) units over the longest possible window
// (dense: a workgroup serves up to eight kv heads of a split), or
// kSparseTargetWorkgroups on the sparse path, whose score kernel runs a
// workgroup per unit: two per CU, all resident at once, instead of 2048
// shorter ones over several rounds (workload 4: score pass 50 -> 43 us).
// On the dense path, then halved while the split kernel would get fewer than
// kMinWorkgroups workgroups (wpu per (sequence, split)) over the longest
// possible window (the table's reach; shorter sequences leave some empty):
// with 194 VGPRs (turbo4 K, G = 8) the matrix-core kernel holds few waves
// per CU, and 32 sequences of 4096-16384 positions in long splits left CUs
// idle (0.35 -> 0.31 ms with shorter splits, the units longest first).
Plan make_plan(uint32_t S, uint32_t nkv, uint32_t G, uint32_t hd, uint32_t max_blocks, uint32_t bs,
               uint32_t window, bool sparse, uint32_t max_pages, uint32_t wpu, uint32_t segs) {
  uint64_t span = uint64_t(max_blocks) * bs;
  if (window && window < span) span = window;
  const uint64_t work = span * S * nkv;
  uint32_t sl = 256;
  const uint64_t target = sparse ? kSparseTargetWorkgroups : kTargetWorkgroups;
  while (sl < kMaxSplitLen && uint64_t(sl) * target < work) sl <<= 1;
  if (sparse && sl > kMaxSparseSplitLen) sl = kMaxSparseSplitLen;
  while (!sparse && sl > 256 && uint64_t(S) * ((span + sl - 1) / sl) * wpu < kMinWorkgroups) sl >>= 1;
  while (sl > 16 && sl / bs + 2 > max_pages) sl >>= 1;
  Plan p;
  p.split_len = sl;
  p.nsplit = uint32_t(span == 0 ? 1 : (span + sl - 1) / sl);
  const uint64_t units = uint64_t(S) * nkv * p.nsplit;
  uint64_t off = 0;
  p.off_ml = off;
  off = up256(off + units * G * 2 * sizeof(float));
  p.off_part = p.off_cnt = p.off_crec = p.off_vpart = p.off_order = 0;
  p.seg_cap = 0;
  p.segs = segs;
  p.vparts = 1;
  p.off_order = off;
  off = up256(off + uint64_t(S) * p.nsplit * sizeof(uint32_t));
  if (!sparse) {
    p.off_part = off;
    off = up256(off + units * G * hd * sizeof(float));
  } else {
    p.seg_cap = cand_segment_cap(sl, segs);
    p.off_cnt = off;
    off = up256(off + units * segs * sizeof(int32_t));
    p.off_crec = off;
    off = up256(off + units * segs * p.seg_cap * cand_record_words(G) * sizeof(uint32_t));
    // V-pass parts: as many as keep the launch within kVTargetWorkgroups and
    // every wave of the longest sequence with a segment of its own
    const uint64_t pairs = uint64_t(S) * nkv;
    while (p.vparts < kMaxVParts && pairs * p.vparts * 2 <= kVTargetWorkgroups &&
           p.vparts * 2 * KVQ_VWAVES <= p.nsplit * segs)
      p.vparts *= 2;
    if (p.vparts > 1) {
      p.off_vpart = off;
      off = up256(off + pairs * p.vparts * G * hd * sizeof(float));
    }
  }
  p.bytes = off;
  return p;
}

}  // namespace

const Codebooks& codebooks() {
  static Codebooks cb;
  static std::once_flag once;
  std::call_once(once, [] { cb = build_codebooks(); });
  return cb;
}

}  // namespace kvq

using namespace kvq;

extern "C" {

int kvq_pool_layout(int32_t k_format, int32_t v_format, uint32_t block_size, uint32_t num_kv_heads,
                    uint32_t head_dim, kvq_layout* out) {
  return layout_impl(k_format, v_format, block_size, num_kv_heads, head_dim, out);
}

int kvq_reshape_and_cache(const kvq_layout* layout, const void* key, const void* value, void* k_cache,
                          void* v_cache, const int64_t* slot_mapping, uint32_t num_tokens, uint32_t key_stride,
                          uint32_t value_stride, float k_scale, float v_scale, void* stream) {
  const int st = check_layout(layout);
  if (st != KVQ_OK) return st;
  if (num_tokens == 0) return KVQ_OK;
  const uint32_t nkv = layout->num_kv_heads, hd = layout->head_dim;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return KVQ_ERR_INVALID_ARG;
  if (uint64_t(num_tokens) * nkv * 2 >= (1ull << 31)) return KVQ_ERR_UNSUPPORTED;
  if (key_stride < nkv * hd || value_stride < nkv * hd) return KVQ_ERR_INVALID_ARG;
  if (key_stride % 8 || value_stride % 8) return KVQ_ERR_ALIGNMENT;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8))
    return KVQ_ERR_ALIGNMENT;
  if (layout->k_format == KVQ_FP8_E4M3 && !good_scale(k_scale)) return KVQ_ERR_INVALID_ARG;
  if (layout->v_format == KVQ_FP8_E4M3 && !good_scale(v_scale)) return KVQ_ERR_INVALID_ARG;
  WriteArgs a;
  std::memset(&a, 0, sizeof(a));
  a.key = static_cast<const uint16_t*>(key);
  a.value = static_cast<const uint16_t*>(value);
  a.k_cache = static_cast<uint8_t*>(k_cache);
  a.v_cache = static_cast<uint8_t*>(v_cache);
  a.slots = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_kv_heads = nkv;
  a.log2_bs = log2u(layout->block_size);
  a.key_stride = key_stride;
  a.value_stride = value_stride;
  a.k_format = layout->k_format;
  a.v_format = layout->v_format;
  a.k_stride = layout->k_block_stride_bytes;
  a.k_data = layout->k_data_section_bytes;
  a.v_stride = layout->v_block_stride_bytes;
  a.v_data = layout->v_data_section_bytes;
  a.k_scale = layout->k_format == KVQ_FP8_E4M3 ? k_scale : 1.0f;
  a.v_scale = layout->v_format == KVQ_FP8_E4M3 ? v_scale : 1.0f;
  a.wht_scale = float(1.0 / std::sqrt(double(hd)));
  a.cb = codebooks();
  return launch_write(int(hd), a, static_cast<hipStream_t>(stream)) == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}

}  // extern "C"

namespace kvq {
namespace {

// The dense decode path: the split kernel of the (K, V) pair, then the merge.
hipError_t launch_dense(const kvq_layout* layout, const DecodeArgs& a, uint32_t hd, uint32_t G, uint32_t nwg,
                        hipStream_t s) {
  const int vf = layout->v_format;
  hipError_t e = a.order ? launch_unit_order(a, s) : hipSuccess;
  if (e == hipSuccess) switch (layout->k_format) {
    case KVQ_BF16: e = launch_split_bf16(vf, int(hd), int(G), a, nwg, s); break;
    case KVQ_FP8_E4M3: e = launch_split_fp8(vf, int(hd), int(G), a, nwg, s); break;
    case KVQ_TURBO2: e = launch_split_turbo2(vf, int(hd), int(G), a, nwg, s); break;
    case KVQ_TURBO3: e = launch_split_turbo3(vf, int(hd), int(G), a, nwg, s); break;
    case KVQ_TURBO8: e = launch_split_turbo8(vf, int(hd), int(G), a, nwg, s); break;
    case KVQ_NVFP4: e = launch_split_nvfp4(vf, int(hd), int(G), a, nwg, s); break;
    default: e = launch_split_turbo4(vf, int(hd), int(G), a, nwg, s); break;
  }
  return e == hipSuccess ? launch_merge(layout->v_rotated != 0, int(hd), int(G), a, s) : e;
}

// Dense-path options: a sequence's splits share its span equally, and
// (KVQ_DENSE_ORDER) the split kernel takes its units longest first.
void dense_options(DecodeArgs& a, uint8_t* ws, const Plan& p) {
  a.eq_split = KVQ_EQ_SPLITS;
  if (KVQ_DENSE_ORDER) a.order = reinterpret_cast<uint32_t*>(ws + p.off_order);
}

// The fields of a decode call's arguments that come from the layout and the
// scales alone.
void fill_common(DecodeArgs& a, const kvq_layout* layout, float inv_sqrt_d, float k_scale, float v_scale) {
  a.log2_bs = log2u(layout->block_size);
  a.num_kv_heads = layout->num_kv_heads;
  a.k_stride = layout->k_block_stride_bytes;
  a.k_data = layout->k_data_section_bytes;
  a.v_stride = layout->v_block_stride_bytes;
  a.v_data = layout->v_data_section_bytes;
  const float log2e = 1.4426950408889634f;
  a.qk_scale = inv_sqrt_d * log2e * (layout->k_format == KVQ_FP8_E4M3 ? k_scale : 1.0f);
  a.v_scale = layout->v_format == KVQ_FP8_E4M3 ? v_scale : 1.0f;
  a.wht_scale = float(1.0 / std::sqrt(double(layout->head_dim)));
  a.cb = codebooks();
}

// kvq_paged_decode's checks, plan and launches, for both decode entry points.
int decode_impl(const kvq_layout* layout, const void* q, const void* k_cache, const void* v_cache,
                     float* out, const int32_t* block_tables, const int32_t* seq_lens,
                     uint32_t max_blocks_per_seq, uint32_t num_seqs, uint32_t num_q_heads, float inv_sqrt_d,
                     uint32_t q_stride, uint32_t sliding_window, float sparse_v_threshold, float k_scale,
                     float v_scale, void* workspace, size_t* workspace_bytes, void* stream) {
  const int st = check_layout(layout);
  if (st != KVQ_OK) return st;
  if (!workspace_bytes) return KVQ_ERR_INVALID_ARG;
  const uint32_t nkv = layout->num_kv_heads, hd = layout->head_dim;
  if (num_q_heads == 0 || num_q_heads % nkv) return KVQ_ERR_INVALID_ARG;
  const uint32_t G = num_q_heads / nkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVQ_ERR_UNSUPPORTED;
  if (!std::isfinite(inv_sqrt_d) || inv_sqrt_d <= 0.0f) return KVQ_ERR_INVALID_ARG;
  if (!std::isfinite(sparse_v_threshold) || sparse_v_threshold < 0.0f) return KVQ_ERR_INVALID_ARG;
  if (layout->k_format == KVQ_FP8_E4M3 && !good_scale(k_scale)) return KVQ_ERR_INVALID_ARG;
  if (layout->v_format == KVQ_FP8_E4M3 && !good_scale(v_scale)) return KVQ_ERR_INVALID_ARG;
  if (num_seqs && max_blocks_per_seq == 0) return KVQ_ERR_INVALID_ARG;
  if (q_stride < num_q_heads * hd) return KVQ_ERR_INVALID_ARG;
  if (q_stride % 8) return KVQ_ERR_ALIGNMENT;
  if (uint64_t(max_blocks_per_seq) * layout->block_size >= (1ull << 31)) return KVQ_ERR_UNSUPPORTED;
  const bool sparse = sparse_v_threshold > 0.0f;
  const uint32_t segs = score_waves(scores_on_mfma(layout->k_format, int(hd), int(G), layout->block_size));
  const Plan p = make_plan(num_seqs, nkv, G, hd, max_blocks_per_seq, layout->block_size, sliding_window, sparse,
                           dense_pages(layout, sparse), wg_per_unit(layout, G, sparse), segs);
  // grids of (unit, kv head) tiles, units padded to a multiple of the 8 XCDs
  const uint64_t nwg = (uint64_t(num_seqs) * p.nsplit + 7) / 8 * 8 * nkv;
  const uint64_t nwg_v = (uint64_t(num_seqs) + 7) / 8 * 8 * nkv * p.vparts;
  if (nwg >= (1ull << 31) || nwg_v >= (1ull << 31) || uint64_t(num_seqs) * num_q_heads >= (1ull << 31))
    return KVQ_ERR_UNSUPPORTED;
  if (!workspace) {
    *workspace_bytes = size_t(p.bytes);
    return KVQ_OK;
  }
  if (*workspace_bytes < p.bytes) return KVQ_ERR_WORKSPACE;
  if (num_seqs == 0) return KVQ_OK;
  if (!q || !k_cache || !v_cache || !out || !block_tables || !seq_lens) return KVQ_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_tables, 4) || !aligned(seq_lens, 4) || !aligned(workspace, 16))
    return KVQ_ERR_ALIGNMENT;

  DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint8_t*>(k_cache);
  a.v_cache = static_cast<const uint8_t*>(v_cache);
  a.out = out;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.ml = reinterpret_cast<float*>(ws + p.off_ml);
  if (!sparse) {
    a.part = reinterpret_cast<float*>(ws + p.off_part);
    dense_options(a, ws, p);
  } else {
    a.cnt = reinterpret_cast<int32_t*>(ws + p.off_cnt);
    a.crec = reinterpret_cast<uint32_t*>(ws + p.off_crec);
    if (p.vparts > 1) a.vpart = reinterpret_cast<float*>(ws + p.off_vpart);
    // Longest units first (a sorting launch ahead of the score kernel) where
    // lengths can differ: without a window.  With one, every sequence at least
    // as long as the window has the same span, and the extra launch (about 4 us)
    // costs more than it saves.
    if (KVQ_SCORE_ORDER && sliding_window == 0) {
      // launches of few units (the VALU form's workgroup holds them all)
      // order themselves in every workgroup instead of a sorting launch
      if (KVQ_SCORE_ORDER_INLINE && segs == score_waves(false) &&
          uint64_t(num_seqs) * p.nsplit <= uint64_t(score_waves(false)) * 64u)
        a.lpt_inline = 1u;
      else
        a.order = reinterpret_cast<uint32_t*>(ws + p.off_order);
    }
  }
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = nkv;
  a.log2_bs = log2u(layout->block_size);
  a.q_stride = q_stride;
  a.window = sliding_window;
  a.split_len = p.split_len;
  a.nsplit = p.nsplit;
  a.seg_cap = p.seg_cap;
  a.segs = p.segs;
  a.vparts = p.vparts;
  a.k_stride = layout->k_block_stride_bytes;
  a.k_data = layout->k_data_section_bytes;
  a.v_stride = layout->v_block_stride_bytes;
  a.v_data = layout->v_data_section_bytes;
  const float log2e = 1.4426950408889634f;
  a.qk_scale = inv_sqrt_d * log2e * (layout->k_format == KVQ_FP8_E4M3 ? k_scale : 1.0f);
  a.v_scale = layout->v_format == KVQ_FP8_E4M3 ? v_scale : 1.0f;
  a.thr = sparse_v_threshold;
  a.wht_scale = float(1.0 / std::sqrt(double(hd)));
  a.cb = codebooks();

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int kf = layout->k_format, vf = layout->v_format;
  hipError_t e;
  if (!sparse) {
    e = launch_dense(layout, a, hd, G, uint32_t(nwg), s);
  } else {
    e = a.order ? launch_unit_order(a, s) : hipSuccess;
    if (e == hipSuccess) switch (kf) {
      case KVQ_BF16: e = launch_scores_bf16(int(hd), int(G), a, uint32_t(nwg), s); break;
      case KVQ_FP8_E4M3: e = launch_scores_fp8(int(hd), int(G), a, uint32_t(nwg), s); break;
      case KVQ_TURBO2: e = launch_scores_turbo2(int(hd), int(G), a, uint32_t(nwg), s); break;
      case KVQ_TURBO3: e = launch_scores_turbo3(int(hd), int(G), a, uint32_t(nwg), s); break;
      case KVQ_TURBO8: e = launch_scores_turbo8(int(hd), int(G), a, uint32_t(nwg), s); break;
      case KVQ_NVFP4: e = launch_scores_nvfp4(int(hd), int(G), a, uint32_t(nwg), s); break;
      default: e = launch_scores_turbo4(int(hd), int(G), a, uint32_t(nwg), s); break;
    }
    if (e == hipSuccess) e = launch_sparse_v(vf, int(hd), int(G), a, uint32_t(nwg_v), s);
    if (e == hipSuccess && p.vparts > 1) e = launch_sparse_v_merge(layout->v_rotated != 0, int(hd), int(G), a, s);
  }
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}

// The allocation-free decode's scratch: one copy per GPU, held until the
// process ends.  In host code the array's name is only a stand-in; the
// device address each GPU holds it at comes from hipGetSymbolAddress.
constexpr size_t kScratchBytes = size_t(64) << 20;
std::mutex g_scratch_mu;
void* g_scratch[256] = {};  // per device ordinal

}  // namespace
}  // namespace kvq

static __device__ __align__(256) uint8_t scratch[kvq::kScratchBytes];

namespace kvq {
namespace {

// The scratch address on the device `stream` belongs to (that device must be
// the current one); looked up once per device.
int scratch_for(void* stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return KVQ_ERR_LAUNCH;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) return KVQ_ERR_INVALID_ARG;
    if (sdev != dev) return KVQ_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVQ_ERR_LAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return KVQ_OK;
}

}  // namespace
}  // namespace kvq

extern "C" {

int kvq_paged_decode(const kvq_layout* layout, const void* q, const void* k_cache, const void* v_cache,
                     float* out, const int32_t* block_tables, const int32_t* seq_lens,
                     uint32_t max_blocks_per_seq, uint32_t num_seqs, uint32_t num_q_heads, float inv_sqrt_d,
                     uint32_t q_stride, uint32_t sliding_window, float sparse_v_threshold, float k_scale,
                     float v_scale, void* workspace, size_t* workspace_bytes, void* stream) {
  return decode_impl(layout, q, k_cache, v_cache, out, block_tables, seq_lens, max_blocks_per_seq, num_seqs,
                     num_q_heads, inv_sqrt_d, q_stride, sliding_window, sparse_v_threshold, k_scale, v_scale,
                     workspace, workspace_bytes, stream);
}

int kvq_paged_decode_noalloc(const kvq_layout* layout, const void* q, const void* k_cache, const void* v_cache,
                             float* out, const int32_t* block_tables, const int32_t* seq_lens,
                             uint32_t max_blocks_per_seq, uint32_t num_seqs, uint32_t num_q_heads, float inv_sqrt_d,
                             uint32_t q_stride, uint32_t sliding_window, float sparse_v_threshold, float k_scale,
                             float v_scale, void* stream) {
  size_t need = 0;
  int st = decode_impl(layout, q, k_cache, v_cache, out, block_tables, seq_lens, max_blocks_per_seq, num_seqs,
                       num_q_heads, inv_sqrt_d, q_stride, sliding_window, sparse_v_threshold, k_scale, v_scale,
                       nullptr, &need, stream);
  if (st != KVQ_OK) return st;
  if (need > kScratchBytes) return KVQ_ERR_WORKSPACE;
  if (num_seqs == 0) return KVQ_OK;
  void* ws = nullptr;
  st = scratch_for(stream, &ws);
  if (st != KVQ_OK) return st;
  size_t have = kScratchBytes;
  return decode_impl(layout, q, k_cache, v_cache, out, block_tables, seq_lens, max_blocks_per_seq, num_seqs,
                     num_q_heads, inv_sqrt_d, q_stride, sliding_window, sparse_v_threshold, k_scale, v_scale, ws,
                     &have, stream);
}

}  // extern "C"

namespace kvq {
namespace {

// Chunked prefill where the tile kernel does not apply (block_size < 4,
// where a thread's four keys would span pages): every query runs as its own
// decode row -- its sequence's block table, the length of its causal span
// (position + 1), its own query and output row -- through the dense decode
// kernels.  Each query then reads its keys and values on its own, so this
// path trades the tiles' reuse for coverage.  The workspace holds the rows'
// map and lengths, then the dense decode workspace of num_seqs *
// max_query_len rows.
int prefill_as_decode(const kvq_layout* layout, const void* q, const void* k_cache, const void* v_cache, float* out,
                      const int32_t* block_tables, const int32_t* seq_lens, const int32_t* query_start,
                      uint32_t max_blocks_per_seq, uint32_t num_seqs, uint32_t num_q_heads, uint32_t max_query_len,
                      float inv_sqrt_d, uint32_t q_stride, uint32_t sliding_window, float k_scale, float v_scale,
                      void* workspace, size_t* workspace_bytes, void* stream) {
  const uint32_t nkv = layout->num_kv_heads, hd = layout->head_dim, G = num_q_heads / nkv;
  const uint64_t rows = uint64_t(num_seqs) * max_query_len;
  if (rows >= (1ull << 31) || rows * num_q_heads >= (1ull << 31)) return KVQ_ERR_UNSUPPORTED;
  const Plan p = make_plan(uint32_t(rows), nkv, G, hd, max_blocks_per_seq, layout->block_size, sliding_window, false,
                           dense_pages(layout, false), wg_per_unit(layout, G, false), 0);
  const uint64_t nwg = (rows * p.nsplit + 7) / 8 * 8 * nkv;
  if (nwg >= (1ull << 31)) return KVQ_ERR_UNSUPPORTED;
  const uint64_t off_vrow = 0, off_vlen = up256(rows * 2 * sizeof(int32_t));
  const uint64_t base = up256(off_vlen + rows * sizeof(int32_t));
  const uint64_t bytes = base + p.bytes;
  if (!workspace) {
    *workspace_bytes = size_t(bytes);
    return KVQ_OK;
  }
  if (*workspace_bytes < bytes) return KVQ_ERR_WORKSPACE;
  if (num_seqs == 0) return KVQ_OK;
  if (!q || !k_cache || !v_cache || !out || !block_tables || !seq_lens || !query_start) return KVQ_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_tables, 4) || !aligned(seq_lens, 4) || !aligned(query_start, 4) || !aligned(workspace, 16))
    return KVQ_ERR_ALIGNMENT;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* vrow = reinterpret_cast<int32_t*>(ws + off_vrow);
  int32_t* vlen = reinterpret_cast<int32_t*>(ws + off_vlen);
  DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint8_t*>(k_cache);
  a.v_cache = static_cast<const uint8_t*>(v_cache);
  a.out = out;
  a.block_tables = block_tables;
  a.seq_lens = vlen;
  a.vrow = vrow;
  a.ml = reinterpret_cast<float*>(ws + base + p.off_ml);
  a.part = reinterpret_cast<float*>(ws + base + p.off_part);
  dense_options(a, ws + base, p);
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = uint32_t(rows);
  a.num_q_heads = num_q_heads;
  a.q_stride = q_stride;
  a.window = sliding_window;
  a.split_len = p.split_len;
  a.nsplit = p.nsplit;
  fill_common(a, layout, inv_sqrt_d, k_scale, v_scale);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_prefill_rows(query_start, seq_lens, num_seqs, max_query_len, vrow, vlen, s);
  if (e == hipSuccess) e = launch_dense(layout, a, hd, G, uint32_t(nwg), s);
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}

// Chunked prefill on the tile kernel (block_size >= 4): a workgroup per
// (sequence, kv head, tile of queries) walks the tile's key range and writes
// finished rows.  A grid too small to fill the GPU (few sequences and tiles,
// long key ranges) splits the range instead: each split writes its rows'
// partials and a merge kernel combines them.  Without splits nothing goes
// through the workspace, which the call still takes (256 bytes) so that a
// null workspace keeps meaning "report the size".
int prefill_tiles(const kvq_layout* layout, const void* q, const void* k_cache, const void* v_cache, float* out,
                  const int32_t* block_tables, const int32_t* seq_lens, const int32_t* query_start,
                  uint32_t max_blocks_per_seq, uint32_t num_seqs, uint32_t num_q_heads, uint32_t max_query_len,
                  float inv_sqrt_d, uint32_t q_stride, uint32_t sliding_window, float k_scale, float v_scale,
                  void* workspace, size_t* workspace_bytes, void* stream) {
  const uint32_t nkv = layout->num_kv_heads, hd = layout->head_dim, G = num_q_heads / nkv;
  const uint32_t rows = uint32_t(prefill_tile_rows(layout->k_format, int(hd)));
  const uint32_t qt = rows / G, nk = 8192 / hd;  // queries per tile, keys per chunk
  const uint64_t ntiles = (uint64_t(max_query_len) + qt - 1) / qt;
  // chunks a tile's key range can span: the table's reach (or the window
  // plus the tile), aligned to chunks
  uint64_t span = uint64_t(max_blocks_per_seq) * layout->block_size;
  if (sliding_window && sliding_window + qt - 1 < span) span = sliding_window + qt - 1;
  const uint64_t nch = (span + nk - 1) / nk + 1;
  const uint64_t base = uint64_t(num_seqs) * nkv * ntiles;
  uint64_t nsplit = 1, split_len = 0;
  if (base < kTilePrefillWorkgroups) {
    nsplit = std::min<uint64_t>((kTilePrefillWorkgroups + base - 1) / base, nch / kTileSplitChunks);
    if (nsplit > 1) {
      const uint64_t cps = (nch + nsplit - 1) / nsplit;
      split_len = cps * nk;
      nsplit = (nch + cps - 1) / cps;
    } else {
      nsplit = 1;
    }
  }
  const uint64_t nwg = (base * nsplit / ntiles + 7) / 8 * 8 * ntiles;
  const uint64_t prow = base * nsplit * rows;  // partial rows
  const uint64_t units = base / ntiles * nsplit;  // (sequence, kv head, split)
  // the units' order, then (with splits) the partial rows' statistics and outputs
  const uint64_t off_order = 0, off_ml = up256(units * sizeof(uint32_t));
  const uint64_t off_part = up256(off_ml + prow * 2 * sizeof(float));
  const uint64_t bytes = nsplit > 1 ? up256(off_part + prow * hd * sizeof(float)) : off_ml;
  if (nwg >= (1ull << 31) || base * nsplit * rows / 4 >= (1ull << 31)) return KVQ_ERR_UNSUPPORTED;
  if (!workspace) {
    *workspace_bytes = size_t(bytes);
    return KVQ_OK;
  }
  if (*workspace_bytes < bytes) return KVQ_ERR_WORKSPACE;
  if (num_seqs == 0) return KVQ_OK;
  if (!q || !k_cache || !v_cache || !out || !block_tables || !seq_lens || !query_start) return KVQ_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_tables, 4) || !aligned(seq_lens, 4) || !aligned(query_start, 4) || !aligned(workspace, 16))
    return KVQ_ERR_ALIGNMENT;
  DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint8_t*>(k_cache);
  a.v_cache = static_cast<const uint8_t*>(v_cache);
  a.out = out;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.query_start = query_start;
  if (nsplit > 1) {
    a.ml = reinterpret_cast<float*>(ws + off_ml);
    a.part = reinterpret_cast<float*>(ws + off_part);
  }
  if (KVQ_PREFILL_ORDER) a.order = reinterpret_cast<uint32_t*>(ws + off_order);
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.q_stride = q_stride;
  a.window = sliding_window;
  a.ntiles = uint32_t(ntiles);
  a.qt = qt;
  a.nsplit = uint32_t(nsplit);
  a.split_len = uint32_t(split_len);
  fill_common(a, layout, inv_sqrt_d, k_scale, v_scale);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // buckets of the unit sort: 256 over the longest key range
  const int width = int(std::max<uint64_t>(16, (nch * nk + 255) / 256));
  hipError_t e = a.order ? launch_unit_order(a, st, 1, width) : hipSuccess;
  if (e == hipSuccess)
    e = launch_prefill_tiles(layout->k_format, layout->v_format, int(hd), int(G), a, uint32_t(nwg), st);
  if (e == hipSuccess && nsplit > 1) e = launch_prefill_tile_merge(layout->v_rotated != 0, int(hd), int(G), a, st);
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}

}  // namespace
}  // namespace kvq

extern "C" {

int kvq_paged_prefill(const kvq_layout* layout, const void* q, const void* k_cache, const void* v_cache, float* out,
                      const int32_t* block_tables, const int32_t* seq_lens, const int32_t* query_start,
                      uint32_t max_blocks_per_seq, uint32_t num_seqs, uint32_t num_q_heads, uint32_t max_query_len,
                      float inv_sqrt_d, uint32_t q_stride, uint32_t sliding_window, float k_scale, float v_scale,
                      void* workspace, size_t* workspace_bytes, void* stream) {
  const int st = check_layout(layout);
  if (st != KVQ_OK) return st;
  if (!workspace_bytes) return KVQ_ERR_INVALID_ARG;
  const uint32_t nkv = layout->num_kv_heads, hd = layout->head_dim, bs = layout->block_size;
  if (num_q_heads == 0 || num_q_heads % nkv) return KVQ_ERR_INVALID_ARG;
  const uint32_t G = num_q_heads / nkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVQ_ERR_UNSUPPORTED;
  if (!std::isfinite(inv_sqrt_d) || inv_sqrt_d <= 0.0f) return KVQ_ERR_INVALID_ARG;
  if (layout->k_format == KVQ_FP8_E4M3 && !good_scale(k_scale)) return KVQ_ERR_INVALID_ARG;
  if (layout->v_format == KVQ_FP8_E4M3 && !good_scale(v_scale)) return KVQ_ERR_INVALID_ARG;
  if (num_seqs && (max_blocks_per_seq == 0 || max_query_len == 0)) return KVQ_ERR_INVALID_ARG;
  if (q_stride < num_q_heads * hd) return KVQ_ERR_INVALID_ARG;
  if (q_stride % 8) return KVQ_ERR_ALIGNMENT;
  if (uint64_t(max_blocks_per_seq) * bs >= (1ull << 31)) return KVQ_ERR_UNSUPPORTED;
  if (KVQ_PREFILL_TILES && bs >= 4)
    return prefill_tiles(layout, q, k_cache, v_cache, out, block_tables, seq_lens, query_start, max_blocks_per_seq,
                         num_seqs, num_q_heads, max_query_len, inv_sqrt_d, q_stride, sliding_window, k_scale,
                         v_scale, workspace, workspace_bytes, stream);
  return prefill_as_decode(layout, q, k_cache, v_cache, out, block_tables, seq_lens, query_start,
                           max_blocks_per_seq, num_seqs, num_q_heads, max_query_len, inv_sqrt_d, q_stride,
                           sliding_window, k_scale, v_scale, workspace, workspace_bytes, stream);
}

int kvq_check_slots(const kvq_layout* layout, const int64_t* slot_mapping, uint32_t num_tokens, uint64_t num_blocks,
                    uint32_t* first_bad) {
  const int st = check_layout(layout);
  if (st != KVQ_OK) return st;
  if (num_tokens && !slot_mapping) return KVQ_ERR_INVALID_ARG;
  const uint64_t nslots = num_blocks * layout->block_size;
  std::vector<std::pair<int64_t, uint32_t>> used;
  used.reserve(num_tokens);
  for (uint32_t t = 0; t < num_tokens; ++t) {
    const int64_t s = slot_mapping[t];
    if (s < 0) continue;
    if (uint64_t(s) >= nslots) {
      if (first_bad) *first_bad = t;
      return KVQ_ERR_INVALID_ARG;
    }
    used.emplace_back(s, t);
  }
  std::sort(used.begin(), used.end());
  uint32_t bad = UINT32_MAX;
  for (size_t i = 1; i < used.size(); ++i)  // the later token of a repeated slot
    if (used[i].first == used[i - 1].first) bad = std::min(bad, std::max(used[i].second, used[i - 1].second));
  if (bad != UINT32_MAX) {
    if (first_bad) *first_bad = bad;
    return KVQ_ERR_INVALID_ARG;
  }
  return KVQ_OK;
}

int kvq_check_tables(const kvq_layout* layout, const int32_t* block_tables, const int32_t* seq_lens,
                     const int32_t* query_start, uint32_t max_blocks_per_seq, uint32_t num_seqs,
                     uint32_t sliding_window, uint64_t num_blocks, uint32_t* first_bad) {
  const int st = check_layout(layout);
  if (st != KVQ_OK) return st;
  if (num_seqs && (!block_tables || !seq_lens)) return KVQ_ERR_INVALID_ARG;
  const int64_t bs = layout->block_size, cap = int64_t(max_blocks_per_seq) * bs, W = sliding_window;
  auto fail = [&](uint32_t s) {
    if (first_bad) *first_bad = s;
    return KVQ_ERR_INVALID_ARG;
  };
  if (query_start && num_seqs && query_start[0] != 0) return fail(0);
  for (uint32_t s = 0; s < num_seqs; ++s) {
    const int64_t L = seq_lens[s];
    if (L < 0 || L > cap) return fail(s);
    int64_t j0 = W > 0 ? std::max<int64_t>(0, L - W) : 0;  // decode's window start
    if (query_start) {
      const int64_t C = int64_t(query_start[s + 1]) - query_start[s];
      if (C < 0 || C > L) return fail(s);
      if (C == 0) continue;                                  // no query reads the table
      j0 = W > 0 ? std::max<int64_t>(0, L - C + 1 - W) : 0;  // the first query's window start
    }
    const int32_t* row = block_tables + uint64_t(s) * max_blocks_per_seq;
    for (int64_t i = j0 / bs; i < (L + bs - 1) / bs; ++i)
      if (row[i] < 0 || uint64_t(row[i]) >= num_blocks) return fail(s);
  }
  return KVQ_OK;
}

int kvq_codebook(int32_t format, float* centroids, float* thresholds, float* inv_cmax, uint32_t* levels) {
  if (!has_codebook(format) || !centroids || !thresholds || !inv_cmax || !levels)
    return KVQ_ERR_INVALID_ARG;
  const Codebooks& cb = codebooks();
  const int b = format;
  const int L = 1 << b;
  for (int k = 0; k < 16; ++k) {
    centroids[k] = k < L ? cb.centroid[b - 2][k] : 0.0f;
    thresholds[k] = k < L ? cb.threshold[b - 2][k] : 0.0f;
  }
  *inv_cmax = cb.inv_cmax[b - 2];
  *levels = uint32_t(L);
  return KVQ_OK;
}

const char* kvq_status_string(int status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported size or format";
    case KVQ_ERR_ALIGNMENT: return "misaligned pointer or stride";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_LAUNCH: return "kernel launch failed";
    case KVQ_ERR_EXHAUSTED: return "no free block left";
    case KVQ_ERR_HOST_MEMORY: return "host memory exhausted";
    default: return "unknown status";
  }
}

}  // extern "C"
