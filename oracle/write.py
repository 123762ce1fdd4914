"""Cache write: quantize new K/V rows and place them in the paged pools.

"metrale_model_layers/layers/ops/kv_cache_bf16k_turbov.rs",
``reshape_and_cache_bf16k_turbo{2,3,4}v``: each token's K and V
(``[num_tokens, num_kv_heads, head_dim]`` with row strides ``key_stride`` /
``value_stride``) go to the slot ``slot_mapping[t]`` of the pools.
"spark_runtime/kv_cache.rs": bf16 is a raw copy, fp8 is E4M3 with a
per-tensor scale, turbo sides are rotated (``wht_bf16_inplace``) before
quantizing to Lloyd-Max codes with one FP8 scale per 16 elements.

Steps for one row x (bf16, head_dim values), by format (readings in
brackets, the pages are silent on them):
  bf16   the 2-byte patterns, little-endian.
  fp8    v = RN32(x / scale) [IEEE division], byte = E4M3(v) [clamp to
         +-448, nearest, ties to even].
  turbo  y = x in fp32; y = WHT(y) [ascending-stride fp32 butterflies, then
         * RN32(1/sqrt(d))]; y = RNE_bf16(y) [the in-place bf16 rotation];
         per group of 16: a = max|y|, s = RN32(a * inv_cmax) [absmax /
         largest centroid, as NVFP4 does, only the codebook differs],
         sigma = E4M3(s), s_q = value(sigma); code = number of thresholds
         k = 1..L-1 with y >= RN32(s_q * t_k) [nearest centroid, ties go
         up]; codes packed low bits first; sigma stored in the scale
         section.
  turbo8 ("WHT + FP8 E4M3" data, "per-group BF16 scales",
         ``KvCacheDtype::Turbo8`` and ``turbo8_scale_bytes``): y as for
         turbo; per group of 16: a = max|y|, s = RN32(a * RN32(1/448))
         [absmax / largest E4M3 value, the same rule with 448 for the
         largest centroid], sigma = RNE_bf16(s), s_q = value(sigma); byte =
         E4M3(RN32(y / s_q)) [IEEE division and the fp8 side's E4M3
         rounding; a zero scale (an all-zero group) gives zero bytes];
         sigma stored as a little-endian 2-byte word.
  nvfp4  ("E2M1 packed nibbles" with "per-group FP8 scale", turbo4's byte
         layout, not rotated): per group of 16 of x itself: a = max|x|,
         s = RN32(a * RN32(1/6)) [absmax / largest E2M1 value, the turbo
         rule with 6 for the largest centroid], sigma = E4M3(s), s_q =
         value(sigma); nibble = E2M1(RN32(x / s_q)) [IEEE division as for
         fp8; saturate to +-6, nearest, ties to the even mantissa, sign
         kept; a zero scale gives zero nibbles]; nibbles packed as turbo4's
         codes, sigma stored in the scale section.
Tokens whose slot is negative write nothing [the slot sentinel].
"""
from __future__ import annotations

import numpy as np

from . import codecs, codebook, wht
from .layout import BITS, GROUP, TURBO, Side

E4M3_INV_MAX = np.float32(1.0 / codecs.E4M3_MAX)   # RN32(1/448)
E2M1_INV_MAX = np.float32(1.0 / codecs.E2M1_MAX)   # RN32(1/6)

_TABLES = {}


def tables(fmt: str):
    bits = BITS[fmt]
    if bits not in _TABLES:
        _TABLES[bits] = codebook.turbo_tables(bits)
    return _TABLES[bits]


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """[N, n] small ints -> [N, n*bits/8] bytes, little-endian bit stream."""
    n = codes.shape[-1]
    shifts = np.arange(bits, dtype=np.uint8)
    bitarr = ((codes[..., None].astype(np.uint8) >> shifts) & 1).reshape(codes.shape[0], n * bits)
    return np.packbits(bitarr, axis=-1, bitorder="little")


def unpack_codes(data: np.ndarray, bits: int, n: int) -> np.ndarray:
    """Inverse of pack_codes: [N, n*bits/8] bytes -> [N, n] codes."""
    bitarr = np.unpackbits(data, axis=-1, bitorder="little")[..., : n * bits]
    bitarr = bitarr.reshape(data.shape[0], n, bits).astype(np.uint8)
    weights = (1 << np.arange(bits)).astype(np.uint8)
    return (bitarr * weights).sum(axis=-1).astype(np.uint8)


def turbo_quantize(x_f32: np.ndarray, fmt: str):
    """Rotated rows -> (codes [N, hd] uint8, scale bytes [N, hd/16] uint8).

    `x_f32` holds the bf16 input values as fp32, shape [N, hd].
    """
    t = tables(fmt)
    N, hd = x_f32.shape
    y = wht.wht_f32(x_f32)                           # butterflies, then * r_d
    y = codecs.bf16_round(y)                         # back to bf16 values
    yg = y.reshape(N, hd // GROUP, GROUP)
    a = np.max(np.abs(yg), axis=-1)                  # exact
    s = (a * t["inv_cmax"]).astype(np.float32)       # one fp32 multiply
    sigma = codecs.e4m3_encode(s)
    sq = codecs.e4m3_decode(sigma)                   # fp32
    thr = (sq[..., None] * t["thresholds"][1:]).astype(np.float32)   # [N, G, L-1]
    codes = np.sum(yg[..., None] >= thr[:, :, None, :], axis=-1).astype(np.uint8)
    return codes.reshape(N, hd), sigma


def turbo8_quantize(x_f32: np.ndarray):
    """Rotated rows -> (E4M3 bytes [N, hd] uint8, BF16 scale patterns [N, hd/16] uint16)."""
    N, hd = x_f32.shape
    y = codecs.bf16_round(wht.wht_f32(x_f32))
    yg = y.reshape(N, hd // GROUP, GROUP)
    a = np.max(np.abs(yg), axis=-1)
    s = (a * E4M3_INV_MAX).astype(np.float32)
    sigma = codecs.bf16_round_bits(s)
    sq = codecs.bf16_bits_to_f32(sigma)
    v = np.zeros_like(yg)
    np.divide(yg, sq[..., None], out=v, where=sq[..., None] > 0)
    return codecs.e4m3_encode(v.astype(np.float32)).reshape(N, hd), sigma


def nvfp4_quantize(x_f32: np.ndarray):
    """Unrotated rows -> (E2M1 nibbles [N, hd] uint8, E4M3 scale bytes [N, hd/16] uint8)."""
    N, hd = x_f32.shape
    xg = x_f32.reshape(N, hd // GROUP, GROUP)
    a = np.max(np.abs(xg), axis=-1)
    s = (a * E2M1_INV_MAX).astype(np.float32)
    sigma = codecs.e4m3_encode(s)
    sq = codecs.e4m3_decode(sigma)
    v = np.zeros_like(xg)
    np.divide(xg, sq[..., None], out=v, where=sq[..., None] > 0)
    return codecs.e2m1_encode(v.astype(np.float32)).reshape(N, hd), sigma


def quantize_rows(x_bits: np.ndarray, fmt: str, scale: float = 1.0):
    """bf16 rows (uint16 [N, hd]) -> (code bytes [N, row_bytes], scale bytes [N, row_scales])."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    N, hd = x_bits.shape
    if fmt == "bf16":
        return x_bits.view(np.uint8).reshape(N, 2 * hd).copy(), np.zeros((N, 0), np.uint8)
    x = codecs.bf16_bits_to_f32(x_bits)
    if fmt == "fp8":
        v = (x / np.float32(scale)).astype(np.float32)
        return codecs.e4m3_encode(v), np.zeros((N, 0), np.uint8)
    if fmt in TURBO:
        codes, sigma = turbo_quantize(x, fmt)
        return pack_codes(codes, BITS[fmt]), sigma
    if fmt == "nvfp4":
        codes, sigma = nvfp4_quantize(x)
        return pack_codes(codes, 4), sigma
    if fmt == "turbo8":
        data, sigma = turbo8_quantize(x)
        return data, np.ascontiguousarray(sigma.astype("<u2")).view(np.uint8).reshape(N, -1)
    raise ValueError(fmt)


def row_addresses(side: Side, slots: np.ndarray, head: np.ndarray):
    """Byte offsets (codes, scales) of row (slot, head) inside the pool."""
    bs, nkv = side.block_size, side.num_kv_heads
    blk = slots // bs
    off = slots % bs
    row = off * nkv + head
    base = blk * side.block_stride_bytes
    return base + row * side.row_bytes, base + side.data_section_bytes + row * side.row_scales


def write_side(pool: np.ndarray, side: Side, x_bits: np.ndarray, slots: np.ndarray,
               scale: float = 1.0) -> None:
    """Write rows x_bits [T, Hkv, hd] (bf16 bits) to `pool` (uint8, flat) at `slots`."""
    T, nkv, hd = x_bits.shape
    keep = slots >= 0
    if not keep.any():
        return
    x = x_bits[keep].reshape(-1, hd)
    sl = np.repeat(slots[keep].astype(np.int64), nkv)
    hh = np.tile(np.arange(nkv, dtype=np.int64), int(keep.sum()))
    data, sc = quantize_rows(x, side.fmt, scale)
    caddr, saddr = row_addresses(side, sl, hh)
    rb = side.row_bytes
    pool[(caddr[:, None] + np.arange(rb)).ravel()] = data.ravel()
    if side.row_scales:
        pool[(saddr[:, None] + np.arange(side.row_scales)).ravel()] = sc.ravel()


def reshape_and_cache(k_side: Side, v_side: Side, key_bits: np.ndarray, value_bits: np.ndarray,
                      k_pool: np.ndarray, v_pool: np.ndarray, slot_mapping: np.ndarray,
                      k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Both sides of one write call (key/value: uint16 [T, Hkv, hd])."""
    slots = np.asarray(slot_mapping, dtype=np.int64)
    write_side(k_pool, k_side, key_bits, slots, k_scale)
    write_side(v_pool, v_side, value_bits, slots, v_scale)
