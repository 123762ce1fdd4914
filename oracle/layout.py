"""Pool layout: bytes per block and where codes and scales sit.

"spark_runtime/kv_cache.rs", ``KvCacheConfig::block_bytes_dims`` with
e = block_size * num_kv_heads * head_dim elements per block per side:
  bf16   2e            fp8  e
  turbo4 e/2 + e/16    turbo3 3e/8 + e/16    turbo2 e/4 + e/16
(codes, then one FP8 scale byte per group of 16 elements), and the
``turbo*_data_bytes`` / ``turbo*_scale_bytes`` split.  ``KvCacheDtype::Turbo8``
with ``turbo8_data_bytes`` / ``turbo8_scale_bytes``: one E4M3 byte per element,
then one BF16 scale (2 bytes) per group of 16: e + 2e/16.  ``KvCacheDtype::Nvfp4``
with ``nvfp4_data_bytes`` / ``nvfp4_scale_bytes``: turbo4's byte layout (E2M1
nibbles, then one FP8 scale byte per group of 16), e/2 + e/16.
"metrale_model_layers/layers/ops/kv_cache_bf16k_turbov.rs", module
invariants: element order ``[num_blocks, block_size, num_kv_heads,
head_dim]``; a V block is its code section followed by its scales; K and V
pools have separate block strides in bytes.

Readings:
  * The same element order holds for every format and both sides; the
    flat element index inside a block is e' = (offset * Hkv + head) * hd + d.
  * Codes occupy bits [e'*b, e'*b + b) of the block's code section read as
    a little-endian bit stream (low bits first): turbo4 puts element 2k in
    the low nibble of byte k, turbo2 packs elements 4k..4k+3 into byte k
    from the low bits up, turbo3 packs each 8 elements into a 24-bit
    little-endian word, element j at bits 3j.
  * The scale of group g = e' / 16 is byte g of the scale section, which
    starts right after the code section (``data_section_bytes``); turbo8's
    BF16 scale of group g is the little-endian 2-byte word at 2g.
  * NVFP4 nibbles pack as turbo4's codes do (element 2k in the low nibble of
    byte k); ``is_wht_rotated`` leaves NVFP4 out, so it is not rotated.
  * The block stride is the block's byte size rounded up to 16 bytes.
"""
from __future__ import annotations

import dataclasses

BITS = {"bf16": 16, "fp8": 8, "turbo2": 2, "turbo3": 3, "turbo4": 4, "turbo8": 8, "nvfp4": 4}
TURBO = ("turbo2", "turbo3", "turbo4")     # Lloyd-Max codes, one E4M3 scale byte per group
ROTATED = TURBO + ("turbo8",)              # turbo8: E4M3 values, one BF16 scale per group
BYTE_SCALED = TURBO + ("nvfp4",)           # one E4M3 scale byte per group (nvfp4: E2M1 values)
GROUP = 16


def is_rotated(fmt: str) -> bool:
    """``is_wht_rotated``: true for the turbo sides."""
    return fmt in ROTATED


@dataclasses.dataclass(frozen=True)
class Side:
    fmt: str
    block_size: int
    num_kv_heads: int
    head_dim: int
    data_section_bytes: int
    scale_bytes: int
    block_stride_bytes: int

    @property
    def bits(self) -> int:
        return BITS[self.fmt]

    @property
    def row_bytes(self) -> int:
        """Code bytes of one (position, kv head) row."""
        return self.head_dim * self.bits // 8

    @property
    def row_scales(self) -> int:
        """Scale bytes of one (position, kv head) row."""
        if self.fmt in BYTE_SCALED:
            return self.head_dim // GROUP
        return 2 * self.head_dim // GROUP if self.fmt == "turbo8" else 0


def side_layout(fmt: str, block_size: int, num_kv_heads: int, head_dim: int) -> Side:
    e = block_size * num_kv_heads * head_dim
    if fmt == "bf16":
        data, scales = 2 * e, 0
    elif fmt == "fp8":
        data, scales = e, 0
    elif fmt in ("turbo4", "nvfp4"):
        data, scales = e // 2, e // GROUP
    elif fmt == "turbo3":
        data, scales = e * 3 // 8, e // GROUP
    elif fmt == "turbo2":
        data, scales = e // 4, e // GROUP
    elif fmt == "turbo8":
        data, scales = e, 2 * (e // GROUP)
    else:
        raise ValueError(fmt)
    stride = (data + scales + 15) // 16 * 16
    return Side(fmt, block_size, num_kv_heads, head_dim, data, scales, stride)


def pool_layout(k_fmt: str, v_fmt: str, block_size: int, num_kv_heads: int, head_dim: int):
    return (side_layout(k_fmt, block_size, num_kv_heads, head_dim),
            side_layout(v_fmt, block_size, num_kv_heads, head_dim))
