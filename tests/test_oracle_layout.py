"""Pool layout pinned to the pages' byte-size statements."""
import json
import os

import pytest

from oracle import layout

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_sizes.json")))


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "turbo2", "turbo3", "turbo4", "turbo8", "nvfp4"])
@pytest.mark.parametrize("bs,nkv,hd", [(16, 8, 128), (16, 2, 64), (16, 4, 256), (32, 8, 128), (1, 1, 64)])
def test_block_bytes_closed_form(fmt, bs, nkv, hd):
    s = layout.side_layout(fmt, bs, nkv, hd)
    e = bs * nkv * hd
    # block_bytes_dims arms, evaluated by hand
    # (turbo8: turbo8_data_bytes = e, turbo8_scale_bytes = 2 bytes per group of 16;
    # nvfp4 shares the turbo4 arm: nibbles plus one scale byte per group of 16)
    expect = {"bf16": e * 2, "fp8": e, "turbo4": e // 2 + e // 16, "nvfp4": e // 2 + e // 16,
              "turbo3": e * 3 // 8 + e // 16, "turbo2": e // 4 + e // 16, "turbo8": e + 2 * (e // 16)}[fmt]
    assert s.data_section_bytes + s.scale_bytes == expect
    assert s.block_stride_bytes % 16 == 0 and 0 <= s.block_stride_bytes - expect < 16


def test_bits_per_element_statements():
    e = 16 * 8 * 128
    bpe = {f: 8 * (layout.side_layout(f, 16, 8, 128).data_section_bytes
                   + layout.side_layout(f, 16, 8, 128).scale_bytes) / e for f in layout.BITS}
    b = GOLD["bits_per_element"]
    assert bpe["bf16"] == b["bf16"]["value"]
    assert bpe["fp8"] == b["fp8"]["value"]
    assert bpe["turbo4"] == b["turbo4"]["value"]
    assert bpe["turbo2"] == b["turbo2_v"]["value"]
    r = GOLD["ratios"]
    assert 16 / bpe["turbo2"] == r["turbo2_compression_vs_bf16"]["value"]
    assert abs((1 - bpe["turbo3"] / bpe["turbo4"]) - r["turbo3_smaller_than_turbo4"]["value"]) \
        < r["turbo3_smaller_than_turbo4"]["tolerance"]


def test_workload_strides():
    # the decode workloads' pools (K, V): stride and code-section bytes
    cases = [(("bf16", "bf16", 16, 2, 64), (4096, 4096), (4096, 4096)),
             (("bf16", "turbo4", 16, 8, 128), (32768, 9216), (32768, 8192)),
             (("fp8", "turbo2", 16, 8, 128), (16384, 5120), (16384, 4096)),
             (("turbo3", "turbo3", 16, 4, 256), (7168, 7168), (6144, 6144)),
             (("turbo4", "turbo3", 32, 8, 128), (18432, 14336), (16384, 12288))]
    for args, strides, data in cases:
        k, v = layout.pool_layout(*args)
        assert (k.block_stride_bytes, v.block_stride_bytes) == strides
        assert (k.data_section_bytes, v.data_section_bytes) == data


def test_rotation_flags():
    assert [layout.is_rotated(f) for f in ("bf16", "fp8", "turbo2", "turbo3", "turbo4", "turbo8", "nvfp4")] == \
        [False, False, True, True, True, True, False]


def test_nvfp4_shares_turbo4_layout():
    # "same byte layout, different codebook": every size and offset agrees
    for bs, nkv, hd in [(16, 8, 128), (1, 1, 64), (32, 4, 256)]:
        a, b = layout.side_layout("nvfp4", bs, nkv, hd), layout.side_layout("turbo4", bs, nkv, hd)
        assert (a.data_section_bytes, a.scale_bytes, a.block_stride_bytes, a.row_bytes, a.row_scales) == \
            (b.data_section_bytes, b.scale_bytes, b.block_stride_bytes, b.row_bytes, b.row_scales)


def test_turbo8_sizes():
    # 1 byte per element plus a 2-byte BF16 scale per 16: 9 bits per element,
    # 6.25% above fp8 ("~6% extra cache memory")
    s = layout.side_layout("turbo8", 16, 8, 128)
    e = 16 * 8 * 128
    assert (s.data_section_bytes, s.scale_bytes) == (e, e // 8)
    assert 8 * (s.data_section_bytes + s.scale_bytes) / e == 9.0
    assert s.row_bytes == 128 and s.row_scales == 16
