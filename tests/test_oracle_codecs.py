"""Oracle codecs pinned to torch's CPU conversions (a library routine)."""
import numpy as np
import pytest
import torch

from oracle import codecs


def _torch_bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _patterns_near_ties(exps, rng):
    """fp32 values whose discarded bits sit at, just below and just above the tie."""
    out = []
    for e in exps:
        top = np.arange(1 << 16, dtype=np.uint32)
        for rest in (0, 1, 0x3F, 0x40, 0x41, 0x7F):
            m = (top << np.uint32(7)) | np.uint32(rest)
            bits = (np.uint32(e + 127) << np.uint32(23)) | (m & np.uint32(0x7FFFFF))
            out.append(bits)
    out.append(rng.integers(0, 0x7F800000, 2_000_000, dtype=np.uint32))
    b = np.concatenate(out)
    b = np.concatenate([b, b | np.uint32(0x80000000)])
    return b.view(np.float32)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    u = rng.integers(0, 0x7F7FFFFF, 4_000_000, dtype=np.uint32)
    ties = (rng.integers(0, 0x7F7F, 100_000, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    near = ties + np.uint32(1)
    below = ties - np.uint32(1)
    u = np.concatenate([u, ties, near, below, np.array([0, 0x00008000, 0x00018000, 0x7F7F8000], np.uint32)])
    u = np.concatenate([u, u | np.uint32(0x80000000)])
    x = u.view(np.float32)
    assert np.array_equal(codecs.bf16_round_bits(x), _torch_bf16_bits(x))


def test_bf16_ties_to_even_examples():
    # 1 + 2^-8 lies halfway between bf16 1.0 and 1 + 2^-7: stays at 1.0 (even)
    assert codecs.bf16_round(np.float32([1.0 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6: goes up
    assert codecs.bf16_round(np.float32([1.0 + 3 * 2.0 ** -8]))[0] == np.float32(1.0 + 2.0 ** -6)


def test_e4m3_table_matches_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    ours = codecs.E4M3_VALUES.astype(np.float32)
    nan = np.isnan(ours)
    assert np.array_equal(nan, np.isnan(b))
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], b[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_e4m3_encode_matches_torch_after_clamp():
    rng = np.random.default_rng(1)
    x = _patterns_near_ties(range(-14, 11), rng)
    x = x[np.isfinite(x)]
    ours = codecs.e4m3_encode(x)
    xc = np.clip(x, -448.0, 448.0).astype(np.float32)
    ref = torch.from_numpy(xc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("v,code", [(0.0, 0x00), (-0.0, 0x80), (448.0, 0x7E), (1e9, 0x7E),
                                    (-1e9, 0xFE), (2.0 ** -9, 0x01), (2.0 ** -10, 0x00),
                                    (1.5 * 2.0 ** -10, 0x01), (17.0, 0x58), (19.0, 0x5A)])
def test_e4m3_encode_examples(v, code):
    # OCP E4M3FN: 17 is halfway between 16 (0x58) and 18 (0x59): ties to even -> 16;
    # 19 is halfway between 18 and 20 (0x5A): ties to even -> 20
    assert codecs.e4m3_encode(np.float32([v]))[0] == code


# ---- E2M1 (the NVFP4 element type)

def test_e2m1_values_follow_the_format_definition():
    # 1 sign, 2 exponent bits with bias 1, 1 mantissa bit: exponent field 0 is
    # subnormal (m/2), otherwise (1 + m/2) * 2^(e - 1)
    assert list(codecs.E2M1_VALUES[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(codecs.E2M1_VALUES[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert np.signbit(codecs.E2M1_VALUES[8])


def _e2m1_by_rint(v):
    """Independent rounding: per binade, scale to its integer grid and let
    np.rint (round half to even) pick; an even grid index is an even mantissa."""
    a = np.minimum(np.abs(v.astype(np.float64)), 6.0)
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    q = np.minimum(np.rint(a / step) * step, 6.0)
    mag = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}
    code = np.array([mag[float(x)] for x in q], dtype=np.uint8)
    return code | np.where(np.signbit(v), np.uint8(8), np.uint8(0))


def test_e2m1_encode_matches_rint_rounding():
    rng = np.random.default_rng(3)
    grid = np.arange(0, 8.0 + 1e-9, 1 / 64, dtype=np.float64)       # every tie, binade edge, saturation
    v = np.concatenate([grid, -grid, rng.uniform(-9, 9, 20000),
                        np.nextafter(np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]), np.float32(0)),
                        np.nextafter(np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]), np.float32(9))])
    v = v.astype(np.float32)
    assert np.array_equal(codecs.e2m1_encode(v), _e2m1_by_rint(v))


@pytest.mark.parametrize("v,code", [(0.25, 0x0), (0.75, 0x2), (1.25, 0x2), (1.75, 0x4), (2.5, 0x4),
                                    (3.5, 0x6), (5.0, 0x6), (5.01, 0x7), (100.0, 0x7), (-0.1, 0x8),
                                    (-0.0, 0x8), (-6.0, 0xF), (0.26, 0x1)])
def test_e2m1_encode_examples(v, code):
    assert int(codecs.e2m1_encode(np.float32([v]))[0]) == code
