"""Oracle cache write pinned to brute force, hand-made bytes and library codecs."""
import numpy as np
import pytest
import torch

from oracle import codebook, codecs, layout, wht
from oracle import write as W


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_roundtrip(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(33, 256)).astype(np.uint8)
    packed = W.pack_codes(codes, bits)
    assert packed.shape == (33, 256 * bits // 8)
    assert np.array_equal(W.unpack_codes(packed, bits, 256), codes)


def test_pack_bytes_by_hand():
    # turbo4: element 2k in the low nibble of byte k
    assert W.pack_codes(np.array([[1, 2, 15, 0]], np.uint8), 4).tolist() == [[0x21, 0x0F]]
    # turbo2: byte k = c0 | c1<<2 | c2<<4 | c3<<6
    assert W.pack_codes(np.array([[1, 2, 3, 0, 3, 3, 3, 3]], np.uint8), 2).tolist() == [[0x39, 0xFF]]
    # turbo3: 8 codes -> 24-bit little-endian word, code j at bits 3j
    c = [1, 2, 3, 4, 5, 6, 7, 0]
    word = sum(v << (3 * j) for j, v in enumerate(c))
    assert W.pack_codes(np.array([c], np.uint8), 3).tolist() == [[word & 0xFF, (word >> 8) & 0xFF, word >> 16]]


def _rows(n, hd, seed, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, hd)).astype(np.float32)
    if outliers:
        x[:, rng.choice(hd, 4, replace=False)] *= 20
    return codecs.bf16_round_bits(x)


@pytest.mark.parametrize("fmt", ["turbo2", "turbo3", "turbo4"])
@pytest.mark.parametrize("hd", [64, 128, 256])
def test_codes_are_nearest_centroid(fmt, hd):
    x = codecs.bf16_bits_to_f32(_rows(300, hd, hd))
    codes, sigma = W.turbo_quantize(x, fmt)
    t = W.tables(fmt)
    y = codecs.bf16_round(wht.wht_f32(x)).astype(np.float64)
    sq = np.repeat(codecs.e4m3_decode(sigma).astype(np.float64), 16, axis=1)
    levels = sq[..., None] * t["centroids"].astype(np.float64)          # [N, hd, L]
    dist = np.abs(y[..., None] - levels)
    chosen = np.take_along_axis(dist, codes[..., None].astype(np.int64), -1)[..., 0]
    best = dist.min(-1)
    # thresholds are RN32(s_q * midpoint), so only elements within rounding of a
    # midpoint may pick the other neighbour
    assert np.all(chosen <= best + 1e-6 * sq + 1e-30)
    assert np.mean(chosen == best) > 0.999


@pytest.mark.parametrize("fmt", ["turbo2", "turbo3", "turbo4"])
def test_group_scale_rule(fmt):
    x = codecs.bf16_bits_to_f32(_rows(200, 128, 3))
    _, sigma = W.turbo_quantize(x, fmt)
    y = codecs.bf16_round(wht.wht_f32(x))
    a = np.abs(y.reshape(200, 8, 16)).max(-1).astype(np.float64)
    cmax = W.tables(fmt)["centroids_f64"][-1]
    sq = codecs.e4m3_decode(sigma).astype(np.float64)
    # E4M3 keeps 3 mantissa bits: relative rounding error at most 2^-4
    assert np.all(np.abs(sq * cmax - a) <= a * 2.0 ** -4 * 1.0001)


@pytest.mark.parametrize("fmt,bound", [("turbo4", 0.015), ("turbo3", 0.05), ("turbo2", 0.2)])
def test_quantization_error_near_lloyd_max(fmt, bound):
    x = codecs.bf16_bits_to_f32(_rows(2000, 128, 5))
    codes, sigma = W.turbo_quantize(x, fmt)
    t = W.tables(fmt)
    y = codecs.bf16_round(wht.wht_f32(x)).astype(np.float64)
    sq = np.repeat(codecs.e4m3_decode(sigma).astype(np.float64), 16, axis=1)
    yhat = sq * t["centroids"].astype(np.float64)[codes]
    rel = ((yhat - y) ** 2).sum() / (y ** 2).sum()
    assert rel < bound
    # the rotation is what makes outliers cheap: without it the error is far larger
    xg = x.astype(np.float64).reshape(-1, 16)
    s0 = np.abs(xg).max(1, keepdims=True) / t["centroids_f64"][-1]
    c0 = np.argmin(np.abs(xg[..., None] / s0[..., None] - t["centroids_f64"]), -1)
    rel0 = ((s0 * t["centroids_f64"][c0] - xg) ** 2).sum() / (xg ** 2).sum()
    assert rel0 > 1.5 * rel


def test_fp8_rows_match_torch():
    x_bits = _rows(500, 128, 9)
    x = codecs.bf16_bits_to_f32(x_bits)
    scale = np.float32(np.abs(x).max() / np.float32(448))
    data, sc = W.quantize_rows(x_bits, "fp8", float(scale))
    v = torch.from_numpy(x) / torch.tensor(scale, dtype=torch.float32)
    ref = v.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(data, ref) and sc.shape == (500, 0)


def _turbo8_reference(x):
    """The turbo8 rule through torch's own bf16 / float8_e4m3fn conversions."""
    y = torch.from_numpy(codecs.bf16_round(wht.wht_f32(x)))
    n, hd = y.shape
    yg = y.reshape(n, hd // 16, 16)
    a = yg.abs().amax(-1)
    s = a * torch.tensor(1.0 / 448.0, dtype=torch.float32)
    sig = s.to(torch.bfloat16)
    sq = sig.to(torch.float32)
    v = torch.where(sq[..., None] > 0, yg / sq.clamp_min(1e-45)[..., None], torch.zeros_like(yg))
    codes = v.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.reshape(n, hd).numpy(), sig.view(torch.int16).numpy().view(np.uint16), y.numpy(), sq.numpy()


@pytest.mark.parametrize("hd", [64, 128, 256])
def test_turbo8_matches_torch_conversions(hd):
    x = codecs.bf16_bits_to_f32(_rows(400, hd, 11 + hd))
    codes, sigma = W.turbo8_quantize(x)
    rc, rs, _, _ = _turbo8_reference(x)
    assert np.array_equal(sigma, rs)
    assert np.array_equal(codes, rc)


def test_turbo8_properties():
    x = codecs.bf16_bits_to_f32(_rows(300, 128, 21))
    x[7] = 0.0                                   # an all-zero row: zero scales, zero bytes
    codes, sigma = W.turbo8_quantize(x)
    y = codecs.bf16_round(wht.wht_f32(x)).astype(np.float64)
    sq = codecs.bf16_bits_to_f32(sigma).astype(np.float64)
    assert np.all(sigma[7] == 0) and np.all(codes[7] == 0)
    vals = codecs.e4m3_decode(codes).astype(np.float64).reshape(300, 8, 16)
    yg = y.reshape(300, 8, 16)
    # the group's largest magnitude lands on the largest E4M3 value (s_q is
    # within 2^-9 of absmax/448, and 448 is 32 away from its neighbour 416)
    idx = np.abs(yg).argmax(-1)
    top = np.take_along_axis(np.abs(vals), idx[..., None], -1)[..., 0]
    live = sq > 0
    assert np.all(top[live] == 448.0)
    # every element within E4M3's relative step (2^-4), or its subnormal step
    err = np.abs(vals * sq[..., None] - yg)
    assert np.all(err <= np.maximum(np.abs(yg) * 2.0 ** -4, sq[..., None] * 2.0 ** -9) * 1.0001)


def test_turbo8_rows_carry_little_endian_scales():
    x_bits = _rows(20, 128, 31)
    data, sc = W.quantize_rows(x_bits, "turbo8")
    codes, sigma = W.turbo8_quantize(codecs.bf16_bits_to_f32(x_bits))
    assert np.array_equal(data, codes) and sc.shape == (20, 16)
    assert np.array_equal(sc[:, 0::2].astype(np.uint16) | (sc[:, 1::2].astype(np.uint16) << 8), sigma)


def test_bf16_rows_are_raw_bytes():
    x_bits = _rows(10, 64, 2)
    data, _ = W.quantize_rows(x_bits, "bf16")
    assert np.array_equal(data.view(np.uint16), x_bits)


@pytest.mark.parametrize("kf,vf", [("bf16", "turbo4"), ("fp8", "turbo2"), ("turbo3", "turbo3"),
                                   ("turbo4", "turbo3"), ("turbo4", "turbo8"), ("turbo8", "turbo8")])
def test_pool_placement(kf, vf):
    bs, nkv, hd, nb = 4, 2, 64, 6
    ks, vs = layout.pool_layout(kf, vf, bs, nkv, hd)
    kp = np.full(nb * ks.block_stride_bytes, 0xAA, np.uint8)
    vp = np.full(nb * vs.block_stride_bytes, 0xAA, np.uint8)
    T = 7
    key = _rows(T * nkv, hd, 11).reshape(T, nkv, hd)
    val = _rows(T * nkv, hd, 12).reshape(T, nkv, hd)
    slots = np.array([5, -1, 0, 23, 9, -3, 14])
    W.reshape_and_cache(ks, vs, key, val, kp, vp, slots, 0.5, 0.25)
    for side, pool, x, sc in ((ks, kp, key, 0.5), (vs, vp, val, 0.25)):
        touched = np.zeros(pool.size, bool)
        for t, slot in enumerate(slots):
            if slot < 0:
                continue
            blk, off = divmod(slot, bs)
            data, scl = W.quantize_rows(x[t], side.fmt, sc)
            for h in range(nkv):
                row = off * nkv + h
                a = blk * side.block_stride_bytes + row * side.row_bytes
                assert np.array_equal(pool[a:a + side.row_bytes], data[h])
                touched[a:a + side.row_bytes] = True
                if side.row_scales:
                    b = blk * side.block_stride_bytes + side.data_section_bytes + row * side.row_scales
                    assert np.array_equal(pool[b:b + side.row_scales], scl[h])
                    touched[b:b + side.row_scales] = True
        assert np.all(pool[~touched] == 0xAA)


# ---- NVFP4

def test_nvfp4_nibbles_are_a_nearest_grid_point():
    rng = np.random.default_rng(11)
    x = codecs.bf16_round(rng.standard_normal((256, 128)).astype(np.float32) * 3)
    x[:, 5] *= 40
    nib, sigma = W.nvfp4_quantize(x)
    sq = codecs.e4m3_decode(sigma).astype(np.float64)                       # [256, 8]
    assert np.array_equal(sigma, codecs.e4m3_encode(
        (np.abs(x).reshape(256, 8, 16).max(-1) * np.float32(1 / 6)).astype(np.float32)))
    grid = codecs.E2M1_VALUES[None, None, None, :] * sq[..., None, None]   # [256, 8, 1, 16]
    xg = x.reshape(256, 8, 16).astype(np.float64)
    deq = codecs.E2M1_VALUES[nib].reshape(256, 8, 16) * sq[..., None]
    best = np.abs(grid - xg[..., None]).min(-1)
    # nearest up to the one rounding of x / s_q in fp32
    assert np.all(np.abs(deq - xg) <= best + np.abs(xg) * 2.0 ** -22)


def test_nvfp4_zero_and_tiny_groups():
    x = np.zeros((2, 64), np.float32)
    x[1, 16:32] = -1e-30                                      # absmax / 6 far below E4M3's smallest step
    nib, sigma = W.nvfp4_quantize(x)
    assert not nib.any() and not sigma.any()


def test_nvfp4_rows_pack_like_turbo4():
    x_bits = codecs.bf16_round_bits(np.linspace(-5, 5, 2 * 64, dtype=np.float32).reshape(2, 64))
    data, sc = W.quantize_rows(x_bits, "nvfp4")
    nib, sigma = W.nvfp4_quantize(codecs.bf16_bits_to_f32(x_bits))
    assert np.array_equal(data[:, 0] & 0xF, nib[:, 0]) and np.array_equal(data[:, 0] >> 4, nib[:, 1])
    assert np.array_equal(sc, sigma) and data.shape == (2, 32)


def test_turbo4_beats_nvfp4_mse_on_gaussian_rows():
    # the Turbo4 doc comment credits rotation + the Lloyd-Max book with about
    # half the NVFP4 error at the same bits; on N(0,1) rows the oracle gives
    # 1.54x (with x20 outlier channels 1.44x), i.e. clearly lower, not 2x
    rng = np.random.default_rng(0)
    x = codecs.bf16_round(rng.standard_normal((4096, 128)).astype(np.float32))
    codes, sig = W.turbo_quantize(x, "turbo4")
    y = codecs.bf16_round(wht.wht_f32(x))
    deq_t = W.tables("turbo4")["centroids"].astype(np.float64)[codes] * \
        np.repeat(codecs.e4m3_decode(sig).astype(np.float64), 16, axis=1)
    nib, s2 = W.nvfp4_quantize(x)
    deq_n = codecs.E2M1_VALUES[nib] * np.repeat(codecs.e4m3_decode(s2).astype(np.float64), 16, axis=1)
    ratio = np.mean((deq_n - x) ** 2) / np.mean((deq_t - y) ** 2)
    assert 1.4 < ratio < 1.7
