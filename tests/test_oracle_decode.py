"""Oracle paged decode pinned to brute force and invariants."""
import itertools
import math

import numpy as np
import pytest

from oracle import codecs, layout, wht
from oracle import decode as D
from oracle import write as W


def _build(kf, vf, L, nkv=2, G=2, hd=64, bs=4, seed=0, outliers=True, extra_blocks=3):
    rng = np.random.default_rng(seed)
    ks, vs = layout.pool_layout(kf, vf, bs, nkv, hd)
    nblk = (L + bs - 1) // bs
    nb = nblk + extra_blocks
    perm = rng.permutation(nb)
    bt = np.full((1, nblk + 2), -1, np.int32)
    bt[0, :nblk] = perm[:nblk]
    x = rng.standard_normal((2, L, nkv, hd)).astype(np.float32)
    if outliers:
        x[..., rng.choice(hd, 3, replace=False)] *= 20
    kb, vb = codecs.bf16_round_bits(x[0]), codecs.bf16_round_bits(x[1])
    kp = np.zeros(nb * ks.block_stride_bytes, np.uint8)
    vp = np.zeros(nb * vs.block_stride_bytes, np.uint8)
    j = np.arange(L)
    slots = bt[0, j // bs].astype(np.int64) * bs + j % bs
    kscale = float(np.float32(np.abs(codecs.bf16_bits_to_f32(kb)).max() / np.float32(448)))
    vscale = float(np.float32(np.abs(codecs.bf16_bits_to_f32(vb)).max() / np.float32(448)))
    W.reshape_and_cache(ks, vs, kb, vb, kp, vp, slots, kscale, vscale)
    q = codecs.bf16_round_bits(rng.standard_normal((1, nkv * G, hd)).astype(np.float32))
    return dict(ks=ks, vs=vs, kp=kp, vp=vp, bt=bt, q=q, kb=kb, vb=vb, kscale=kscale,
                vscale=vscale, L=L, hd=hd)


def _dequant_contig(bits, fmt, scale):
    """Quantize + dequantize rows in position order, without any pool."""
    L, nkv, hd = bits.shape
    data, sc = W.quantize_rows(bits.reshape(-1, hd), fmt, scale)
    if fmt == "bf16":
        v = codecs.bf16_bits_to_f32(data.view(np.uint16)).astype(np.float64)
    elif fmt == "fp8":
        v = codecs.e4m3_decode(data).astype(np.float64) * np.float64(np.float32(scale))
    elif fmt == "turbo8":
        sq = (sc[:, 0::2].astype(np.uint32) | (sc[:, 1::2].astype(np.uint32) << 8)) << 16
        v = codecs.e4m3_decode(data).astype(np.float64) * \
            np.repeat(sq.astype(np.uint32).view(np.float32).astype(np.float64), 16, axis=1)
    elif fmt == "nvfp4":
        nib = np.stack([data & 0xF, data >> 4], axis=-1).reshape(data.shape[0], hd)
        v = codecs.E2M1_VALUES[nib] * np.repeat(codecs.e4m3_decode(sc).astype(np.float64), 16, axis=1)
    else:
        codes = W.unpack_codes(data, layout.BITS[fmt], hd)
        v = W.tables(fmt)["centroids"].astype(np.float64)[codes] * \
            np.repeat(codecs.e4m3_decode(sc).astype(np.float64), 16, axis=1)
    return v.reshape(L, nkv, hd)


PAIRS = [("bf16", "bf16"), ("fp8", "fp8"), ("turbo2", "turbo2"), ("turbo3", "turbo3"),
         ("turbo4", "turbo4"), ("turbo4", "turbo3"), ("bf16", "turbo4"), ("bf16", "turbo3"),
         ("bf16", "turbo2"), ("fp8", "turbo4"), ("fp8", "turbo3"), ("fp8", "turbo2"),
         ("turbo8", "turbo8"), ("turbo4", "turbo8"), ("turbo3", "turbo8"), ("bf16", "turbo8"),
         ("nvfp4", "nvfp4"), ("bf16", "nvfp4"), ("nvfp4", "turbo3"), ("turbo4", "nvfp4")]


@pytest.mark.parametrize("kf,vf", PAIRS)
@pytest.mark.parametrize("thr", [0.0, 0.02])
def test_paged_equals_contiguous_brute_force(kf, vf, thr):
    c = _build(kf, vf, L=37, seed=hash((kf, vf)) % 1000)
    inv = float(np.float32(1 / math.sqrt(c["hd"])))
    out = D.paged_decode(c["ks"], c["vs"], c["q"], c["kp"], c["vp"], c["bt"], np.array([37]),
                         inv, 0, thr, c["kscale"], c["vscale"])
    K = _dequant_contig(c["kb"], kf, c["kscale"])
    V = _dequant_contig(c["vb"], vf, c["vscale"])
    q = codecs.bf16_bits_to_f32(c["q"][0]).astype(np.float64)
    H = wht.hadamard_f64(c["hd"])
    if layout.is_rotated(kf):
        q = q @ H.T
    o = D.contiguous_attention(q, K, V, inv, thr)
    if layout.is_rotated(vf):
        o = o @ H.T
    assert np.allclose(out[0], o, rtol=0, atol=1e-5 * np.abs(o).max())
    assert np.abs(out[0].astype(np.float64) - o).max() <= np.abs(o).max() * 2.0 ** -23


def test_bookends_equal_attention_in_original_basis():
    # turbo sides store rotated rows; attention in the original basis over
    # H^T(dequantized rows) must give the same output as the rotated decode
    c = _build("turbo4", "turbo3", L=50, seed=4)
    inv = float(np.float32(1 / 8))
    out = D.paged_decode(c["ks"], c["vs"], c["q"], c["kp"], c["vp"], c["bt"], np.array([50]), inv)
    H = wht.hadamard_f64(64)
    K = _dequant_contig(c["kb"], "turbo4", 1.0) @ H      # back to the original basis (H = H^T)
    V = _dequant_contig(c["vb"], "turbo3", 1.0) @ H
    q = codecs.bf16_bits_to_f32(c["q"][0]).astype(np.float64)
    o = D.contiguous_attention(q, K, V, inv)
    assert np.allclose(out[0], o, rtol=0, atol=1e-12 + 1e-6 * np.abs(o).max())


def test_brute_force_loops_tiny():
    # pure-python loops over positions, no numpy linear algebra
    c = _build("bf16", "bf16", L=9, nkv=1, G=3, hd=64, bs=4, seed=3, outliers=False)
    thr = 0.08
    inv = float(np.float32(0.125))
    out = D.paged_decode(c["ks"], c["vs"], c["q"], c["kp"], c["vp"], c["bt"], np.array([9]), inv, 0, thr)
    K = codecs.bf16_bits_to_f32(c["kb"]).astype(float)
    V = codecs.bf16_bits_to_f32(c["vb"]).astype(float)
    q = codecs.bf16_bits_to_f32(c["q"][0]).astype(float)
    for h in range(3):
        s = [sum(q[h][d] * K[j][0][d] for d in range(64)) * inv for j in range(9)]
        m = max(s)
        e = [math.exp(v - m) for v in s]
        z = sum(e)
        o = [0.0] * 64
        for j in range(9):
            if e[j] / z > thr:
                for d in range(64):
                    o[d] += e[j] / z * V[j][0][d]
        assert np.allclose(out[0, h], o, rtol=0, atol=1e-6)


def test_threshold_zero_is_dense():
    c = _build("bf16", "turbo2", L=64, seed=5)
    inv = float(np.float32(1 / 8))
    a = D.paged_decode(c["ks"], c["vs"], c["q"], c["kp"], c["vp"], c["bt"], np.array([64]), inv, 0, 0.0)
    K = _dequant_contig(c["kb"], "bf16", 1.0)
    V = _dequant_contig(c["vb"], "turbo2", 1.0)
    H = wht.hadamard_f64(64)
    q = codecs.bf16_bits_to_f32(c["q"][0]).astype(np.float64)
    for h in range(4):
        s = K[:, h // 2] @ q[h] * inv
        p = np.exp(s - s.max()); p /= p.sum()
        o = H @ (p @ V[:, h // 2])
        assert np.allclose(a[0, h], o, rtol=0, atol=1e-5 * np.abs(o).max())


def test_window_covering_everything_is_off_and_window_truncates():
    c = _build("fp8", "turbo3", L=45, seed=6)
    args = (c["ks"], c["vs"], c["q"], c["kp"], c["vp"], c["bt"], np.array([45]), 0.125)
    full = D.paged_decode(*args, 0, 0.0, c["kscale"], c["vscale"])
    assert np.array_equal(full, D.paged_decode(*args, 45, 0.0, c["kscale"], c["vscale"]))
    assert np.array_equal(full, D.paged_decode(*args, 1000, 0.0, c["kscale"], c["vscale"]))
    win = D.paged_decode(*args, 10, 0.0, c["kscale"], c["vscale"])
    K = _dequant_contig(c["kb"], "fp8", c["kscale"])[35:]
    V = _dequant_contig(c["vb"], "turbo3", c["vscale"])[35:]
    H = wht.hadamard_f64(64)
    q = codecs.bf16_bits_to_f32(c["q"][0]).astype(np.float64)
    o = D.contiguous_attention(q, K, V, 0.125) @ H.T
    assert np.allclose(win[0], o, rtol=0, atol=1e-5 * np.abs(o).max())
    assert not np.allclose(win, full)


def test_page_permutation_invariance():
    c = _build("turbo3", "turbo4", L=41, seed=7, extra_blocks=0)
    out = D.paged_decode(c["ks"], c["vs"], c["q"], c["kp"], c["vp"], c["bt"], np.array([41]), 0.125)
    # move every page to a new physical block and rewrite the table
    bs = 4
    n = (41 + bs - 1) // bs
    perm = np.random.default_rng(1).permutation(n)
    kp2, vp2 = np.zeros_like(c["kp"]), np.zeros_like(c["vp"])
    bt2 = c["bt"].copy()
    for i in range(n):
        old, new = c["bt"][0, i], perm[i]
        for side, src, dst in ((c["ks"], c["kp"], kp2), (c["vs"], c["vp"], vp2)):
            st = side.block_stride_bytes
            dst[new * st:(new + 1) * st] = src[old * st:(old + 1) * st]
        bt2[0, i] = new
    out2 = D.paged_decode(c["ks"], c["vs"], c["q"], kp2, vp2, bt2, np.array([41]), 0.125)
    assert np.array_equal(out, out2)


def test_empty_sequence_gives_zero():
    c = _build("bf16", "bf16", L=8, seed=8)
    out = D.paged_decode(c["ks"], c["vs"], c["q"], c["kp"], c["vp"], c["bt"], np.array([0]), 0.125)
    assert np.all(out == 0)


def test_mha_equals_per_head():
    c = _build("bf16", "fp8", L=20, nkv=3, G=1, seed=9)
    out = D.paged_decode(c["ks"], c["vs"], c["q"], c["kp"], c["vp"], c["bt"], np.array([20]), 0.125,
                         0, 0.0, 1.0, c["vscale"])
    K = _dequant_contig(c["kb"], "bf16", 1.0)
    V = _dequant_contig(c["vb"], "fp8", c["vscale"])
    q = codecs.bf16_bits_to_f32(c["q"][0]).astype(np.float64)
    for h in range(3):
        o = D.contiguous_attention(q[h:h + 1], K[:, h:h + 1], V[:, h:h + 1], 0.125)
        assert np.allclose(out[0, h], o[0], rtol=0, atol=1e-6)
