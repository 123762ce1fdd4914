"""The oracle's sparse-V ambiguity band (``paged_decode(detail=True)``), pinned.

"metrale_model_layers/layers/ops/kv_cache_bf16k_turbov.rs",
``paged_decode_attn_bf16k_turbo{2,3,4}v``: a position's V is skipped when its
attention weight is at most the threshold.  An fp32 implementation can decide
either way for a weight within 1e-4 * thr of thr; the oracle reports those
positions (``n_amb``) and the most they can move each output element
(``band``, in the basis the output is returned in).

The weights here are known in closed form: q = e_0 and every K row is 0 or
e_0 (bf16 K), so position 0 scores 0 and the other L - 1 score c = inv_sqrt_d,
and p_0 = 1 / (1 + (L - 1) e^c).  The threshold is placed relative to p_0.
The band's basis is checked against the oracle's own output path: keeping
position 0 instead of dropping it changes the output by exactly p_0 times
that position's V row in the output basis.
"""
import math

import numpy as np
import pytest

from oracle import codecs, layout
from oracle import decode as D
from oracle import write as W

L, HD, BS, INV = 8, 64, 4, 0.5


def _case(vf, seed=0):
    """One sequence, Hkv = 1, G = 2 (head 1's query is zero: uniform weights)."""
    rng = np.random.default_rng(seed)
    ks, vs = layout.pool_layout("bf16", vf, BS, 1, HD)
    nblk = L // BS
    bt = np.array([[2, 0, -1]], np.int32)[:, :nblk + 1]
    kx = np.zeros((L, 1, HD), np.float32)
    kx[1:, 0, 0] = 1.0
    vx = rng.standard_normal((L, 1, HD)).astype(np.float32)
    kp = np.zeros(4 * ks.block_stride_bytes, np.uint8)
    vp = np.zeros(4 * vs.block_stride_bytes, np.uint8)
    j = np.arange(L)
    slots = bt[0, j // BS].astype(np.int64) * BS + j % BS
    W.reshape_and_cache(ks, vs, codecs.bf16_round_bits(kx), codecs.bf16_round_bits(vx), kp, vp, slots)
    q = np.zeros((1, 2, HD), np.float32)
    q[0, 0, 0] = 1.0
    return ks, vs, kp, vp, bt, codecs.bf16_round_bits(q)


def _p0():
    c = float(np.float32(INV))   # the scale is an fp32 argument
    return 1.0 / (1.0 + (L - 1) * math.exp(c)), math.exp(c) / (1.0 + (L - 1) * math.exp(c))


def _run(case, thr):
    ks, vs, kp, vp, bt, q = case
    return D.paged_decode(ks, vs, q, kp, vp, bt, np.array([L], np.int32), INV, 0, thr, detail=True)


@pytest.mark.parametrize("vf", ["bf16", "turbo4", "turbo2", "turbo8", "nvfp4"])
def test_band_counts_the_weight_near_thr(vf):
    case = _case(vf)
    p0, p1 = _p0()
    assert abs(p1 - p0) > 0.1 * p0 and abs(1.0 / 8.0 - p0) > 0.1 * p0   # only p0 is near thr
    # kept (just above thr) or dropped (just below): ambiguous either way
    for rel in (1 + 5e-5, 1 - 5e-5):
        thr = p0 / rel
        _, o64, band, n_amb = _run(case, thr)
        assert n_amb[0, 0] == 1, (rel, n_amb)
        assert n_amb[0, 1] == 0 and not band[0, 1].any()
        # what position 0 adds to head 0's output, in the output basis
        _, keep, _, _ = _run(case, p0 * 0.9)
        _, drop, _, _ = _run(case, p0 * 1.1)
        contrib = keep[0, 0] - drop[0, 0]
        assert np.abs(contrib).max() > 1e-3
        np.testing.assert_allclose(band[0, 0], np.abs(contrib), rtol=1e-9, atol=1e-15)
        # the decision itself: p0 > thr keeps position 0
        np.testing.assert_allclose(o64[0, 0], keep[0, 0] if p0 > thr else drop[0, 0], rtol=0, atol=1e-15)


@pytest.mark.parametrize("vf", ["bf16", "turbo4"])
def test_band_empty_away_from_thr(vf):
    case = _case(vf)
    p0, p1 = _p0()
    for thr in (p0 / (1 + 3e-4), p0 / (1 - 3e-4), p0 * 0.5, (p0 + p1) / 2):
        _, _, band, n_amb = _run(case, thr)
        assert not n_amb.any() and not band.any(), thr
    # dense attention has no band
    _, _, band, n_amb = _run(case, 0.0)
    assert not n_amb.any() and not band.any()


def test_band_counts_every_ambiguous_position():
    """The L - 1 equal weights p1 all sit at thr: each is counted, and the band
    is the sum of their elementwise magnitudes."""
    case = _case("bf16", seed=3)
    p0, p1 = _p0()
    _, _, band, n_amb = _run(case, p1 / (1 + 2e-5))
    assert n_amb[0, 0] == L - 1
    ks, vs, kp, vp, bt, q = case
    j = np.arange(1, L)
    slots = bt[0, j // BS].astype(np.int64) * BS + j % BS
    # bf16 V rows straight from the pool bytes: row (offset, head 0) of the block
    rows = [vp[(s // BS) * vs.block_stride_bytes + (s % BS) * 2 * HD:][:2 * HD].view(np.uint16) for s in slots]
    v = codecs.bf16_bits_to_f32(np.stack(rows)).astype(np.float64)
    np.testing.assert_allclose(band[0, 0], (p1 * np.abs(v)).sum(axis=0), rtol=1e-12)
