"""Oracle chunked prefill pinned to a masked-matrix brute force, to decode and
to its special cases."""
import math

import numpy as np
import pytest

from oracle import codecs, layout, wht
from oracle import decode as D
from oracle import prefill as PF
from oracle import write as W

from test_oracle_decode import _build, _dequant_contig


def _masked_matrix(q, K, V, pos, inv, window, G):
    """Bottom-right causal attention as one masked score matrix per head:
    q [C, Hq, hd], K/V [L, Hkv, hd]; query i sits at position pos + i."""
    C, Hq, _ = q.shape
    L = K.shape[0]
    qp = (pos + np.arange(C))[:, None]
    kp = np.arange(L)[None, :]
    allowed = kp <= qp
    if window > 0:
        allowed &= kp > qp - window
    out = np.zeros(q.shape)
    for h in range(Hq):
        S = q[:, h, :] @ K[:, h // G, :].T * inv
        S = np.where(allowed, S, -np.inf)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        out[:, h, :] = P @ V[:, h // G, :]
    return out


@pytest.mark.parametrize("kf,vf", [("bf16", "bf16"), ("fp8", "turbo2"), ("turbo4", "turbo3"), ("turbo8", "nvfp4"),
                                   ("nvfp4", "turbo8")])
@pytest.mark.parametrize("C,window", [(1, 0), (7, 0), (37, 0), (20, 5)])
def test_prefill_equals_masked_matrix(kf, vf, C, window):
    L, G = 37, 2
    c = _build(kf, vf, L=L, G=G, seed=C * 7 + len(kf))
    inv = float(np.float32(1 / math.sqrt(c["hd"])))
    rng = np.random.default_rng(C)
    q = codecs.bf16_round_bits(rng.standard_normal((C, c["q"].shape[1], c["hd"])).astype(np.float32))
    out, o64 = PF.paged_prefill(c["ks"], c["vs"], q, np.array([0, C]), c["kp"], c["vp"], c["bt"], np.array([L]),
                                inv, window, c["kscale"], c["vscale"])
    K = _dequant_contig(c["kb"], kf, c["kscale"])
    V = _dequant_contig(c["vb"], vf, c["vscale"])
    qq = codecs.bf16_bits_to_f32(q).astype(np.float64)
    H = wht.hadamard_f64(c["hd"])
    if layout.is_rotated(kf):
        qq = qq @ H.T
    ref = _masked_matrix(qq, K, V, L - C, np.float64(np.float32(inv)), window, G)
    if layout.is_rotated(vf):
        ref = ref @ H.T
    assert np.abs(o64 - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_last_query_equals_decode_and_ragged_batch():
    # two sequences in one call: lengths 37 and 20, chunks of 5 and 20 (the
    # second is a whole prompt); each chunk's last query is that sequence's decode
    c1 = _build("turbo4", "turbo3", L=37, G=2, seed=3)
    c2 = _build("turbo4", "turbo3", L=20, G=2, seed=4)
    ks, vs = c1["ks"], c1["vs"]
    off = len(c1["kp"]) // ks.block_stride_bytes
    kp = np.concatenate([c1["kp"], c2["kp"]])
    vp = np.concatenate([c1["vp"], c2["vp"]])
    bt = np.full((2, max(c1["bt"].shape[1], c2["bt"].shape[1])), -1, np.int32)
    bt[0, :c1["bt"].shape[1]] = c1["bt"][0]
    b2 = c2["bt"][0]
    bt[1, :len(b2)] = np.where(b2 >= 0, b2 + off, -1)
    lens = np.array([37, 20])
    rng = np.random.default_rng(9)
    Hq, hd = c1["q"].shape[1], c1["hd"]
    q = codecs.bf16_round_bits(rng.standard_normal((25, Hq, hd)).astype(np.float32))
    qs = np.array([0, 5, 25])
    inv = float(np.float32(1 / math.sqrt(hd)))
    out, _ = PF.paged_prefill(ks, vs, q, qs, kp, vp, bt, lens, inv)
    dq = np.stack([q[4], q[24]])
    dec = D.paged_decode(ks, vs, dq, kp, vp, bt, lens, inv)
    assert np.array_equal(out[4], dec[0]) or np.abs(out[4] - dec[0]).max() <= 1e-6 * np.abs(dec[0]).max()
    assert np.abs(out[24] - dec[1]).max() <= 1e-6 * np.abs(dec[1]).max()
    # the first query of the whole prompt attends to position 0 only: its output is V[0]
    V = _dequant_contig(c2["vb"], "turbo3", c2["vscale"])
    H = wht.hadamard_f64(hd)
    for h in range(Hq):
        assert np.allclose(out[5, h], (V[0, h // 2] @ H.T).astype(np.float32), rtol=0, atol=1e-6)


def test_window_at_least_the_length_is_no_window():
    c = _build("bf16", "turbo4", L=30, G=2, seed=1)
    rng = np.random.default_rng(2)
    q = codecs.bf16_round_bits(rng.standard_normal((12, c["q"].shape[1], c["hd"])).astype(np.float32))
    inv = float(np.float32(1 / math.sqrt(c["hd"])))
    a = PF.paged_prefill(c["ks"], c["vs"], q, np.array([0, 12]), c["kp"], c["vp"], c["bt"], np.array([30]), inv, 0)
    b = PF.paged_prefill(c["ks"], c["vs"], q, np.array([0, 12]), c["kp"], c["vp"], c["bt"], np.array([30]), inv, 30)
    assert np.array_equal(a[1], b[1])
