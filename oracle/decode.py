"""Paged decode attention over the quantized pools, in fp64.

"metrale_model_layers/layers/ops/kv_cache_bf16k_turbov.rs",
``paged_decode_attn_bf16k_turbo{2,3,4}v``: one query token per sequence
attends to the sequence's cached positions through ``block_tables`` and
``seq_lens`` with scale ``inv_sqrt_d``, an optional ``sliding_window``, and
skips a position's V when its attention weight is at most the sparse-V
threshold.  "combs_models/kv.rs": ``repeat_kv`` (q head h reads kv head
h // (Hq/Hkv)), ``attend`` (scores * scale, softmax, P @ V; a single decode
query needs no mask), the paged gather (position j lives in page
table[j // page_size] at offset j % page_size) and the contiguous cache as
the brute-force baseline.  "spark_runtime/kv_cache.rs", ``is_wht_rotated``:
a rotated K side is read with the rotated query, a rotated V side yields a
rotated output that is rotated back.

Readings:
  * seq_lens[s] counts the token just written (append, then attend).
  * sliding_window W > 0 attends positions j >= L - W; W = 0 is off.
  * The sparse-V "attention weight" is the normalized softmax probability
    over the whole attended window; a position contributes iff p > thr,
    with no renormalization.  thr = 0 is dense attention.
  * q is bf16, the output fp32 (RN32 of the fp64 result).
"""
from __future__ import annotations

import numpy as np

from . import codecs, wht
from .layout import BITS, GROUP, TURBO, Side, is_rotated
from .write import tables, unpack_codes


def dequant_rows(pool: np.ndarray, side: Side, slots: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """Dequantized rows for every kv head of `slots`: fp64 [P, Hkv, hd]."""
    P = len(slots)
    nkv, hd, bs = side.num_kv_heads, side.head_dim, side.block_size
    slots = np.asarray(slots, dtype=np.int64)
    blk = slots // bs
    off = slots % bs
    row = off[:, None] * nkv + np.arange(nkv)[None, :]           # [P, Hkv]
    base = (blk * side.block_stride_bytes)[:, None]
    caddr = base + row * side.row_bytes
    data = pool[(caddr.reshape(-1, 1) + np.arange(side.row_bytes)).ravel()]
    data = data.reshape(P * nkv, side.row_bytes)
    if side.fmt == "bf16":
        vals = codecs.bf16_bits_to_f32(data.view(np.uint16)).astype(np.float64)
    elif side.fmt == "fp8":
        vals = codecs.e4m3_decode(data).astype(np.float64) * np.float64(np.float32(scale))
    elif side.fmt == "turbo8":
        saddr = base + side.data_section_bytes + row * side.row_scales
        sig = pool[(saddr.reshape(-1, 1) + np.arange(side.row_scales)).ravel()]
        sig = np.ascontiguousarray(sig.reshape(P * nkv, side.row_scales)).view("<u2")
        sq = codecs.bf16_bits_to_f32(sig).astype(np.float64)
        vals = codecs.e4m3_decode(data).astype(np.float64) * np.repeat(sq, GROUP, axis=1)
    elif side.fmt == "nvfp4":
        codes = unpack_codes(data, 4, hd)
        saddr = base + side.data_section_bytes + row * side.row_scales
        sig = pool[(saddr.reshape(-1, 1) + np.arange(side.row_scales)).ravel()]
        sq = codecs.e4m3_decode(sig.reshape(P * nkv, side.row_scales)).astype(np.float64)
        vals = codecs.E2M1_VALUES[codes] * np.repeat(sq, GROUP, axis=1)
    else:
        t = tables(side.fmt)
        codes = unpack_codes(data, BITS[side.fmt], hd)
        saddr = base + side.data_section_bytes + row * side.row_scales
        sig = pool[(saddr.reshape(-1, 1) + np.arange(side.row_scales)).ravel()]
        sq = codecs.e4m3_decode(sig.reshape(P * nkv, side.row_scales)).astype(np.float64)
        cen = t["centroids"].astype(np.float64)[codes]               # [P*Hkv, hd]
        vals = cen * np.repeat(sq, GROUP, axis=1)
    return vals.reshape(P, nkv, hd)


def attend(qv: np.ndarray, K: np.ndarray, V: np.ndarray, inv_sqrt_d: float, thr: float):
    """One query against a materialised window, fp64.

    qv [hd]; K, V [P, hd].  Returns (o [hd], p [P], keep [P]).
    """
    s = (K @ qv) * np.float64(np.float32(inv_sqrt_d))
    m = np.max(s)
    e = np.exp(s - m)
    p = e / np.sum(e)
    keep = p > thr
    o = p[keep] @ V[keep]
    return o, p, keep


def paged_decode(k_side: Side, v_side: Side, q_bits: np.ndarray, k_pool: np.ndarray,
                 v_pool: np.ndarray, block_tables: np.ndarray, seq_lens: np.ndarray,
                 inv_sqrt_d: float, sliding_window: int = 0, thr: float = 0.0,
                 k_scale: float = 1.0, v_scale: float = 1.0, seqs=None, detail: bool = False):
    """out fp32 [S, Hq, hd] (rows of sequences not in `seqs` stay zero).

    With detail=True also returns, per (s, h), the fp64 output and the
    element-wise bound on what positions with |p - thr| <= 1e-4*thr can change
    (the band inside which an fp32 implementation may decide either way).
    """
    S, Hq, hd = q_bits.shape
    nkv, bs = k_side.num_kv_heads, k_side.block_size
    G = Hq // nkv
    out = np.zeros((S, Hq, hd), dtype=np.float32)
    o64 = np.zeros((S, Hq, hd), dtype=np.float64)
    band = np.zeros((S, Hq, hd), dtype=np.float64)
    n_amb = np.zeros((S, Hq), dtype=np.int64)
    H = wht.hadamard_f64(hd) if (is_rotated(k_side.fmt) or is_rotated(v_side.fmt)) else None
    q = codecs.bf16_bits_to_f32(q_bits).astype(np.float64)
    for s in (range(S) if seqs is None else seqs):
        L = int(seq_lens[s])
        if L <= 0:
            continue
        j0 = max(0, L - sliding_window) if sliding_window > 0 else 0
        j = np.arange(j0, L, dtype=np.int64)
        slots = block_tables[s, j // bs].astype(np.int64) * bs + j % bs
        K = dequant_rows(k_pool, k_side, slots, k_scale)
        V = dequant_rows(v_pool, v_side, slots, v_scale)
        for h in range(Hq):
            g = h // G
            qv = q[s, h]
            if is_rotated(k_side.fmt):
                qv = H @ qv
            o, p, keep = attend(qv, K[:, g, :], V[:, g, :], inv_sqrt_d, thr)
            if is_rotated(v_side.fmt):
                o = H @ o
            o64[s, h] = o
            out[s, h] = o.astype(np.float32)
            if detail and thr > 0:
                amb = np.abs(p - thr) <= 1e-4 * thr
                n_amb[s, h] = int(amb.sum())
                if amb.any():
                    d = p[amb, None] * V[amb, g, :]
                    if is_rotated(v_side.fmt):
                        d = d @ H.T
                    band[s, h] = np.abs(d).sum(axis=0)
    if detail:
        return out, o64, band, n_amb
    return out


def contiguous_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, inv_sqrt_d: float,
                         thr: float = 0.0) -> np.ndarray:
    """Brute force over contiguous K/V, GQA by repeating kv heads.

    q [Hq, hd] fp64, K/V [L, Hkv, hd] fp64 (already in the basis the scores
    are taken in).  Materialises the full [Hq, L] score matrix.
    """
    Hq = q.shape[0]
    L, nkv, hd = K.shape
    rep = Hq // nkv
    Kx = np.repeat(K.transpose(1, 0, 2), rep, axis=0)       # [Hq, L, hd]
    Vx = np.repeat(V.transpose(1, 0, 2), rep, axis=0)
    scores = np.einsum("hd,hld->hl", q, Kx) * np.float64(np.float32(inv_sqrt_d))
    scores -= scores.max(axis=1, keepdims=True)
    w = np.exp(scores)
    w /= w.sum(axis=1, keepdims=True)
    w = np.where(w > thr, w, 0.0)
    return np.einsum("hl,hld->hd", w, Vx)
