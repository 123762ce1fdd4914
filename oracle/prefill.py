"""Chunked prefill attention over the quantized pools, in fp64.

Test infrastructure: the reference the library's prefill kernel is checked
against.

"combs_models/kv.rs", ``attend``: a chunk of ``seq`` query tokens whose first
one sits at absolute position ``pos`` attends to the ``total`` cached
positions with the causal mask aligned to the bottom right: query
``pos + i`` sees keys ``0 .. pos + i`` (a key after the query is masked out),
after the chunk's own K/V were appended; scale, softmax and P @ V as for
decode, GQA by ``repeat_kv``.  "spark_runtime/kv_cache.rs", full write +
paged-decode + chunked-prefill coverage of the quantized formats; a rotated
K side is read with the rotated query, a rotated V side gives a rotated
output that is rotated back (``is_wht_rotated``).

Readings:
  * Sequence s has seq_lens[s] cached positions (its chunk included) and
    C = query_start[s + 1] - query_start[s] <= seq_lens[s] query rows, for
    positions seq_lens[s] - C .. seq_lens[s] - 1, in that order.
  * sliding_window W > 0 applies to every query on its own: query p attends
    keys j with p - W < j <= p.
  * No sparse-V skip: the threshold is a decode feature.
  * q is bf16, the output fp32 (RN32 of the fp64 result).
"""
from __future__ import annotations

import numpy as np

from . import codecs, wht
from .decode import dequant_rows
from .layout import Side, is_rotated


def paged_prefill(k_side: Side, v_side: Side, q_bits: np.ndarray, query_start: np.ndarray,
                  k_pool: np.ndarray, v_pool: np.ndarray, block_tables: np.ndarray, seq_lens: np.ndarray,
                  inv_sqrt_d: float, sliding_window: int = 0, k_scale: float = 1.0, v_scale: float = 1.0,
                  seqs=None, rows=None):
    """(out fp32 [T, Hq, hd], out fp64 [T, Hq, hd]); rows of sequences not in `seqs`, and rows not
    in `rows` when it is given (a set of query row indices), stay zero."""
    T, Hq, hd = q_bits.shape
    nkv, bs = k_side.num_kv_heads, k_side.block_size
    G = Hq // nkv
    o64 = np.zeros((T, Hq, hd), dtype=np.float64)
    H = wht.hadamard_f64(hd) if (is_rotated(k_side.fmt) or is_rotated(v_side.fmt)) else None
    q = codecs.bf16_bits_to_f32(q_bits).astype(np.float64)
    scale = np.float64(np.float32(inv_sqrt_d))
    S = len(seq_lens)
    for s in (range(S) if seqs is None else seqs):
        L = int(seq_lens[s])
        q0, q1 = int(query_start[s]), int(query_start[s + 1])
        C = q1 - q0
        if C <= 0:
            continue
        assert C <= L, "a chunk cannot hold more queries than cached positions"
        j = np.arange(L, dtype=np.int64)
        slots = block_tables[s, j // bs].astype(np.int64) * bs + j % bs
        K = dequant_rows(k_pool, k_side, slots, k_scale)          # [L, Hkv, hd]
        V = dequant_rows(v_pool, v_side, slots, v_scale)
        for i in range(C):
            if rows is not None and q0 + i not in rows:
                continue
            p = L - C + i
            j0 = max(0, p + 1 - sliding_window) if sliding_window > 0 else 0
            for h in range(Hq):
                g = h // G
                qv = q[q0 + i, h]
                if is_rotated(k_side.fmt):
                    qv = H @ qv
                sc = (K[j0:p + 1, g, :] @ qv) * scale
                e = np.exp(sc - sc.max())
                o = (e / e.sum()) @ V[j0:p + 1, g, :]
                if is_rotated(v_side.fmt):
                    o = H @ o
                o64[q0 + i, h] = o
    return o64.astype(np.float32), o64
