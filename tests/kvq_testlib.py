"""Helpers shared by the GPU parity tests: the oracle's side of a staged
workload and the comparison rules.

Bars (from the benchmark spec of the method): slots, packed codes and scale
bytes bit-exact; decode outputs within max-abs 2e-3 and relative L2 1e-3 of
the fp64 oracle.  With a sparse-V threshold, positions whose weight lies
within 1e-4 * thr of the threshold may be decided either way by an fp32
implementation; each output element's max-abs bound grows by what those
positions contribute (computed by the oracle), and rows holding any such
position are left out of the relative-L2 sum.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

from oracle import decode as odecode
from oracle import layout as olayout
from oracle import write as owrite

MAX_ABS = 2e-3
REL_L2 = 1e-3
POISON = 0x7F


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class OracleCache:
    """Oracle pools holding only the sampled sequences' blocks (renumbered)."""

    def __init__(self, st, seqs, from_window=False):
        w = st.w
        self.w, self.seqs = w, list(seqs)
        self.ks, self.vs = olayout.pool_layout(w.k_format, w.v_format, w.block_size, w.num_kv_heads, w.head_dim)
        bs = w.block_size
        self.remap = {}
        self.first_pos = {}
        for s in self.seqs:
            L = int(st.lens[s])
            start = 0
            if from_window and w.sliding_window and L > w.sliding_window:
                start = (L - w.sliding_window) // bs * bs
            self.first_pos[s] = start
            for b in st.bt[s, start // bs:(L + bs - 1) // bs]:
                self.remap.setdefault(int(b), len(self.remap))
        n = len(self.remap) + 1
        self.kp = np.full(n * self.ks.block_stride_bytes, POISON, np.uint8)
        self.vp = np.full(n * self.vs.block_stride_bytes, POISON, np.uint8)
        self.bt = np.full_like(st.bt, -1)
        for s in self.seqs:
            L = int(st.lens[s])
            nbk = (L + bs - 1) // bs
            for i in range(self.first_pos[s] // bs, nbk):
                self.bt[s, i] = self.remap[int(st.bt[s, i])]
            if L == 0:
                continue
            K, V = st.host_kv[s]
            pos = np.arange(self.first_pos[s], L)
            slots = self.bt[s, pos // bs].astype(np.int64) * bs + pos % bs
            owrite.reshape_and_cache(self.ks, self.vs, K[pos], V[pos], self.kp, self.vp, slots,
                                     st.k_scale, st.v_scale)

    def compare_pools(self, st):
        """GPU pool bytes of every sampled block == the oracle's (bit-exact)."""
        bad = []
        for side, gp, op in (("k", st.k_pool, self.kp), ("v", st.v_pool, self.vp)):
            stride = (self.ks if side == "k" else self.vs).block_stride_bytes
            ids = np.array(sorted(self.remap), dtype=np.int64)
            new = np.array([self.remap[i] for i in ids], dtype=np.int64)
            idx = (ids[:, None] * stride + np.arange(stride)[None, :]).ravel()
            g = gp[torch.as_tensor(idx, device=gp.device)].cpu().numpy().reshape(len(ids), stride)
            o = op.reshape(-1, stride)[new]
            if not np.array_equal(g, o):
                diff = np.argwhere(g != o)
                bad.append((side, len(diff), diff[:5].tolist()))
        assert not bad, f"pool bytes differ from the oracle: {bad}"

    def decode(self, st, inv_sqrt_d):
        w = self.w
        q = st.q.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return odecode.paged_decode(self.ks, self.vs, q, self.kp, self.vp, self.bt, st.lens, inv_sqrt_d,
                                    w.sliding_window, w.sparse_v_threshold, st.k_scale, st.v_scale,
                                    seqs=self.seqs, detail=True)


def check_decode(out_gpu: np.ndarray, ref, seqs, label=""):
    out, o64, band, n_amb = ref
    rows = np.asarray(seqs)
    g = out_gpu[rows].astype(np.float64)
    r = o64[rows]
    assert np.all(np.isfinite(g)), f"{label}: non-finite output"
    err = np.abs(g - r)
    lim = MAX_ABS + band[rows]
    worst = float((err - lim).max()) if err.size else -1.0
    assert np.all(err <= lim), f"{label}: max-abs error {err.max():.3e} exceeds bound (excess {worst:.3e})"
    clean = (n_amb[rows] == 0)
    num = np.sqrt(((g - r) ** 2)[clean].sum())
    den = np.sqrt((r ** 2)[clean].sum())
    rel = num / den if den > 0 else 0.0
    assert rel <= REL_L2, f"{label}: relative L2 error {rel:.3e} > {REL_L2}"
    return float(err.max()) if err.size else 0.0, float(rel), int(n_amb[rows].sum())


def timed(msg):
    class _T:
        def __enter__(self):
            self.t = time.time()
            say(f"[start] {msg}")
            return self

        def __exit__(self, *a):
            say(f"[done ] {msg} ({time.time() - self.t:.1f}s)")
    return _T()
