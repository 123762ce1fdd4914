"""Seeded synthetic inputs for the paged KV-cache write and paged decode.

This module is the one piece that both the CPU oracle and the GPU path use.
It only *makes inputs*: sequence lengths, page placement, slot mappings,
query/key/value tensors and the per-tensor fp8 scales the caller hands to the
write.  It holds none of the cache formats' arithmetic (no rotation, no
codebook, no fp8 encoding, no attention).

Every random draw comes from its own seeded stream, keyed by
``(workload id, stream id, sequence)``, so any one sequence can be rebuilt
alone.  Values are drawn in fp32 and rounded to bf16 by torch's own
conversion.  Large tensors are drawn with torch generators on the device
that will consume them; the oracle gets host copies of exactly those bits.

Workloads (shapes and value mixes follow the decode configurations the
paged-attention pages describe: GQA with 32/8 heads, head_dim 128, block
size 16, long contexts, sliding window, sparse-V threshold 1e-3):

  1  tiny   bf16 / bf16, 1 seq x 256, Hq 4, Hkv 2, hd 64, 32-block pool
  2         bf16 / turbo4, 64 seqs, L ~ U{1024..8192}, Hq 32, Hkv 8, hd 128, thr 1e-3
  3         fp8 / turbo2, 128 seqs x 32768, Hq 32, Hkv 8, hd 128
  4         turbo3 / turbo3, 16 seqs x 65536, Hq 16, Hkv 4, hd 256, W 4096, thr 1e-3,
            Student-t(5) values
  5         turbo4 / turbo3, write 8192 tokens (last 256 of 32 seqs, shuffled),
            then decode 32 seqs, L ~ U{4096..16384}, Hq 64, Hkv 8, hd 128, bs 32
  6         turbo4 / turbo8, 64 seqs, L ~ U{4096..16384}, Hq 32, Hkv 8, hd 128
  7         turbo8 / turbo8, the same sequences and shapes as 6 (the symmetric pairing
            the asymmetric one is measured against)
  8         nvfp4 / nvfp4, the same sequences and shapes as 6
  9         chunked prefill, bf16 / turbo4: 16 seqs, L ~ U{2048..8192}, the last 512 positions of
            each written by the step and attended by 512 queries, Hq 32, Hkv 8, hd 128
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

FORMATS = ("bf16", "fp8", "turbo2", "turbo3", "turbo4", "turbo8", "nvfp4")

# stream ids
_S_LENS, _S_PERM, _S_OUTLIER, _S_Q, _S_K, _S_V, _S_ORDER = range(7)


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    k_format: str
    v_format: str
    seq_len: Tuple[int, int]          # inclusive range; lo == hi for a fixed length
    dist: str = "normal"              # "normal" | "student_t5"
    outliers: bool = False            # 4 channels per kv head x20 on K and V
    sparse_v_threshold: float = 0.0
    sliding_window: int = 0
    pool_blocks: Optional[int] = None  # None: exactly the blocks the sequences need
    write_tail: int = 1               # positions per sequence written by the timed step
    fixed_lens: Optional[Tuple[int, ...]] = None  # explicit per-sequence lengths
    seed_wid: Optional[int] = None    # draw every stream as this workload does (same sequences, other formats)
    prefill: bool = False             # the step is a chunked prefill of the write_tail positions

    @property
    def seed_id(self) -> int:
        return self.wid if self.seed_wid is None else self.seed_wid

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "tiny-bf16", 1, 4, 2, 64, 16, "bf16", "bf16", (256, 256), pool_blocks=32),
    2: Workload(2, "bf16k-turbo4v", 64, 32, 8, 128, 16, "bf16", "turbo4", (1024, 8192),
                outliers=True, sparse_v_threshold=1e-3),
    3: Workload(3, "fp8k-turbo2v", 128, 32, 8, 128, 16, "fp8", "turbo2", (32768, 32768),
                outliers=True),
    4: Workload(4, "turbo3-window", 16, 16, 4, 256, 16, "turbo3", "turbo3", (65536, 65536),
                dist="student_t5", sparse_v_threshold=1e-3, sliding_window=4096),
    5: Workload(5, "turbo4k-turbo3v-write", 32, 64, 8, 128, 32, "turbo4", "turbo3",
                (4096, 16384), write_tail=256),
    6: Workload(6, "turbo4k-turbo8v", 64, 32, 8, 128, 16, "turbo4", "turbo8", (4096, 16384),
                outliers=True),
    7: Workload(7, "turbo8-turbo8", 64, 32, 8, 128, 16, "turbo8", "turbo8", (4096, 16384),
                outliers=True, seed_wid=6),
    8: Workload(8, "nvfp4-nvfp4", 64, 32, 8, 128, 16, "nvfp4", "nvfp4", (4096, 16384),
                outliers=True, seed_wid=6),
    9: Workload(9, "prefill-bf16k-turbo4v", 16, 32, 8, 128, 16, "bf16", "turbo4", (2048, 8192),
                outliers=True, write_tail=512, prefill=True),
}


def _seed(wid: int, stream: int, idx: int) -> int:
    return (wid * 1_000_003 + stream) * 10_000_019 + idx


def _gen(wid: int, stream: int, idx: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(wid, stream, idx))
    return g


def seq_lens(w: Workload) -> np.ndarray:
    if w.fixed_lens is not None:
        return np.asarray(w.fixed_lens, dtype=np.int32)
    lo, hi = w.seq_len
    if lo == hi:
        return np.full(w.num_seqs, lo, dtype=np.int32)
    g = _gen(w.seed_id, _S_LENS, 0, "cpu")
    return torch.randint(lo, hi + 1, (w.num_seqs,), generator=g).numpy().astype(np.int32)


def block_tables(w: Workload, lens: np.ndarray, max_blocks_per_seq: Optional[int] = None):
    """Pages for every sequence, drawn from one shuffled shared pool.

    Returns (block_tables int32 [S, max_blocks_per_seq], num_blocks).  Entries
    past a sequence's last page are -1 and never read.
    """
    bs = w.block_size
    need = [(int(L) + bs - 1) // bs for L in lens]
    total = sum(need)
    num_blocks = total if w.pool_blocks is None else max(w.pool_blocks, total)
    g = _gen(w.seed_id, _S_PERM, 0, "cpu")
    perm = torch.randperm(num_blocks, generator=g).numpy().astype(np.int32)
    longest = max([int(x) for x in lens] + [w.seq_len[1]])
    mb = max_blocks_per_seq or max(1, (longest + bs - 1) // bs)
    bt = np.full((len(lens), mb), -1, dtype=np.int32)
    o = 0
    for s, n in enumerate(need):
        bt[s, :n] = perm[o:o + n]
        o += n
    return bt, num_blocks


def outlier_channels(w: Workload) -> np.ndarray:
    """4 distinct channels per kv head, fixed for the whole workload."""
    g = _gen(w.seed_id, _S_OUTLIER, 0, "cpu")
    ch = np.stack([torch.randperm(w.head_dim, generator=g)[:4].numpy()
                   for _ in range(w.num_kv_heads)])
    return ch.astype(np.int64)


def _draw(w: Workload, stream: int, idx: int, shape, device) -> torch.Tensor:
    g = _gen(w.seed_id, stream, idx, device)
    if w.dist == "normal":
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if w.dist == "student_t5":
        # t_5 = Z / sqrt(chi2_5 / 5), chi2_5 a sum of 5 squared normals; scaled by
        # sqrt(3/5) to unit variance.
        z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        c = torch.zeros(shape, device=device, dtype=torch.float32)
        for _ in range(5):
            c += torch.randn(shape, generator=g, device=device, dtype=torch.float32) ** 2
        return z / torch.sqrt(c / 5.0) * math.sqrt(3.0 / 5.0)
    raise ValueError(w.dist)


def kv_values(w: Workload, side: str, seq: int, length: int, device="cpu") -> torch.Tensor:
    """bf16 [length, Hkv, hd] for positions 0..length-1 of one sequence."""
    stream = _S_K if side == "k" else _S_V
    x = _draw(w, stream, seq, (length, w.num_kv_heads, w.head_dim), device)
    if w.outliers:
        ch = torch.as_tensor(outlier_channels(w), device=device)
        mult = torch.ones(w.num_kv_heads, w.head_dim, device=device)
        mult.scatter_(1, ch, 20.0)
        x = x * mult
    return x.to(torch.bfloat16)


def queries(w: Workload, device="cpu") -> torch.Tensor:
    """bf16 [S, Hq, hd], N(0,1), no outliers."""
    g = _gen(w.seed_id, _S_Q, 0, device)
    x = torch.randn((w.num_seqs, w.num_q_heads, w.head_dim), generator=g, device=device,
                    dtype=torch.float32)
    return x.to(torch.bfloat16)


def prefill_queries(w: Workload, num_rows: int, device="cpu") -> torch.Tensor:
    """bf16 [num_rows, Hq, hd], N(0,1): the query rows of a chunked prefill."""
    g = _gen(w.seed_id, _S_Q, 1, device)
    x = torch.randn((num_rows, w.num_q_heads, w.head_dim), generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16)


def fp8_scale_from_absmax(absmax: float) -> float:
    """Per-tensor fp8 scale chosen by the caller: absmax / 448, in fp32."""
    return float(np.float32(np.float32(absmax) / np.float32(448.0)))


def slots_for(w: Workload, bt: np.ndarray, seq: int, positions: np.ndarray) -> np.ndarray:
    """slot = page * block_size + offset for the given positions of one sequence."""
    bs = w.block_size
    pages = bt[seq, positions // bs].astype(np.int64)
    return pages * bs + (positions % bs)


def write_order(w: Workload, n: int) -> np.ndarray:
    """Seeded shuffle of the timed write batch (scattered slot_mapping)."""
    g = _gen(w.seed_id, _S_ORDER, 0, "cpu")
    return torch.randperm(n, generator=g).numpy()


def inv_sqrt_d(head_dim: int) -> float:
    return float(np.float32(1.0 / math.sqrt(head_dim)))


@dataclasses.dataclass
class Case:
    """A fully materialised workload: every input both sides consume."""
    w: Workload
    lens: np.ndarray                  # int32 [S]
    bt: np.ndarray                    # int32 [S, max_blocks]
    num_blocks: int
    q: torch.Tensor                   # bf16 [S, Hq, hd]
    k: list                           # per seq bf16 [L, Hkv, hd]
    v: list
    k_scale: float
    v_scale: float


def make_case(w: Workload, device="cpu", seqs: Optional[Sequence[int]] = None) -> Case:
    """Materialise a workload (all sequences, or the listed ones) on `device`.

    fp8 scales are absmax/448 over the tensors generated here (the whole
    workload when `seqs` is None).
    """
    lens = seq_lens(w)
    bt, nb = block_tables(w, lens)
    idx = range(w.num_seqs) if seqs is None else seqs
    k = [kv_values(w, "k", s, int(lens[s]), device) for s in idx]
    v = [kv_values(w, "v", s, int(lens[s]), device) for s in idx]
    kmax = max((float(t.abs().max().float()) for t in k if t.numel()), default=1.0)
    vmax = max((float(t.abs().max().float()) for t in v if t.numel()), default=1.0)
    return Case(w, lens, bt, nb, queries(w, device), k, v,
                fp8_scale_from_absmax(kmax), fp8_scale_from_absmax(vmax))


def small(wid: int, *, lens, num_q_heads, num_kv_heads, head_dim, block_size, k_format, v_format,
          dist="normal", outliers=True, sparse_v_threshold=0.0, sliding_window=0,
          extra_blocks=3) -> Workload:
    """A test-sized workload with explicit sequence lengths (ragged, empty, ...)."""
    need = sum((int(L) + block_size - 1) // block_size for L in lens)
    return Workload(wid, f"small-{wid}", len(lens), num_q_heads, num_kv_heads, head_dim, block_size,
                    k_format, v_format, (max(lens), max(lens)), dist=dist, outliers=outliers,
                    sparse_v_threshold=sparse_v_threshold, sliding_window=sliding_window,
                    pool_blocks=need + extra_blocks, fixed_lens=tuple(int(L) for L in lens))
