"""Stage a workload in GPU memory: inputs drawn on the device, pools prefilled.

The cache contents that exist before a decode step are written through the
library's own write (kvq_reshape_and_cache), sequence by sequence.  The
positions of the timed step (the last `write_tail` of every sequence) are
held back and returned as one batch, in a seeded shuffled order, so a caller
can write them (scattered slot_mapping) and then decode.

Unused blocks and the page-table entries past a sequence's end point at a
poison block (every byte 0x7F: NaN in E4M3, a huge bf16), so a stray read
shows up as a non-finite output instead of silently passing.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterable, Optional, Tuple

import numpy as np
import torch

from . import Workload, block_tables, fp8_scale_from_absmax, kv_values, queries, seq_lens, slots_for, \
    write_order

POISON = 0x7F


@dataclasses.dataclass
class Staged:
    w: Workload
    layout: object
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    num_blocks: int                 # blocks in use (the poison block is id num_blocks)
    lens: np.ndarray                # int32 [S]
    bt: np.ndarray                  # int32 [S, mb], -1 past the end
    bt_dev: torch.Tensor            # same, -1 replaced by the poison block id
    lens_dev: torch.Tensor
    q: torch.Tensor                 # bf16 [S, Hq, hd]
    k_scale: float
    v_scale: float
    tail_key: torch.Tensor          # bf16 [N, Hkv, hd]: the held-back positions
    tail_value: torch.Tensor
    tail_slots: torch.Tensor        # int64 [N]
    tail_index: np.ndarray          # [N, 2]: (sequence, position) of each row
    host_kv: Dict[int, Tuple[np.ndarray, np.ndarray]]  # seq -> (K bits, V bits) uint16 [L, Hkv, hd]


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def stage(w: Workload, kvq, device="cuda", keep_host: Iterable[int] = (), write_tail: Optional[int] = None,
          log=None) -> Staged:
    keep_host = set(int(s) for s in keep_host)
    tail = w.write_tail if write_tail is None else write_tail
    lens = seq_lens(w)
    bt, nb = block_tables(w, lens)
    lay = kvq.pool_layout(w.k_format, w.v_format, w.block_size, w.num_kv_heads, w.head_dim)
    k_pool = kvq.alloc_pool(lay, "k", nb + 1, device, fill=POISON)
    v_pool = kvq.alloc_pool(lay, "v", nb + 1, device, fill=POISON)
    bt_fix = np.where(bt < 0, nb, bt).astype(np.int32)

    k_scale = v_scale = 1.0
    if "fp8" in (w.k_format, w.v_format):
        kmax = vmax = 0.0
        for s in range(w.num_seqs):
            L = int(lens[s])
            if L == 0:
                continue
            if w.k_format == "fp8":
                kmax = max(kmax, float(kv_values(w, "k", s, L, device).abs().max().float()))
            if w.v_format == "fp8":
                vmax = max(vmax, float(kv_values(w, "v", s, L, device).abs().max().float()))
        k_scale = fp8_scale_from_absmax(kmax) if kmax > 0 else 1.0
        v_scale = fp8_scale_from_absmax(vmax) if vmax > 0 else 1.0

    host_kv = {}
    tk, tv, ts, ti = [], [], [], []
    for s in range(w.num_seqs):
        L = int(lens[s])
        if L == 0:
            if s in keep_host:
                z = np.zeros((0, w.num_kv_heads, w.head_dim), np.uint16)
                host_kv[s] = (z, z)
            continue
        K = kv_values(w, "k", s, L, device)
        V = kv_values(w, "v", s, L, device)
        if s in keep_host:
            host_kv[s] = (_bits(K), _bits(V))
        pre = max(0, L - tail)
        if pre:
            slots = torch.as_tensor(slots_for(w, bt, s, np.arange(pre)), device=device)
            kvq.reshape_and_cache(lay, K[:pre], V[:pre], k_pool, v_pool, slots, k_scale, v_scale)
        if pre < L:
            pos = np.arange(pre, L)
            tk.append(K[pre:])
            tv.append(V[pre:])
            ts.append(slots_for(w, bt, s, pos))
            ti.append(np.stack([np.full(len(pos), s), pos], 1))
        if log and s % 16 == 15:
            log(f"staged {s + 1}/{w.num_seqs} sequences")
    if tk:
        order = write_order(w, sum(len(x) for x in ts))
        o = torch.as_tensor(order, device=device)
        tail_key = torch.cat(tk)[o].contiguous()
        tail_value = torch.cat(tv)[o].contiguous()
        tail_slots = torch.as_tensor(np.concatenate(ts)[order], device=device)
        tail_index = np.concatenate(ti)[order]
    else:
        e = torch.empty((0, w.num_kv_heads, w.head_dim), dtype=torch.bfloat16, device=device)
        tail_key, tail_value = e, e.clone()
        tail_slots = torch.empty(0, dtype=torch.int64, device=device)
        tail_index = np.zeros((0, 2), np.int64)
    torch.cuda.synchronize()
    return Staged(w, lay, k_pool, v_pool, nb, lens, bt, torch.as_tensor(bt_fix, device=device),
                  torch.as_tensor(lens, device=device), queries(w, device), k_scale, v_scale,
                  tail_key, tail_value, tail_slots, tail_index, host_kv)
