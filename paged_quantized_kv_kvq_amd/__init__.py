"""Python binding of libkvq (paged quantized KV cache for MI355X / gfx950).

Argument marshalling only: every step of the write and of the decode runs in
the HIP kernels of libkvq.so, reached through its C ABI (include/kvq.h) with
ctypes.  torch supplies device memory and the current HIP stream.  There is
no CPU fallback: without the built library every call raises.

    import paged_quantized_kv_kvq_amd as kvq
    lay = kvq.pool_layout("bf16", "turbo4", block_size=16, num_kv_heads=8, head_dim=128)
    k_pool = kvq.alloc_pool(lay, "k", num_blocks)
    kvq.reshape_and_cache(lay, key, value, k_pool, v_pool, slot_mapping)
    out = kvq.paged_decode(lay, q, k_pool, v_pool, block_tables, seq_lens, inv_sqrt_d,
                           sparse_v_threshold=1e-3)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["FORMATS", "KvqError", "Layout", "load", "pool_layout", "alloc_pool",
           "reshape_and_cache", "paged_decode", "decode_workspace_bytes", "codebook",
           "library_path", "BlockManager", "paged_prefill", "prefill_workspace_bytes", "check_slots",
           "check_tables", "paged_decode_noalloc"]

FORMATS = {"bf16": 0, "fp8": 1, "turbo2": 2, "turbo3": 3, "turbo4": 4, "nvfp4": 5, "turbo8": 8}
_NAMES = {v: k for k, v in FORMATS.items()}
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkvq.so")
_lib = None


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = _lib.kvq_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{what}: {msg} (status {status})")


class Layout(ctypes.Structure):
    """Mirror of struct kvq_layout."""
    _fields_ = [("k_format", ctypes.c_int32), ("v_format", ctypes.c_int32),
                ("block_size", ctypes.c_uint32), ("num_kv_heads", ctypes.c_uint32),
                ("head_dim", ctypes.c_uint32), ("k_rotated", ctypes.c_uint32),
                ("v_rotated", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
                ("k_data_section_bytes", ctypes.c_uint64), ("k_block_stride_bytes", ctypes.c_uint64),
                ("v_data_section_bytes", ctypes.c_uint64), ("v_block_stride_bytes", ctypes.c_uint64)]

    @property
    def k_fmt(self) -> str:
        return _NAMES[self.k_format]

    @property
    def v_fmt(self) -> str:
        return _NAMES[self.v_format]

    def __repr__(self):
        return (f"Layout({self.k_fmt}/{self.v_fmt}, bs={self.block_size}, Hkv={self.num_kv_heads}, "
                f"hd={self.head_dim}, K stride {self.k_block_stride_bytes} B, V stride "
                f"{self.v_block_stride_bytes} B)")


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libkvq.so (built in-tree by ``python -m paged_quantized_kv_kvq_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m paged_quantized_kv_kvq_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, U32, I32, F32, SZ = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.kvq_pool_layout.argtypes = [I32, I32, U32, U32, U32, ctypes.POINTER(Layout)]
    lib.kvq_reshape_and_cache.argtypes = [ctypes.POINTER(Layout), P, P, P, P, P, U32, U32, U32, F32, F32, P]
    lib.kvq_paged_decode.argtypes = [ctypes.POINTER(Layout), P, P, P, P, P, P, U32, U32, U32, F32, U32, U32,
                                     F32, F32, F32, P, ctypes.POINTER(SZ), P]
    lib.kvq_paged_decode_noalloc.argtypes = [ctypes.POINTER(Layout), P, P, P, P, P, P, U32, U32, U32, F32, U32,
                                             U32, F32, F32, F32, P]
    lib.kvq_paged_decode_noalloc.restype = ctypes.c_int
    lib.kvq_paged_prefill.argtypes = [ctypes.POINTER(Layout), P, P, P, P, P, P, P, U32, U32, U32, U32, F32, U32,
                                      U32, F32, F32, P, ctypes.POINTER(SZ), P]
    lib.kvq_paged_prefill.restype = ctypes.c_int
    lib.kvq_codebook.argtypes = [I32, ctypes.POINTER(F32), ctypes.POINTER(F32), ctypes.POINTER(F32),
                                 ctypes.POINTER(U32)]
    U64 = ctypes.c_uint64
    lib.kvq_check_slots.argtypes = [ctypes.POINTER(Layout), P, U32, U64, ctypes.POINTER(U32)]
    lib.kvq_check_tables.argtypes = [ctypes.POINTER(Layout), P, P, P, U32, U32, U32, U64, ctypes.POINTER(U32)]
    lib.kvq_check_slots.restype = ctypes.c_int
    lib.kvq_check_tables.restype = ctypes.c_int
    lib.kvq_status_string.argtypes = [ctypes.c_int]
    lib.kvq_status_string.restype = ctypes.c_char_p
    for f in ("kvq_pool_layout", "kvq_reshape_and_cache", "kvq_paged_decode", "kvq_codebook"):
        getattr(lib, f).restype = ctypes.c_int
    PU32, PI32, PI64 = ctypes.POINTER(U32), ctypes.POINTER(I32), ctypes.POINTER(ctypes.c_int64)
    block_fns = {
        "kvq_blocks_create": [U32, U32, ctypes.POINTER(P)],
        "kvq_blocks_reset": [P],
        "kvq_blocks_num_free": [P, PU32],
        "kvq_blocks_ref_count": [P, U32, PU32],
        "kvq_blocks_seq_new": [P, PU32],
        "kvq_blocks_seq_fork": [P, U32, PU32],
        "kvq_blocks_seq_free": [P, U32],
        "kvq_blocks_seq_len": [P, U32, PU32, PU32],
        "kvq_blocks_append": [P, U32, U32, PI64, PI32, PI32],
        "kvq_blocks_popn": [P, U32, U32, PU32],
        "kvq_blocks_append_many": [P, PU32, PU32, U32, PI64, PI32],
        "kvq_blocks_table": [P, PU32, U32, U32, PI32, PI32],
    }
    for f, args in block_fns.items():
        getattr(lib, f).argtypes = args
        getattr(lib, f).restype = ctypes.c_int
    lib.kvq_blocks_destroy.argtypes = [P]
    lib.kvq_blocks_destroy.restype = None
    _lib = lib
    return lib


def _check(status: int, what: str) -> None:
    if status != 0:
        raise KvqError(status, what)


def _fmt(f) -> int:
    return FORMATS[f] if isinstance(f, str) else int(f)


def pool_layout(k_format, v_format, block_size: int, num_kv_heads: int, head_dim: int) -> Layout:
    lib = load()
    lay = Layout()
    _check(lib.kvq_pool_layout(_fmt(k_format), _fmt(v_format), block_size, num_kv_heads, head_dim,
                               ctypes.byref(lay)), "kvq_pool_layout")
    return lay


def alloc_pool(layout: Layout, side: str, num_blocks: int, device="cuda", fill: Optional[int] = None):
    """uint8 device tensor holding num_blocks blocks of one side's pool."""
    stride = layout.k_block_stride_bytes if side == "k" else layout.v_block_stride_bytes
    if fill is None:
        return torch.empty(num_blocks * stride, dtype=torch.uint8, device=device)
    return torch.full((num_blocks * stride,), fill, dtype=torch.uint8, device=device)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t: torch.Tensor, dtype, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _same_device(*named) -> None:
    devs = {t.device for _, t in named}
    if len(devs) > 1:
        raise ValueError("tensors on different devices: " + ", ".join(f"{n} {t.device}" for n, t in named))


def _rows_of(t: torch.Tensor, name: str, heads: int, head_dim: int) -> None:
    if t.dim() != 3 or t.shape[1] != heads or t.shape[2] != head_dim:
        raise ValueError(f"{name} must be [rows, {heads}, {head_dim}] for this layout, got {tuple(t.shape)}")


def _debug_checks(validate) -> bool:
    """Debug mode: validate index arrays on the host before a launch
    (validate=True, or KVQ_VALIDATE=1 in the environment when None)."""
    if validate is None:
        return os.environ.get("KVQ_VALIDATE", "0") not in ("", "0")
    return bool(validate)


def _pool_blocks(layout: Layout, k_cache: torch.Tensor, v_cache: torch.Tensor) -> int:
    return min(k_cache.numel() // layout.k_block_stride_bytes, v_cache.numel() // layout.v_block_stride_bytes)


def _host(t: torch.Tensor, dtype):
    import numpy as np
    return np.ascontiguousarray(t.detach().to("cpu").numpy(), dtype=dtype)


def check_slots(layout: Layout, slot_mapping: torch.Tensor, num_blocks: int) -> None:
    """kvq_check_slots on a host copy of slot_mapping (raises KvqError naming the token)."""
    import numpy as np
    lib = load()
    sl = _host(slot_mapping, np.int64)
    bad = ctypes.c_uint32(0)
    st = lib.kvq_check_slots(ctypes.byref(layout), sl.ctypes.data, sl.size, num_blocks, ctypes.byref(bad))
    _check(st, f"kvq_check_slots (token {bad.value})")


def check_tables(layout: Layout, block_tables: torch.Tensor, seq_lens: torch.Tensor, num_blocks: int,
                 sliding_window: int = 0, query_start: Optional[torch.Tensor] = None) -> None:
    """kvq_check_tables on host copies (raises KvqError naming the sequence)."""
    import numpy as np
    lib = load()
    bt, ln = _host(block_tables, np.int32), _host(seq_lens, np.int32)
    qs = None if query_start is None else _host(query_start, np.int32)
    if qs is not None and qs.size != ln.size + 1:
        raise ValueError("query_start must hold num_seqs + 1 entries")
    bad = ctypes.c_uint32(0)
    st = lib.kvq_check_tables(ctypes.byref(layout), bt.ctypes.data, ln.ctypes.data,
                              None if qs is None else qs.ctypes.data, bt.shape[1] if bt.ndim == 2 else 0,
                              ln.size, sliding_window, num_blocks, ctypes.byref(bad))
    _check(st, f"kvq_check_tables (sequence {bad.value})")


def _row_stride(t: torch.Tensor, name: str) -> int:
    """Elements between rows of [rows, heads, head_dim] with contiguous heads."""
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name} must be [rows, heads, head_dim] with contiguous heads")
    return t.stride(0)


def reshape_and_cache(layout: Layout, key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, slot_mapping: torch.Tensor, k_scale: float = 1.0,
                      v_scale: float = 1.0, stream=None, validate=None) -> None:
    """Write key/value rows ([T, Hkv, hd] bf16) into the pools at slot_mapping (int64 [T]).
    validate (or KVQ_VALIDATE=1): check the slots on the host first (synchronizes)."""
    lib = load()
    T = key.shape[0]
    if value.shape[0] != T or slot_mapping.numel() != T:
        raise ValueError("key, value and slot_mapping disagree on the number of tokens")
    _rows_of(key, "key", layout.num_kv_heads, layout.head_dim)
    _rows_of(value, "value", layout.num_kv_heads, layout.head_dim)
    _same_device(("key", key), ("value", value), ("k_cache", k_cache), ("v_cache", v_cache),
                 ("slot_mapping", slot_mapping))
    if _debug_checks(validate):
        check_slots(layout, slot_mapping, _pool_blocks(layout, k_cache, v_cache))
    _check(lib.kvq_reshape_and_cache(
        ctypes.byref(layout), _dev(key, torch.bfloat16, "key"), _dev(value, torch.bfloat16, "value"),
        _dev(k_cache, torch.uint8, "k_cache"), _dev(v_cache, torch.uint8, "v_cache"),
        _dev(slot_mapping, torch.int64, "slot_mapping"), T, _row_stride(key, "key"),
        _row_stride(value, "value"), k_scale, v_scale, _stream(stream)), "kvq_reshape_and_cache")


def decode_workspace_bytes(layout: Layout, num_seqs: int, num_q_heads: int, max_blocks_per_seq: int,
                           sliding_window: int = 0, sparse_v_threshold: float = 0.0) -> int:
    lib = load()
    n = ctypes.c_size_t(0)
    _check(lib.kvq_paged_decode(ctypes.byref(layout), None, None, None, None, None, None,
                                max_blocks_per_seq, num_seqs, num_q_heads, 1.0,
                                num_q_heads * layout.head_dim, sliding_window, sparse_v_threshold,
                                1.0, 1.0, None, ctypes.byref(n), None), "kvq_paged_decode (size)")
    return n.value


def paged_decode(layout: Layout, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 block_tables: torch.Tensor, seq_lens: torch.Tensor, inv_sqrt_d: float,
                 sliding_window: int = 0, sparse_v_threshold: float = 0.0, k_scale: float = 1.0,
                 v_scale: float = 1.0, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None, validate=None) -> torch.Tensor:
    """fp32 [S, Hq, hd] attention output for bf16 q [S, Hq, hd].
    validate (or KVQ_VALIDATE=1): check the tables on the host first (synchronizes)."""
    lib = load()
    if q.dim() != 3 or q.shape[2] != layout.head_dim:
        raise ValueError(f"q must be [S, Hq, {layout.head_dim}] for this layout, got {tuple(q.shape)}")
    S, Hq, hd = q.shape
    if q.stride(2) != 1 or q.stride(1) != hd:
        raise ValueError("q must be [S, Hq, head_dim] with contiguous heads")
    if seq_lens.numel() != S:
        raise ValueError(f"seq_lens holds {seq_lens.numel()} entries for {S} sequences")
    _same_device(("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("block_tables", block_tables),
                 ("seq_lens", seq_lens), *((("out", out),) if out is not None else ()),
                 *((("workspace", workspace),) if workspace is not None else ()))
    if block_tables.dim() != 2 or block_tables.shape[0] != S or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32 [S, max_blocks_per_seq]")
    mb = block_tables.shape[1]
    if _debug_checks(validate):
        check_tables(layout, block_tables, seq_lens, _pool_blocks(layout, k_cache, v_cache), sliding_window)
    if out is None:
        out = torch.empty((S, Hq, hd), dtype=torch.float32, device=q.device)
    elif not out.is_contiguous() or tuple(out.shape) != (S, Hq, hd):
        raise ValueError("out must be contiguous fp32 [S, Hq, head_dim]")
    need = decode_workspace_bytes(layout, S, Hq, mb, sliding_window, sparse_v_threshold)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    n = ctypes.c_size_t(workspace.numel())
    _check(lib.kvq_paged_decode(
        ctypes.byref(layout), _dev(q, torch.bfloat16, "q"), _dev(k_cache, torch.uint8, "k_cache"),
        _dev(v_cache, torch.uint8, "v_cache"), _dev(out, torch.float32, "out"),
        _dev(block_tables, torch.int32, "block_tables"), _dev(seq_lens, torch.int32, "seq_lens"),
        mb, S, Hq, inv_sqrt_d, q.stride(0), sliding_window, sparse_v_threshold, k_scale, v_scale,
        _dev(workspace, torch.uint8, "workspace"), ctypes.byref(n), _stream(stream)), "kvq_paged_decode")
    return out


def paged_decode_noalloc(layout: Layout, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         block_tables: torch.Tensor, seq_lens: torch.Tensor, inv_sqrt_d: float,
                         sliding_window: int = 0, sparse_v_threshold: float = 0.0, k_scale: float = 1.0,
                         v_scale: float = 1.0, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """paged_decode through kvq_paged_decode_noalloc: no workspace, the library's
    own per-GPU scratch (pass `out` to allocate nothing at all)."""
    lib = load()
    if q.dim() != 3 or q.shape[2] != layout.head_dim:
        raise ValueError(f"q must be [S, Hq, {layout.head_dim}] for this layout, got {tuple(q.shape)}")
    S, Hq, hd = q.shape
    if q.stride(2) != 1 or q.stride(1) != hd:
        raise ValueError("q must be [S, Hq, head_dim] with contiguous heads")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32 [S, max_blocks_per_seq]")
    if seq_lens.numel() != S:
        raise ValueError(f"seq_lens holds {seq_lens.numel()} entries for {S} sequences")
    if out is None:
        out = torch.empty((S, Hq, hd), dtype=torch.float32, device=q.device)
    elif not out.is_contiguous() or tuple(out.shape) != (S, Hq, hd):
        raise ValueError("out must be contiguous fp32 [S, Hq, head_dim]")
    _same_device(("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("block_tables", block_tables),
                 ("seq_lens", seq_lens), ("out", out))
    _check(lib.kvq_paged_decode_noalloc(
        ctypes.byref(layout), _dev(q, torch.bfloat16, "q"), _dev(k_cache, torch.uint8, "k_cache"),
        _dev(v_cache, torch.uint8, "v_cache"), _dev(out, torch.float32, "out"),
        _dev(block_tables, torch.int32, "block_tables"), _dev(seq_lens, torch.int32, "seq_lens"),
        block_tables.shape[1], S, Hq, inv_sqrt_d, q.stride(0), sliding_window, sparse_v_threshold, k_scale,
        v_scale, _stream(stream)), "kvq_paged_decode_noalloc")
    return out


def prefill_workspace_bytes(layout: Layout, num_seqs: int, num_q_heads: int, max_blocks_per_seq: int,
                            max_query_len: int, sliding_window: int = 0) -> int:
    lib = load()
    n = ctypes.c_size_t(0)
    _check(lib.kvq_paged_prefill(ctypes.byref(layout), None, None, None, None, None, None, None,
                                 max_blocks_per_seq, num_seqs, num_q_heads, max_query_len, 1.0,
                                 num_q_heads * layout.head_dim, sliding_window, 1.0, 1.0, None, ctypes.byref(n),
                                 None), "kvq_paged_prefill (size)")
    return n.value


def paged_prefill(layout: Layout, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                  block_tables: torch.Tensor, seq_lens: torch.Tensor, query_start: torch.Tensor, max_query_len: int,
                  inv_sqrt_d: float, sliding_window: int = 0, k_scale: float = 1.0, v_scale: float = 1.0,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  stream=None, validate=None) -> torch.Tensor:
    """fp32 [T, Hq, hd] chunked-prefill attention output for bf16 q [T, Hq, hd]
    (sequence s's queries are rows query_start[s] .. query_start[s + 1] - 1)."""
    lib = load()
    if q.dim() != 3 or q.shape[2] != layout.head_dim:
        raise ValueError(f"q must be [T, Hq, {layout.head_dim}] for this layout, got {tuple(q.shape)}")
    T, Hq, hd = q.shape
    S = seq_lens.numel()
    if q.stride(2) != 1 or q.stride(1) != hd:
        raise ValueError("q must be [T, Hq, head_dim] with contiguous heads")
    _same_device(("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("block_tables", block_tables),
                 ("seq_lens", seq_lens), ("query_start", query_start),
                 *((("out", out),) if out is not None else ()),
                 *((("workspace", workspace),) if workspace is not None else ()))
    if block_tables.dim() != 2 or block_tables.shape[0] != S or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32 [S, max_blocks_per_seq]")
    if query_start.numel() != S + 1:
        raise ValueError("query_start must hold num_seqs + 1 entries")
    mb = block_tables.shape[1]
    if _debug_checks(validate):
        check_tables(layout, block_tables, seq_lens, _pool_blocks(layout, k_cache, v_cache), sliding_window,
                     query_start)
    if out is None:
        out = torch.empty((T, Hq, hd), dtype=torch.float32, device=q.device)
    elif not out.is_contiguous() or tuple(out.shape) != (T, Hq, hd):
        raise ValueError("out must be contiguous fp32 [T, Hq, head_dim]")
    need = prefill_workspace_bytes(layout, S, Hq, mb, max_query_len, sliding_window)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    n = ctypes.c_size_t(workspace.numel())
    _check(lib.kvq_paged_prefill(
        ctypes.byref(layout), _dev(q, torch.bfloat16, "q"), _dev(k_cache, torch.uint8, "k_cache"),
        _dev(v_cache, torch.uint8, "v_cache"), _dev(out, torch.float32, "out"),
        _dev(block_tables, torch.int32, "block_tables"), _dev(seq_lens, torch.int32, "seq_lens"),
        _dev(query_start, torch.int32, "query_start"), mb, S, Hq, max_query_len, inv_sqrt_d, q.stride(0),
        sliding_window, k_scale, v_scale, _dev(workspace, torch.uint8, "workspace"), ctypes.byref(n),
        _stream(stream)), "kvq_paged_prefill")
    return out


def codebook(fmt) -> dict:
    """The library's fp32 Lloyd-Max tables for a turbo format."""
    lib = load()
    c = (ctypes.c_float * 16)()
    t = (ctypes.c_float * 16)()
    inv = ctypes.c_float()
    L = ctypes.c_uint32()
    _check(lib.kvq_codebook(_fmt(fmt), c, t, ctypes.byref(inv), ctypes.byref(L)), "kvq_codebook")
    n = L.value
    import numpy as np
    return {"levels": n, "centroids": np.array(c[:n], dtype=np.float32),
            "thresholds": np.array(t[:n], dtype=np.float32), "inv_cmax": np.float32(inv.value)}


class BlockManager:
    """The library's host block manager (include/kvq_blocks.h), argument
    marshalling only.  Block ids index every pool built for the same
    num_blocks (all layers, K and V)."""

    def __init__(self, num_blocks: int, block_size: int):
        self._lib = load()
        h = ctypes.c_void_p()
        _check(self._lib.kvq_blocks_create(num_blocks, block_size, ctypes.byref(h)), "kvq_blocks_create")
        self._h = h
        self.num_blocks, self.block_size = num_blocks, block_size

    def __del__(self):
        if getattr(self, "_h", None) is not None:
            self._lib.kvq_blocks_destroy(self._h)
            self._h = None

    def _u32(self, fn, *args) -> int:
        out = ctypes.c_uint32()
        _check(getattr(self._lib, fn)(self._h, *args, ctypes.byref(out)), fn)
        return out.value

    def reset(self) -> None:
        _check(self._lib.kvq_blocks_reset(self._h), "kvq_blocks_reset")

    def num_free(self) -> int:
        return self._u32("kvq_blocks_num_free")

    def ref_count(self, block: int) -> int:
        return self._u32("kvq_blocks_ref_count", block)

    def seq_new(self) -> int:
        return self._u32("kvq_blocks_seq_new")

    def seq_fork(self, parent: int) -> int:
        return self._u32("kvq_blocks_seq_fork", parent)

    def seq_free(self, seq: int) -> None:
        _check(self._lib.kvq_blocks_seq_free(self._h, seq), "kvq_blocks_seq_free")

    def seq_len(self, seq: int):
        n, b = ctypes.c_uint32(), ctypes.c_uint32()
        _check(self._lib.kvq_blocks_seq_len(self._h, seq, ctypes.byref(n), ctypes.byref(b)), "kvq_blocks_seq_len")
        return n.value, b.value

    def append(self, seq: int, n: int):
        """(slots int64 numpy [n], (cow_src, cow_dst))."""
        import numpy as np
        slots = np.zeros(max(n, 1), dtype=np.int64)
        src, dst = ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.kvq_blocks_append(self._h, seq, n, slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                           ctypes.byref(src), ctypes.byref(dst)), "kvq_blocks_append")
        return slots[:n], (src.value, dst.value)

    def append_many(self, seqs, counts):
        """(slots int64 numpy [sum(counts)], cow int32 numpy [len(seqs), 2])."""
        import numpy as np
        ids = np.ascontiguousarray(seqs, dtype=np.uint32)
        cnt = np.ascontiguousarray(counts, dtype=np.uint32)
        slots = np.zeros(max(int(cnt.sum()), 1), dtype=np.int64)
        cow = np.zeros((max(len(ids), 1), 2), dtype=np.int32)
        PU = ctypes.POINTER(ctypes.c_uint32)
        _check(self._lib.kvq_blocks_append_many(self._h, ids.ctypes.data_as(PU), cnt.ctypes.data_as(PU), len(ids),
                                                slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                                cow.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))),
               "kvq_blocks_append_many")
        return slots[:int(cnt.sum())], cow[:len(ids)]

    def popn(self, seq: int, n: int) -> int:
        return self._u32("kvq_blocks_popn", seq, n)

    def table(self, seqs, max_blocks: int):
        """(block_tables int32 numpy [len(seqs), max_blocks], seq_lens int32 numpy)."""
        import numpy as np
        ids = np.ascontiguousarray(seqs, dtype=np.uint32)
        bt = np.zeros((len(ids), max_blocks), dtype=np.int32)
        lens = np.zeros(len(ids), dtype=np.int32)
        P32 = ctypes.POINTER(ctypes.c_int32)
        _check(self._lib.kvq_blocks_table(self._h, ids.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)), len(ids),
                                          max_blocks, bt.ctypes.data_as(P32), lens.ctypes.data_as(P32)),
               "kvq_blocks_table")
        return bt, lens
