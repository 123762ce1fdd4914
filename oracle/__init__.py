"""CPU oracle for the paged quantized KV cache: test infrastructure only.

This package is a plain, slow, obviously-correct CPU statement of what the
cache write and the paged decode compute.  It exists so that the GPU library
can be checked against something other than itself.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product path (the HIP library and its Python binding) never
does, and it shares no code, table or constant generator with it.

Precision: quantization runs in fp32 with a fixed operation order (so that
codes can be compared bit for bit); attention runs in fp64 over the
dequantized values.

Sources (web pages, cited by title and item):
  * "spark_runtime/kv_cache.rs" (atlas docs): the ``KvCacheDtype`` catalogue
    (bf16, fp8 with a per-tensor scale, turbo2/3/4 = Walsh-Hadamard rotation
    + Lloyd-Max Gaussian codebook + one FP8 scale per 16 elements, the
    asymmetric K/V pairs), ``is_wht_rotated`` (WHT(Q) / iWHT(out)
    bookends) and ``block_bytes_dims`` (bytes per block per side).
  * "metrale_model_layers/layers/ops/kv_cache_bf16k_turbov.rs": module
    invariants (pool layout ``[num_blocks, block_size, num_kv_heads,
    head_dim]``, V code section followed by its scales, separate K/V byte
    strides) and the launcher argument lists (slot_mapping, block_tables,
    seq_lens, inv_sqrt_d, sliding_window, sparse-V skip threshold).
  * "combs_models/kv.rs": GQA ``repeat_kv``, the reference attention path
    (scores * scale, softmax, P @ V; decode needs no mask), the paged
    gather, and the contiguous cache kept as the cross-validation baseline.

Readings of points the pages leave open are listed in each function's
docstring (and collected in the design notes).

Parity pins: every function here is checked by ``tests/test_oracle_*.py``
against values that do not come from the oracle itself (library codecs,
closed forms, textbook Lloyd-Max tables, brute force).  Parity unpinned:
the per-16 scale rule (absmax / c_max), the bf16 re-round after the
rotation, code numbering / bit packing order, and the exact sparse-V rule
(normalized global softmax weight > threshold).  No page fixes them; they
are readings shared by both implementations and bit-exactness there is
between two independent implementations only.
"""
from . import codecs, codebook, wht, layout, write, decode  # noqa: F401
