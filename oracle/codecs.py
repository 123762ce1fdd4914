"""bf16, FP8 E4M3 and FP4 E2M1 codecs, written from the formats' definitions.

"spark_runtime/kv_cache.rs", ``KvCacheDtype::Fp8`` ("1 byte per element (FP8
E4M3 with per-tensor scale)"), the turbo scales ("FP8 per-group scales") and
``KvCacheDtype::Nvfp4`` (4-bit E2M1 values packed two to a byte).

Readings (the pages name the format only):
  * E4M3 is the OCP "E4M3FN" variant: 1 sign, 4 exponent bits (bias 7),
    3 mantissa bits, no infinities, 0x7F / 0xFF are NaN, largest finite 448,
    subnormals m/8 * 2^-6 kept.
  * Encoding clamps to [-448, 448] first, then rounds to the nearest
    representable value, ties to the even mantissa.  The sign of -0 is kept.
  * bf16 rounding is round-to-nearest-even on the fp32 value.
  * E2M1 is the OCP FP4 element type: 1 sign, 2 exponent bits (bias 1),
    1 mantissa bit, no infinities or NaN; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4,
    6 (codes 0..7, the sign in bit 3).  Encoding saturates to +-6, then
    rounds to the nearest value, ties to the even mantissa; the sign of -0
    is kept.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns, round to nearest, ties to even.

    bf16 keeps the top 16 bits of an fp32 pattern.  The two candidates are the
    truncated pattern and the next one up (in magnitude); the discarded low 16
    bits decide: above half goes up, below half stays, exactly half goes to the
    candidate whose last kept bit is 0.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    low = u & np.uint32(0xFFFF)
    down = u >> np.uint32(16)
    up = down + np.uint32(1)
    half = np.uint32(0x8000)
    go_up = (low > half) | ((low == half) & ((down & np.uint32(1)) == 1))
    out = np.where(go_up, up, down).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out = np.where(nan, ((u >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16), out)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 value, returned as fp32."""
    return bf16_bits_to_f32(bf16_round_bits(x))


def _e4m3_table() -> np.ndarray:
    """Value of every E4M3FN byte (float64; NaN for the two NaN codes)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()
# positive finite codes 0x00..0x7E are increasing in value
_POS_VALS = E4M3_VALUES[:0x7F]


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(code, dtype=np.uint8)].astype(np.float32)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """fp32 -> E4M3FN byte: clamp to +-448, nearest value, ties to even code."""
    v = np.asarray(v, dtype=np.float32)
    a = np.minimum(np.abs(v.astype(np.float64)), E4M3_MAX)
    hi = np.searchsorted(_POS_VALS, a, side="left")       # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(v)
    return (code | np.where(neg, np.uint8(0x80), np.uint8(0))).astype(np.uint8)


E2M1_MAX = 6.0


def _e2m1_table() -> np.ndarray:
    """Value of every E2M1 nibble (float64)."""
    vals = np.empty(16, dtype=np.float64)
    for code in range(16):
        sign = -1.0 if code & 0x8 else 1.0
        e = (code >> 1) & 0x3
        m = code & 0x1
        vals[code] = sign * (m / 2.0 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return vals


E2M1_VALUES = _e2m1_table()
_E2M1_POS = E2M1_VALUES[:8]   # codes 0..7 are increasing in value


def e2m1_decode(code: np.ndarray) -> np.ndarray:
    return E2M1_VALUES[np.asarray(code, dtype=np.uint8) & 0xF].astype(np.float32)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """fp32 -> E2M1 nibble (uint8 0..15): saturate to +-6, nearest value, ties to even."""
    v = np.asarray(v, dtype=np.float32)
    a = np.minimum(np.abs(v.astype(np.float64)), E2M1_MAX)
    hi = np.minimum(np.searchsorted(_E2M1_POS, a, side="left"), 7)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E2M1_POS[lo]
    d_hi = _E2M1_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return (code | np.where(np.signbit(v), np.uint8(0x8), np.uint8(0))).astype(np.uint8)
