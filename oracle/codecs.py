"""Storage codecs of the oracle (test infrastructure): bf16 and fp8 e4m3fn.

* bfloat16: the top 16 bits of an IEEE binary32; decoding shifts the bits back up.
* OCP 8-bit float E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits; exponent field 0 encodes subnormals m * 2^-9; the single pattern
  S.1111.111 is NaN; there are no infinities; the largest finite magnitude is
  1.75 * 2^8 = 448.  The decode table below is built from that definition alone.
* Quantisation (the fp8 KV-cache write): one IEEE float32 multiply by the inverse
  scale, clamp to +-448, then round to the nearest e4m3fn value with ties going to
  the code whose mantissa is even.  The rounding is done by an explicit nearest-value
  search over the 127 non-negative finite codes, not by bit tricks, so that it can be
  read against the definition.

Pinned by ``tests/test_oracle_codecs.py``: every bf16 code and every e4m3fn code
against torch's own casts, the quantiser against torch's cast on in-range values and
against hand-written codes at the format's landmarks (tests/golden/e4m3fn_codes.json).
"""
from __future__ import annotations

import numpy as np

E4M3FN_MAX = 448.0


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _e4m3fn_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3FN_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)
# Non-negative finite values, indexed by code 0x00..0x7E (strictly increasing).
_POS_GRID = E4M3FN_TABLE[:0x7F].copy()


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """e4m3fn codes (uint8) -> float64, exactly."""
    return E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]


def inverse_scale(scale) -> np.float32:
    """float32 reciprocal of a per-tensor dequantisation scale (one IEEE division)."""
    return np.float32(np.float32(1.0) / np.float32(scale))


def quantize_e4m3fn(x_f32: np.ndarray, inv_scale) -> np.ndarray:
    """float32 values -> e4m3fn codes: RNE(clamp(x * inv_scale, +-448)), ties to even."""
    x = np.asarray(x_f32, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):   # +-inf past float32 (clamped to +-448); NaN stays NaN
        y = (x * np.float32(inv_scale)).astype(np.float32)  # one float32 multiply
    nan = np.isnan(y)
    a = np.minimum(np.abs(np.where(nan, 0, y)).astype(np.float64), E4M3FN_MAX)
    hi = np.clip(np.searchsorted(_POS_GRID, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = np.abs(a - _POS_GRID[lo])
    d_hi = np.abs(_POS_GRID[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F) | np.where(np.signbit(y), np.uint8(0x80), np.uint8(0)), code)
    return code.astype(np.uint8)


def quantize_bf16_to_e4m3fn(bits: np.ndarray, inv_scale) -> np.ndarray:
    """bf16-stored values -> e4m3fn codes (the bf16 -> float32 step is exact)."""
    return quantize_e4m3fn(bf16_to_f32(bits), inv_scale)


_BF16_TO_E4M3FN = {}


def bf16_to_e4m3fn_table(inv_scale) -> np.ndarray:
    """``quantize_bf16_to_e4m3fn`` evaluated once for each of the 2^16 bf16 bit patterns (a
    uint8 table indexed by the bits): a bf16 input has only that many values, so looking its
    code up gives the quantiser's own result without searching the grid per element."""
    key = np.float32(inv_scale).tobytes()
    if key not in _BF16_TO_E4M3FN:
        with np.errstate(over="ignore", invalid="ignore"):   # the table spans inf and NaN inputs too
            _BF16_TO_E4M3FN[key] = quantize_bf16_to_e4m3fn(
                np.arange(1 << 16, dtype=np.uint32).astype(np.uint16), inv_scale)
    return _BF16_TO_E4M3FN[key]
