"""FP8 E4M3 (OCP "e4m3fn") codec and per-token cache quantisation, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages give one FP8 figure for the latent cache (the FP8 per-token size in
"DeepSeek'in MLA'si latent attention ile KV cache'i %93 sikistiriyor",
section "Decode bir bellek problemidir") and no format.  The reading used
here: OCP E4M3 -- 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
subnormals, no infinities, the all-ones magnitude 0x7F is NaN, largest finite
value 448.  One float32 scale per token covers all of its latent and rotary
channels: scale = amax / 448, codes = round-to-nearest-even(x / scale),
saturating at +-448.

For query vectors (the fp8 score product) the scale is a power of two
instead: the pages give no fp8 query arithmetic; this reading follows the
power-of-two (e8m0) block scales of the OCP microscaling formats, which keep
the division exact.

The decoder is written from that bit layout, not from any library table.
"""

from __future__ import annotations


import numpy as np

E4M3FN_MAX = 448.0


def _code_value(code: int) -> float:
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        mag = (man / 8.0) * 2.0 ** (1 - 7)          # subnormal
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp - 7)   # normal
    return sign * mag


_TABLE = np.array([_code_value(c) for c in range(256)], dtype=np.float64)
# non-negative finite codes 0x00..0x7E are increasing in value
_POS_VALUES = _TABLE[:0x7F].copy()


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3fn_encode(x: np.ndarray) -> np.ndarray:
    """float -> uint8 codes, round to nearest (ties to the even code),
    saturating finite values beyond 448 to +-448.  NaN maps to 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    sat = np.minimum(mag, E4M3FN_MAX)
    hi = np.searchsorted(_POS_VALUES, sat, side="left")    # first value >= sat
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi = _POS_VALUES[hi] - sat
    d_lo = sat - _POS_VALUES[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
    code = np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)
    return code


def quantize_rows_fp8(rows: np.ndarray):
    """Per-token quantisation of cache rows [T, D] -> (codes uint8 [T, D],
    scale float32 [T]).  scale = float32(amax / 448) (1 for an all-zero row)."""
    rows = np.asarray(rows, dtype=np.float64)
    amax = np.max(np.abs(rows), axis=-1)
    scale = np.where(amax > 0, amax / E4M3FN_MAX, 1.0).astype(np.float32)
    codes = e4m3fn_encode(rows / scale.astype(np.float64)[:, None])
    return codes, scale


def dequantize_rows_fp8(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """float(code) * scale, in float64."""
    return e4m3fn_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]
