"""FP8 E4M3 and FP16 rounding for the oracle, by exhaustive value tables.

[GR] "What KVarN changes in vLLM's serving path": the shipped preset keeps its scales in FP8
and its zero-points in FP16. Reading R11: FP8 is the OCP E4M3 format ("e4m3fn": exponent bias
7, three mantissa bits, no infinities, the all-ones pattern of each sign is NaN, largest finite
value 448, smallest normal 2^-6, smallest subnormal 2^-9). FP16 is IEEE-754 binary16.

Every representable finite value of each format is enumerated from its bit-level definition
and sorted; rounding is a search in that sorted list. Nothing here mirrors a bit-manipulation
rounding routine: the rounding modes are the definitions themselves (nearest with ties to the
even code, largest value not above, smallest value not below).

Test infrastructure only (see the package header).
"""

import numpy as np

# ---------------------------------------------------------------- E4M3 (OCP) value table


def _e4m3_decode_code(code: int) -> float:
    """Value of one E4M3 byte from the format definition; NaN for the two NaN codes."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_DECODE = np.array([_e4m3_decode_code(c) for c in range(256)], dtype=np.float64)
# Non-negative finite codes 0x00..0x7E: their values increase with the code.
_E4M3_POS_CODES = np.arange(0x7F, dtype=np.int64)
_E4M3_POS_VALUES = E4M3_DECODE[:0x7F].copy()
assert np.all(np.diff(_E4M3_POS_VALUES) > 0)
E4M3_MAX = float(_E4M3_POS_VALUES[-1])          # 448
E4M3_MIN_SUBNORMAL = float(_E4M3_POS_VALUES[1])  # 2^-9


def e4m3_rne(x):
    """Nearest non-negative finite E4M3 value, ties to the even code (code LSB = mantissa LSB).

    Defined for 0 <= x <= 448 (callers clamp first). Returns (values, codes)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(x < 0) or np.any(x > E4M3_MAX) or np.any(np.isnan(x)):
        raise ValueError("e4m3_rne: input outside [0, 448]")
    hi = np.searchsorted(_E4M3_POS_VALUES, x, side="left")  # first value >= x
    hi = np.minimum(hi, len(_E4M3_POS_VALUES) - 1)
    lo = np.where(_E4M3_POS_VALUES[hi] == x, hi, np.maximum(hi - 1, 0))
    dlo = x - _E4M3_POS_VALUES[lo]
    dhi = _E4M3_POS_VALUES[hi] - x
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_E4M3_POS_CODES[hi] % 2 == 0) & (hi != lo))
    idx = np.where(pick_hi, hi, lo)
    return _E4M3_POS_VALUES[idx], _E4M3_POS_CODES[idx].astype(np.uint8)


def e4m3_ru(x):
    """Smallest non-negative finite E4M3 value >= x (0 <= x <= 448). Returns (values, codes)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(x < 0) or np.any(x > E4M3_MAX) or np.any(np.isnan(x)):
        raise ValueError("e4m3_ru: input outside [0, 448]")
    idx = np.searchsorted(_E4M3_POS_VALUES, x, side="left")
    return _E4M3_POS_VALUES[idx], _E4M3_POS_CODES[idx].astype(np.uint8)


def e4m3_value(codes):
    """Decode E4M3 bytes to float64."""
    return E4M3_DECODE[np.asarray(codes, dtype=np.uint8)]


# ---------------------------------------------------------------- FP16 value table


def _fp16_all_values() -> np.ndarray:
    bits = np.arange(1 << 16, dtype=np.uint32)
    sign = np.where(bits & 0x8000, -1.0, 1.0)
    e = (bits >> 10) & 0x1F
    m = (bits & 0x3FF).astype(np.float64)
    val = np.where(e == 0, sign * (m / 1024.0) * 2.0 ** -14,
                   sign * (1.0 + m / 1024.0) * np.power(2.0, e.astype(np.float64) - 15))
    val = np.where(e == 0x1F, np.nan, val)
    return val


FP16_DECODE = _fp16_all_values()
_FP16_FINITE = np.unique(FP16_DECODE[~np.isnan(FP16_DECODE)])  # sorted, -0 and +0 merged
FP16_MAX = float(_FP16_FINITE[-1])  # 65504


def fp16_rd(x):
    """Largest finite FP16 value <= x, for -65504 <= x (callers clamp first).

    Returns (values, bits) with bits the binary16 pattern (uint16; zero is +0)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(x < -FP16_MAX) or np.any(np.isnan(x)):
        raise ValueError("fp16_rd: input below -65504")
    idx = np.searchsorted(_FP16_FINITE, x, side="right") - 1
    vals = _FP16_FINITE[idx]
    return vals, fp16_bits(vals)


def fp16_bits(vals):
    """Binary16 bit patterns of values that are exactly representable (zero -> +0)."""
    vals = np.asarray(vals, dtype=np.float64)
    h = vals.astype(np.float16)
    if not np.array_equal(h.astype(np.float64), vals):
        raise ValueError("fp16_bits: value not representable in FP16")
    b = h.view(np.uint16).copy()
    b[vals == 0] = 0
    return b


def fp16_value(bits):
    """Decode binary16 bit patterns to float64."""
    return FP16_DECODE[np.asarray(bits, dtype=np.uint16)]
