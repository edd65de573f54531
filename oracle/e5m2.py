"""OCP E5M2 value table and table-driven encoder (oracle; test infrastructure only).

Follows [FP8] section "FP8 是什么" (format table: E5M2 has 1 sign, 5 exponent and
2 mantissa bits, largest value 57344, smallest normal 2^-14, smallest
subnormal 2^-16; the wider range and coarser grid of the two FP8 formats) and
section "什么是 FP8 量化" (the representable set is the quantization grid; values
are rounded to the nearest grid point, ties to even). [VS] api.makesence.top,
"LLM推理量化:FP8 versus INT8", section 1 gives the same range, and its section 2
serves a W8A8 E4M3 model with an E5M2 KV cache.

Readings taken where the pages are silent:

* The encoding is OCP E5M2, the one consistent with the table: bias 15,
  exponent field 0 holds subnormals m * 2^-16, exponent field 31 holds
  infinity (mantissa 0) and NaN (mantissa != 0), so 0 11110 11 = 57344 is the
  largest finite code (0x7B).
* The pages state saturation only for E4M3. The quantizer keeps the same
  rule for E5M2: magnitudes at or above 57344 encode as +-57344, never as
  infinity (with s = amax / 57344 only a rounding hair above 57344 can occur).
* The sign of a zero result is copied from the input, as for E4M3.
* Non-finite inputs are outside the contract; the encoder raises on them.
"""

import math

import numpy as np

E5M2_MAX = 57344.0
MAX_CODE = 0x7B                                  # 0 11110 11
NONFINITE_CODES = (0x7C, 0x7D, 0x7E, 0x7F, 0xFC, 0xFD, 0xFE, 0xFF)   # S 11111 mm


def _value_of_code(c: int) -> float:
    """Real value of one 8-bit E5M2 code (bias 15, subnormals at exponent 0,
    infinity and NaN at exponent 31)."""
    sign = -1.0 if (c & 0x80) else 1.0
    e = (c >> 2) & 0x1F
    m = c & 0x3
    if e == 0x1F:
        return sign * math.inf if m == 0 else math.nan
    if e == 0:
        return sign * (m / 4.0) * 2.0 ** (1 - 15)
    return sign * (1.0 + m / 4.0) * 2.0 ** (e - 15)


#: float64 value of every code 0..255 (+-inf at 0x7C / 0xFC, NaN at the other
#: exponent-31 codes).
DECODE = np.array([_value_of_code(c) for c in range(256)], dtype=np.float64)

#: non-negative finite grid, index == code (0x00 .. 0x7B), strictly increasing.
GRID = DECODE[: MAX_CODE + 1].copy()

#: the 123 midpoints between neighbouring non-negative grid values (exact in
#: float64: every grid value has at most 3 significant bits).
MIDPOINTS = (GRID[:-1] + GRID[1:]) / 2.0


def decode(codes) -> np.ndarray:
    """float64 values of uint8 codes (table lookup)."""
    return DECODE[np.asarray(codes, dtype=np.uint8)]


def encode(v) -> np.ndarray:
    """Round-to-nearest-even, saturating encode of real values to E5M2 codes.

    Each magnitude is compared exactly, in float64, with the table of
    midpoints: below a midpoint it takes the lower grid value, above it the
    upper one, exactly on it the code whose mantissa LSB is 0. Magnitudes at
    or above 57344 map to 57344. The sign bit is copied from the input.
    """
    v = np.asarray(v)
    if not np.all(np.isfinite(v)):
        raise ValueError("E5M2 encode: non-finite input is outside the contract")
    a = np.abs(v.astype(np.float64))
    i = np.searchsorted(MIDPOINTS, a, side="left")
    on_mid = (i < MIDPOINTS.size) & (a == MIDPOINTS[np.minimum(i, MIDPOINTS.size - 1)])
    code = np.where(on_mid & (i % 2 == 1), i + 1, i)
    code = np.where(a >= E5M2_MAX, MAX_CODE, code)
    code = code | (np.signbit(v).astype(np.int64) << 7)
    return code.astype(np.uint8)


def finite_codes() -> np.ndarray:
    """All 248 finite codes."""
    return np.array([c for c in range(256) if c not in NONFINITE_CODES], dtype=np.uint8)
