"""OCP E4M3 value table and table-driven encoder (oracle; test infrastructure only).

Follows [FP8] section "FP8 是什么" (format table: E4M3 has 1 sign, 4 exponent and
3 mantissa bits, largest value 448, smallest normal 2^-6, smallest subnormal
2^-9; no infinity, rounding saturates at +-448) and section "什么是 FP8 量化"
(the representable set is the quantization grid; values are rounded to the
nearest grid point, ties to even, and out-of-range values saturate).

Readings taken where the pages are silent or garbled:

* The value formula printed in section "什么是 FP8 量化" has no exponent bias
  and no subnormals. Read literally its maximum would be 1.875 * 2^15, which
  contradicts the format table. The only encoding consistent with the table
  (max 448, min normal 2^-6, min subnormal 2^-9) is OCP E4M3FN: bias 7,
  exponent field 0 holds subnormals m * 2^-9, and S.1111.111 is NaN (so
  0 1111 110 = 448 is the largest finite code).
* The sign of a zero result is copied from the input (IEEE style): a negative
  value that rounds to zero encodes as 0x80.
* Non-finite inputs are outside the contract; the encoder raises on them.
"""

import math

import numpy as np

E4M3_MAX = 448.0
MAX_CODE = 0x7E            # 0 1111 110
NAN_CODES = (0x7F, 0xFF)   # S 1111 111


def _value_of_code(c: int) -> float:
    """Real value of one 8-bit E4M3 code (bias 7, subnormals at exponent 0)."""
    sign = -1.0 if (c & 0x80) else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


#: float64 value of every code 0..255 (NaN at 0x7F and 0xFF).
DECODE = np.array([_value_of_code(c) for c in range(256)], dtype=np.float64)

#: non-negative finite grid, index == code (0x00 .. 0x7E), strictly increasing.
GRID = DECODE[: MAX_CODE + 1].copy()

#: the 126 midpoints between neighbouring non-negative grid values. Every grid
#: value is a dyadic rational with at most 4 significant bits, so each midpoint
#: is exact in float64.
MIDPOINTS = (GRID[:-1] + GRID[1:]) / 2.0


def decode(codes) -> np.ndarray:
    """float64 values of uint8 codes (table lookup)."""
    return DECODE[np.asarray(codes, dtype=np.uint8)]


def encode(v) -> np.ndarray:
    """Round-to-nearest-even, saturating encode of real values to E4M3 codes.

    ``v`` holds finite numbers (typically float32 quotients x/s). Each
    magnitude is compared exactly, in float64, with the table of midpoints:
    below a midpoint it takes the lower grid value, above it the upper one, and
    exactly on it the code whose mantissa LSB is 0 (ties to even). Magnitudes
    at or above 448 map to 448 (saturation; rounding first and clamping after
    gives the same code because 448's upper neighbour would be the NaN code).
    The sign bit is copied from the input.
    """
    v = np.asarray(v)
    if not np.all(np.isfinite(v)):
        raise ValueError("E4M3 encode: non-finite input is outside the contract")
    a = np.abs(v.astype(np.float64))
    # number of midpoints strictly below a  ==  code of the nearest grid value
    # when a is not exactly on a midpoint
    i = np.searchsorted(MIDPOINTS, a, side="left")
    on_mid = (i < MIDPOINTS.size) & (a == MIDPOINTS[np.minimum(i, MIDPOINTS.size - 1)])
    # a tie sits between codes i and i+1; keep the one with an even mantissa
    code = np.where(on_mid & (i % 2 == 1), i + 1, i)
    code = np.where(a >= E4M3_MAX, MAX_CODE, code)
    code = code | (np.signbit(v).astype(np.int64) << 7)
    return code.astype(np.uint8)


def finite_codes() -> np.ndarray:
    """All 254 finite codes."""
    return np.array([c for c in range(256) if c not in NAN_CODES], dtype=np.uint8)
