"""E2M1 and E4M3 codecs written from the format definitions (oracle, test infrastructure).

E2M1 (SOAR Notes 05, "02 NVFP4 KV Cache"; SGLang x Qwen x NVIDIA story, "The Core
of the Ledger" paragraph 1): one sign bit, two exponent bits, one mantissa bit.
With exponent bias 1 the eight magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.

E4M3 (the block-scale type of the same section): the OCP "fn" variant -- one sign
bit, four exponent bits with bias 7, three mantissa bits, subnormals, no
infinities, S.1111.111 is NaN, largest finite value 448.  The pages name only
"FP8 (E4M3)"; the variant is fixed by the global-scale formula amax / (6 * 448),
whose 448 is the OCP maximum (the FNUZ variant stops at 240).

Encoders implement round-to-nearest with ties to the even mantissa and saturation
to the largest finite magnitude.  The pages name no rounding mode for the
encoders; the only mode they mention is round-to-nearest (the decode kernel's
`cvt.rn` pair conversion in the "Three Paths" section), and ties-to-even is the
IEEE default.  The encoders literally search the finite grid for the nearest
value, so they read as the definition of RNE-with-saturation.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "E2M1_MAGNITUDES",
    "e2m1_decode",
    "e2m1_encode_magnitude",
    "e4m3_decode",
    "e4m3_encode",
    "E4M3_MAX",
]


def _e2m1_value(code: int) -> float:
    """Value of one 4-bit E2M1 code, from the bit fields (sign, 2-bit exponent, 1-bit mantissa)."""
    sign = (code >> 3) & 1
    exp = (code >> 1) & 3
    man = code & 1
    if exp == 0:  # subnormal: 0.m x 2^(1 - bias), bias 1
        mag = man * 0.5
    else:  # normal: 1.m x 2^(exp - bias)
        mag = (1.0 + man / 2.0) * 2.0 ** (exp - 1)
    return -mag if sign else mag


#: value of each of the 16 codes (index = code), fp64
E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)
#: the 8 non-negative magnitudes, index = code 0..7
E2M1_MAGNITUDES = E2M1_TABLE[:8].copy()


def e2m1_decode(codes) -> np.ndarray:
    """fp64 values of an array of 4-bit codes (low nibble of each element)."""
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def e2m1_encode_magnitude(abs_y) -> np.ndarray:
    """3-bit magnitude code of |y|: nearest E2M1 magnitude, ties to even mantissa, saturating at 6.

    ``abs_y`` holds non-negative fp32 values (widened to fp64, which is exact, so the distances
    below are exact).  The two grid points that bracket each value are found by binary search;
    the nearer one wins and a tie goes to the one with mantissa bit 0 (even code).  Values above 6
    -- including +inf -- saturate to code 7 (= 6).  NaN is outside the contract and raises.
    """
    a = np.asarray(abs_y, dtype=np.float32).astype(np.float64)
    if np.isnan(a).any():
        raise ValueError("E2M1 encode: NaN input is outside the contract")
    if (a < 0).any():
        raise ValueError("E2M1 encode expects magnitudes")
    flat = a.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for s in range(0, flat.size, _CHUNK):
        out[s:s + _CHUNK] = _nearest_even(E2M1_MAGNITUDES, flat[s:s + _CHUNK])
    return out.reshape(a.shape)


_CHUNK = 1 << 20   # elements per piece (keeps temporaries small; results do not depend on it)


def _nearest_even(grid: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Index of the grid point nearest to each v >= 0 (fp64, exact distances); a tie goes to the
    even index (mantissa bit 0); values at or above the last point map to it (saturation)."""
    big = v >= grid[-1]
    hi = np.clip(np.searchsorted(grid, v, side="left"), 1, grid.size - 1)   # grid[hi-1] < v <= grid[hi]
    lo = hi - 1
    d_lo = v - grid[lo]
    d_hi = grid[hi] - v
    code = np.where(d_lo < d_hi, lo, hi)
    code = np.where(d_lo == d_hi, np.where((lo & 1) == 0, lo, hi), code)
    return np.where(big, grid.size - 1, code).astype(np.uint8)


def _e4m3_value(byte: int) -> float:
    """Value of one OCP E4M3 byte from its bit fields (bias 7, subnormals, S.1111.111 = NaN)."""
    sign = (byte >> 7) & 1
    exp = (byte >> 3) & 0xF
    man = byte & 7
    if exp == 0xF and man == 7:
        return float("nan")
    if exp == 0:
        mag = (man / 8.0) * 2.0 ** (1 - 7)
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return -mag if sign else mag


E4M3_TABLE = np.array([_e4m3_value(b) for b in range(256)], dtype=np.float64)
#: the 127 finite non-negative values, index = byte 0x00..0x7E (increasing)
E4M3_POSITIVE = E4M3_TABLE[:0x7F].copy()
E4M3_MAX = float(E4M3_POSITIVE[-1])  # 448.0


def e4m3_decode(codes) -> np.ndarray:
    """fp64 values of an array of E4M3 bytes."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """E4M3 byte of each fp32 value: nearest finite value, ties to even mantissa, saturating at +-448.

    The sign bit is copied from ``x`` (so -0.0 and small negatives that round to
    zero give 0x80).  NaN is outside the contract and raises.
    """
    x32 = np.asarray(x, dtype=np.float32)
    if np.isnan(x32).any():
        raise ValueError("E4M3 encode: NaN input is outside the contract")
    flat = x32.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for s in range(0, flat.size, _CHUNK):
        part = flat[s:s + _CHUNK]
        sign = np.signbit(part).astype(np.uint8) << 7
        out[s:s + _CHUNK] = _nearest_even(E4M3_POSITIVE, np.abs(part).astype(np.float64)) | sign
    return out.reshape(x32.shape)
