"""MXFP8 (E4M3) activation quantization for the native scaled-MFMA mode.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name natively MXFP4-quantized routed experts for DeepSeek-V4-Flash
(FreeToken quantization page, "Formatos compatibles, hardware y perfil de
rendimiento") and say no more about the arithmetic.  A matrix unit that takes
MXFP4 weights directly multiplies them by activations in another MX format,
so the native mode quantizes the bf16 activations to MXFP8.  Everything below
follows the published definition, OCP Microscaling Formats (MX) v1.0:

* FP8 E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent
  field 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; there is no
  infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
* A block of 32 consecutive elements along the contraction axis shares one
  E8M0 scale X = 2^(floor(log2(amax)) - 8), 8 being the exponent of E4M3's
  largest normal; each element becomes the E4M3 value nearest to v / X
  (ties to the even code), magnitudes beyond 448 saturating to 448.

Readings of what v1.0 leaves open (listed in the design notes):
* a block whose elements are all zero gets scale byte 0 and zero codes;
* a scale exponent below -127 is clamped to -127 (byte 0);
* the sign is kept when a value rounds to zero (negative -> code 0x80);
* the SwiGLU hidden vector is rounded to bf16 (nearest, ties to even) before
  it is quantized, as it is stored as bf16 between the two projections.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK = 32


def e4m3_to_f64(code: np.ndarray) -> np.ndarray:
    """FP8 E4M3 code (0..255) -> float64 from its bit fields (NaN for S.1111.111)."""
    c = np.asarray(code, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    sub = (m / 8.0) * 2.0 ** -6
    nor = np.power(2.0, e - 7) * (1.0 + m / 8.0)
    mag = np.where(e == 0, sub, nor)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


# the finite non-negative E4M3 values, ascending with their codes 0x00..0x7E
_GRID = e4m3_to_f64(np.arange(0x7F))


def round_to_e4m3(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of each float64 value: ties to the even code,
    magnitudes above 448 saturate to 448, the sign bit follows v."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_GRID, a, side="left")          # _GRID[hi] >= a
    hi = np.minimum(hi, len(_GRID) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _GRID[lo]
    d_hi = _GRID[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def block_scale_bytes(v: np.ndarray) -> np.ndarray:
    """E8M0 scale byte of each 32-element block along the last axis of v [n, K]."""
    v = np.asarray(v, dtype=np.float64)
    n, K = v.shape
    if K % BLOCK:
        raise ValueError("the contraction length must be a multiple of 32")
    amax = np.abs(v).reshape(n, K // BLOCK, BLOCK).max(axis=2)
    # floor(log2(amax)) exactly: amax = f * 2^p with f in [0.5, 1)
    _, p = np.frexp(amax)
    e = (p.astype(np.int64) - 1) - 8
    byte = np.clip(e + 127, 0, 254)
    return np.where(amax == 0, 0, byte).astype(np.uint8)


def mxfp8_quantize(v: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantize rows v [n, K] to MXFP8 E4M3: codes [n, K] uint8, scales [n, K/32] uint8."""
    v = np.asarray(v, dtype=np.float64)
    n, K = v.shape
    sb = block_scale_bytes(v)
    X = np.repeat(np.power(2.0, sb.astype(np.float64) - 127), BLOCK, axis=1)
    return round_to_e4m3(v / X), sb


def mxfp8_to_f64(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode MXFP8 rows: codes [n, K], scales [n, K/32] -> float64 [n, K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    n, K = codes.shape
    if scales.shape != (n, K // BLOCK):
        raise ValueError("scale array does not match the code array")
    X = np.repeat(np.power(2.0, scales.astype(np.float64) - 127), BLOCK, axis=1)
    return e4m3_to_f64(codes) * X


def mxfp8_round_trip(v: np.ndarray) -> np.ndarray:
    """The values a scaled matrix unit sees for activations v: quantize, decode."""
    return mxfp8_to_f64(*mxfp8_quantize(v))


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """float64 -> nearest bfloat16 value (8 significant bits, ties to even), as float64.

    Normal range only (the hidden vectors here stay far from bf16's limits).
    """
    v = np.asarray(v, dtype=np.float64)
    f, p = np.frexp(v)                 # v = f * 2^p, |f| in [0.5, 1)
    return np.ldexp(np.round(f * 256.0) / 256.0, p)   # np.round: half to even
