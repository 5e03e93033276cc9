"""Decoding of the weight and activation storage formats, exactly, to float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name MXFP4 routed experts for DeepSeek-V4-Flash and BF16 for the
Qwen3.6 comparison (FreeToken quantization page, "Formatos compatibles,
hardware y perfil de rendimiento", hardware and results tables) but define
neither format.  Both are taken from their published definitions:

* bfloat16: the upper 16 bits of an IEEE-754 binary32 value.
* MXFP4 (OCP Microscaling Formats v1.0): blocks of 32 FP4 E2M1 elements that
  share one E8M0 scale.  E2M1 = 1 sign bit, 2 exponent bits (bias 1), 1
  mantissa bit, exponent field 0 encoding subnormals; E8M0 = an unsigned
  8-bit exponent with bias 127 and 0xFF meaning NaN.

Storage layout read here (the repository's reading, fixed for both sides):
element 2i of a row is the low nibble of byte i, element 2i+1 the high nibble;
scale j of a row covers elements 32j .. 32j+31 of that row.

The pages also name NVFP4 (the Qwen3.6 laptop build and GLM-5.2's routed
experts: FreeToken quantization page, results and hardware tables) without
defining it.  Taken from NVIDIA's published description of the format: FP4
E2M1 elements in blocks of 16 that share one FP8 E4M3 scale, and one FP32
scale per tensor; an element is E2M1 x E4M3(block scale) x tensor scale.
Same nibble order as MXFP4; scale j of a row covers elements 16j .. 16j+15.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def e2m1_to_f64(nibble: np.ndarray) -> np.ndarray:
    """FP4 E2M1 code (0..15) -> float64, from the bit fields.

    sign = bit 3, exponent field = bits 2..1, mantissa bit = bit 0, bias 1.
    exponent field 0: value = m * 2^(1-1) * 0.5 (subnormal);
    otherwise:        value = 2^(e-1) * (1 + m/2).
    """
    n = np.asarray(nibble, dtype=np.int64)
    s = (n >> 3) & 1
    e = (n >> 1) & 3
    m = n & 1
    sub = m * 0.5
    nor = np.power(2.0, e - 1) * (1.0 + m / 2.0)
    mag = np.where(e == 0, sub, nor)
    return np.where(s == 1, -mag, mag)


def e8m0_to_f64(byte: np.ndarray) -> np.ndarray:
    """E8M0 scale byte -> 2^(byte-127); 255 encodes NaN."""
    b = np.asarray(byte, dtype=np.int64)
    v = np.power(2.0, (b - 127).astype(np.float64))
    return np.where(b == 255, np.nan, v)


def _e2m1_byte_pairs() -> np.ndarray:
    """[256, 2] float64: the (element 2i, element 2i+1) values a code byte holds.

    Built from e2m1_to_f64 on the low and the high nibble of every byte value,
    so a matrix decodes by one table lookup per byte.
    """
    b = np.arange(256)
    return np.stack([e2m1_to_f64(b & 0x0F), e2m1_to_f64(b >> 4)], axis=1)


_E2M1_PAIRS = _e2m1_byte_pairs()


def _fp4_block_decode(codes: np.ndarray, block_scale: np.ndarray, block: int) -> np.ndarray:
    """E2M1 codes [rows, K/2] times one scale per `block` consecutive elements -> [rows, K]."""
    rows, half = codes.shape
    K = 2 * half
    vals = _E2M1_PAIRS[codes].reshape(rows, K)
    vals.reshape(rows, K // block, block)[...] *= block_scale[:, :, None]
    return vals


def mxfp4_to_f64(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode one MXFP4 matrix.

    codes  [rows, K/2] uint8, scales [rows, K/32] uint8  ->  float64 [rows, K].
    Each element is E2M1(nibble) * 2^(scale-127) of its 32-element block.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    rows, half = codes.shape
    K = 2 * half
    if scales.shape != (rows, K // 32) or K % 32:
        raise ValueError("scale array does not match the code array")
    return _fp4_block_decode(codes, e8m0_to_f64(scales), 32)


def nvfp4_to_f64(codes: np.ndarray, scales: np.ndarray, tensor_scale) -> np.ndarray:
    """Decode one NVFP4 matrix.

    codes [rows, K/2] uint8, scales [rows, K/16] uint8 (E4M3 codes), tensor_scale
    (a float32 value) -> float64 [rows, K]: E2M1(nibble) * E4M3(block scale) *
    tensor_scale.
    """
    from .mx import e4m3_to_f64
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    rows, half = codes.shape
    K = 2 * half
    if scales.shape != (rows, K // 16) or K % 16:
        raise ValueError("scale array does not match the code array")
    return _fp4_block_decode(codes, e4m3_to_f64(scales), 16) * float(np.float32(tensor_scale))


def expert_to_f64(fmt: str, arrays: dict) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """An expert's (W_gate [I,H], W_up [I,H], W_down [H,I]) as float64."""
    if fmt == "f32":
        return tuple(np.asarray(arrays[n], dtype=np.float32).astype(np.float64)
                     for n in ("wg", "wu", "wd"))
    if fmt == "bf16":
        return tuple(bf16_to_f64(arrays[n]) for n in ("wg", "wu", "wd"))
    if fmt == "mxfp4":
        return tuple(mxfp4_to_f64(arrays[f"{n}_codes"], arrays[f"{n}_scales"])
                     for n in ("gate", "up", "down"))
    if fmt == "nvfp4":
        ts = np.asarray(arrays["tensor_scales"], dtype=np.float32)
        return tuple(nvfp4_to_f64(arrays[f"{n}_codes"], arrays[f"{n}_scales"], ts[i])
                     for i, n in enumerate(("gate", "up", "down")))
    raise ValueError(fmt)


def activations_to_f64(fmt: str, x: np.ndarray) -> np.ndarray:
    """Activations in float32 or bf16 storage -> float64."""
    if fmt == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        return bf16_to_f64(x)
    raise ValueError(fmt)
