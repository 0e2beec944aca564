"""bfloat16 bit helpers for the oracle (test infrastructure only).

bfloat16 is the upper half of an IEEE-754 binary32: 1 sign bit, 8 exponent
bits, 7 stored fraction bits.  The shuffle's payload is bf16 (TensorRT-LLM PR
#13888, performance commit message: BF16 DeepSeek-V3 profile); the combine
returns bf16 rounded to nearest, ties to even.
"""

from __future__ import annotations

import numpy as np


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32: the bits become the upper half."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(values: np.ndarray) -> np.ndarray:
    """Round float32 to bf16, nearest-even, returning uint16 bit patterns.

    Adding 0x7FFF plus the lowest kept bit to the 32-bit pattern and dropping
    the low 16 bits rounds to nearest with ties to the even neighbour; a
    carry out of the fraction bumps the exponent, which also rounds the
    largest finite values up to infinity as the rounding rule requires.
    NaNs keep their sign and top payload bits and are made quiet.
    """
    f = np.ascontiguousarray(values, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    is_nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    quiet = ((u >> np.uint64(16)) | np.uint64(0x0040)) & np.uint64(0xFFFF)
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Number of representable bf16 values between two bit patterns.

    Maps each pattern to a monotone integer (negatives mirrored below zero,
    so +0 and -0 coincide) and subtracts.
    """
    def ordered(bits):
        v = np.asarray(bits, dtype=np.uint16).astype(np.int64)
        mag = v & 0x7FFF
        return np.where(v & 0x8000, -mag, mag)

    return np.abs(ordered(a_bits) - ordered(b_bits))
