"""bfloat16 helpers for the CPU oracle (test infrastructure only).

bf16 tensors travel as their uint16 bit patterns.  Widening bf16 -> float
is exact (the 16 bits become the high half of a float32).  Narrowing
float32 -> bf16 is IEEE round-to-nearest-even on the 16 dropped bits:
add 0x7FFF plus the lowest kept bit, then drop the low half; NaN maps to
the quiet NaN 0x7FC0 with the sign kept.  This is the textbook bit method
for RNE on a truncated significand, written out here; it is checked
against torch's CPU cast in the oracle's tests.
"""
import numpy as np


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even). Returns uint16 bit patterns."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    is_nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    qnan = (((u >> np.uint32(16)) & np.uint32(0x8000)) | np.uint32(0x7FC0)).astype(np.uint16)
    return np.where(is_nan, qnan, rounded)


def f64_to_bf16_bits(x64: np.ndarray) -> np.ndarray:
    """Round a float64 value to bf16 through float32 (each step RNE).

    The double rounding f64 -> f32 -> bf16 can differ from a direct f64 ->
    bf16 rounding only when the f64 value lies within one f32 ulp of a bf16
    rounding boundary; the GPU path rounds its fp32 accumulator the same
    f32 -> bf16 way, so the oracle does too.
    """
    return f32_to_bf16_bits(np.asarray(x64, dtype=np.float64).astype(np.float32))
