"""bfloat16 storage helpers for generated inputs.

NumPy has no bfloat16 type, so generated bf16 tensors are held as their uint16
bit patterns. Conversion from float32 rounds to nearest, ties to even; the
reverse is exact (a bf16 value is the top half of a float32).
"""
import numpy as np


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest-even) and return uint16 bits.

    NaNs are kept quiet NaNs. Used only to produce inputs.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding_bias = ((u >> 16) & 1) + 0x7FFF
    r = ((u + rounding_bias) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b):
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)
