"""bfloat16 <-> float32 bit conversion on the host (no ml_dtypes in this image).

bfloat16 is the top half of an IEEE binary32 word. Rounding float32 to bfloat16 uses
round-to-nearest, ties-to-even on the 16 dropped bits, the same rule hardware converters use.
"""
import numpy as np


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the uint16 bit patterns.

    Inputs must be finite or +-inf (NaN payloads are not preserved).
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # Adding 0x7FFF plus the lowest kept bit rounds half-way cases towards the even result.
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Expand uint16 bfloat16 bit patterns to float32 exactly."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)
