"""Storage-dtype conversions for the oracle (test infrastructure only).

bfloat16 is the upper half of an IEEE float32 (1 sign, 8 exponent, 7 mantissa
bits). The pages store KV in fp16/bf16 on GPUs (Helios blog, "Model": BF16
whenever supported) and in float32 on MPS (llm-serving-engine README, "KV cache
memory layout"). The oracle holds bf16 tensors as their raw uint16 bit
patterns so that "bit-exact" means exactly that.

Rounding from float32 to bfloat16 is round-to-nearest, ties-to-even, the IEEE
default; NaN stays NaN (quiet), infinities stay infinite, and finite values
that round past the largest finite bf16 become infinity.
"""

import numpy as np

BF16 = "bf16"
F32 = "f32"


def bf16_bits_to_f32(bits):
    """Widen bf16 bit patterns (uint16) to float32 exactly: the bits become the
    high half of the float32 word and the low half is zero."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x):
    """Round float32 values to the nearest bfloat16, ties to even; return uint16 bits.

    Written from the definition: keep the high 16 bits, look at the dropped low
    16 bits as a fraction of one bf16 ulp, round up when that fraction is above
    one half, or exactly one half and the kept value is odd.
    """
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    hi = u >> np.uint64(16)
    lo = u & np.uint64(0xFFFF)
    half = np.uint64(0x8000)
    odd = hi & np.uint64(1)
    round_up = (lo > half) | ((lo == half) & (odd == np.uint64(1)))
    out = hi + round_up.astype(np.uint64)
    # NaN: exponent all ones and a nonzero mantissa. Keep it a (quiet) NaN.
    is_nan = np.isnan(x)
    out = np.where(is_nan, (hi | np.uint64(0x0040)) & np.uint64(0xFFFF), out)
    return out.astype(np.uint16)


def storage_to_f32(a, dtype):
    """Stored tensor (float32 array, or uint16 bf16 bits) -> float32 values."""
    if dtype == F32:
        return np.asarray(a, dtype=np.float32)
    if dtype == BF16:
        return bf16_bits_to_f32(a)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def f32_to_storage(x, dtype):
    """float32 values -> stored representation (float32, or bf16 bits by RNE)."""
    if dtype == F32:
        return np.asarray(x, dtype=np.float32).copy()
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown storage dtype {dtype!r}")
