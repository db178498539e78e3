"""Storage types of the KV pool, handled bit by bit on the CPU.

The pool holds raw element bits: uint32 for fp32, uint16 for fp16 and bf16.
Rounding is not part of the paged-attention method; the oracle rounds the
float32 inputs once, with round-to-nearest-even, then does all arithmetic on
the rounded values upcast to float64.

Pinned by tests/test_oracle_pins.py (hand-checked bit patterns and ties).
"""
import numpy as np

BITS_DTYPE = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest, ties to even.

    bfloat16 keeps the top 16 bits of the float32 pattern.  Adding 0x7FFF plus
    the lowest kept bit to the full pattern and truncating rounds to nearest
    with ties going to the even kept pattern.  NaNs stay NaN (quiet bit set).
    (Only NaN patterns can wrap around 2**32 in the addition.)
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    t = bits >> 16
    t &= 1
    t += 0x7FFF
    t += bits
    t >>= 16
    rounded = t.astype(np.uint16)
    is_nan = (bits & 0x7FFFFFFF) > 0x7F800000
    if np.any(is_nan):
        rounded[is_nan] = ((bits[is_nan] >> 16) | 0x0040).astype(np.uint16)
    return rounded


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit pattern -> float64 (exact: bf16 is the high half of an fp32)."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_storage_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> raw storage bits of `dtype`."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.view(np.uint32).copy()
    if dtype == "f16":
        # numpy's float32 -> float16 conversion rounds to nearest even
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        flat = x.reshape(-1)
        out = np.empty(flat.shape, dtype=np.uint16)
        step = 1 << 20            # cache-sized pieces; the result is the same
        for i in range(0, flat.size, step):
            out[i:i + step] = f32_to_bf16_bits(flat[i:i + step])
        return out.reshape(x.shape)
    raise ValueError(dtype)


def storage_bits_to_f64(b: np.ndarray, dtype: str) -> np.ndarray:
    """raw storage bits of `dtype` -> float64 values."""
    if dtype == "f32":
        return np.asarray(b, dtype=np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(b)
    raise ValueError(dtype)


def poison_bits(dtype: str):
    """All-ones pattern: a NaN in fp32, fp16 and bf16 alike."""
    return BITS_DTYPE[dtype](np.iinfo(BITS_DTYPE[dtype]).max)
