"""Seeded random streams and storage-precision rounding for synthetic inputs.

``bf16_round`` rounds float32 values to the nearest bfloat16 value (ties to
even), which is how every bf16 tensor handed to either side is stored.  The
values are kept as float32 arrays that are exactly representable in bf16, so
the oracle can read them as plain floats and the HIP path can take their upper
16 bits.
"""
import zlib

import numpy as np


def rng_for(seed: int, name: str) -> np.random.Generator:
    """Independent PCG64 stream for tensor ``name`` under ``seed``."""
    key = zlib.crc32(name.encode("utf-8")) & 0xFFFFFFFF
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), key])))


def bf16_round(x) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even); returns float32 values."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if not np.all(np.isfinite(a)):
        raise ValueError("bf16_round expects finite values")
    bits = a.view(np.uint32)
    # finite inputs have bits <= 0xFF7FFFFF, so the sum below cannot wrap in uint32
    rounded = bits + (np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1)))
    rounded &= np.uint32(0xFFFF0000)
    return rounded.view(np.float32).reshape(a.shape)


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of values that are already bf16-representable."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = a.view(np.uint32)
    if np.any(bits & np.uint32(0xFFFF)):
        raise ValueError("bf16_bits: values are not bf16-representable; call bf16_round first")
    return (bits >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(bits) -> np.ndarray:
    """float32 values of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def dtype_round(x, dtype: str) -> np.ndarray:
    """Round to the storage precision ``dtype`` ('bf16' or 'fp32'); float32 result."""
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def normal(seed: int, name: str, shape, std: float = 1.0, mean: float = 0.0,
           dtype: str = "fp32") -> np.ndarray:
    """N(mean, std^2) samples stored in ``dtype`` precision (float32 array)."""
    g = rng_for(seed, name)
    v = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    if mean != 0.0:
        v += np.float32(mean)
    return dtype_round(v, dtype)


def uniform_int(seed: int, name: str, low: int, high_inclusive: int, size) -> np.ndarray:
    """Integers uniform over [low, high_inclusive] (int64)."""
    g = rng_for(seed, name)
    return g.integers(low, high_inclusive + 1, size=size, dtype=np.int64)
