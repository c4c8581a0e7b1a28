"""Storage precision of the tensors the method keeps between operators.

The pages fix no arithmetic precision.  The configurations name a storage
dtype (fp32 or bf16) for weights, activations and the K/V cache.  Reading
taken: a tensor that one operator hands to the next -- a normalised row, the
QKV projection, q and k after the rotary embedding, the K/V cache entries,
the attention output, the feed-forward intermediate, the final-norm rows fed
to the LM head -- is stored in the model dtype, rounded to nearest with ties
to even.  Accumulations (GEMM sums, softmax sums) and the residual stream are
not rounded by this reading (the residual stream is kept in fp32).

``store(x, None)`` is the identity: the exact (fp64) oracle.  ``store(x,
'bf16')`` / ``store(x, 'fp32')`` round to that storage dtype and return fp64
values.  Parity of the bf16 GPU path is checked against both oracles: tightly
against the storage-precision one (same rounding points), and against the
exact one within the bf16 tolerance.
"""
import numpy as np


def round_to_bf16(x):
    """Nearest bfloat16 value of each element (ties to even), as fp64.

    bfloat16 keeps the sign, the 8 exponent bits and the top 7 fraction bits
    of a float32: go through float32 (exact for values that come from
    float32/bf16 data and harmless otherwise), then round the low 16 bits of
    the bit pattern half-to-even.
    """
    a = np.asarray(x, dtype=np.float64).astype(np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("round_to_bf16 expects finite values")
    u = a.view(np.uint32).astype(np.int64)
    low = u & 0xFFFF
    high = u >> 16
    up = (low > 0x8000) | ((low == 0x8000) & ((high & 1) == 1))
    high = high + up.astype(np.int64)
    out = (high << 16).astype(np.uint32).view(np.float32)
    return out.astype(np.float64)


def store(x, dtype):
    """Value of x once stored in ``dtype`` (None: no rounding)."""
    if dtype is None:
        return np.asarray(x, dtype=np.float64)
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")
