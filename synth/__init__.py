"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

This package holds only data: model shapes, seeded random tensors and request
mixes.  It contains none of the method's arithmetic (no attention, no norm, no
scheduling), so the CPU oracle and the HIP path can both draw their inputs from
it without sharing any computation.

Every random stream is a numpy PCG64 generator keyed by ``(seed, crc32(name))``
so that a tensor's values depend only on the seed and its name, never on the
order in which tensors are drawn.
"""
from .gen import (  # noqa: F401
    bf16_round,
    bf16_bits,
    bits_to_f32,
    dtype_round,
    rng_for,
    normal,
    uniform_int,
)
from .configs import (  # noqa: F401
    ModelDims,
    TOY,
    MINI,
    LLAMA8B,
    GPT175B_LAYER,
    make_weights,
    init_std,
    kv_std,
    make_layer_weights,
    qkv_rows,
    ffn1_rows,
)
from .workloads import (  # noqa: F401
    Req,
    figure5_requests,
    p4_grid_requests,
    exercise4_batch,
    mini_decode_batch,
    llama_mixed_batch,
    gpt175b_mixed_batch,
    poisson_trace,
    synthetic_kv,
    random_ragged_batch,
)
