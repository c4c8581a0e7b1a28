"""Selective batching on MI355X: one Orca-style selective-batched Transformer
iteration over a ragged batch, with its K/V manager and iteration-level
scheduler, behind the C ABI of libsb.so (include/sb.h, include/sb_ops.h).

``import selective_batching_amd`` fails loudly if libsb.so is not built: there
is no fallback path.
"""
from ._lib import (  # noqa: F401
    LIB_PATH,
    SBError,
    SB_OK, SB_ERR_INVALID, SB_ERR_NO_SLOTS, SB_ERR_NOT_FOUND, SB_ERR_TOO_LARGE, SB_ERR_DEVICE, SB_ERR_WORKSPACE,
    SB_ERR_STATE, SB_ERR_CAPACITY,
    SB_F32, SB_BF16, SB_ARCH_GPT, SB_ARCH_LLAMA,
    SB_EPI_STORE, SB_EPI_GELU, SB_EPI_RESID, SB_EPI_SWIGLU,
    SB_RESERVE_MAX, SB_RESERVE_POW2, SB_RESERVE_ORACLE,
    SB_ATTN_NOALLOC_SCRATCH_BYTES,
    KERNEL_CLASSES,
    sb_model_dims, sb_layer_weights, sb_model_weights, sb_ragged,
)
from .api import *  # noqa: F401,F403
