"""ctypes binding of libsb.so: the C ABI declared in include/sb.h and include/sb_ops.h.

Argument marshalling only -- every step of the iteration runs in the library's
host code or HIP kernels.  Every wrapper raises ``SBError`` on a non-zero
status.  Importing this module fails loudly when the library is not built.
"""
import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsb.so")

SB_OK, SB_ERR_INVALID, SB_ERR_NO_SLOTS, SB_ERR_NOT_FOUND, SB_ERR_TOO_LARGE = 0, -1, -2, -3, -4
SB_ERR_DEVICE, SB_ERR_WORKSPACE, SB_ERR_STATE, SB_ERR_CAPACITY = -5, -6, -7, -8
SB_F32, SB_BF16 = 0, 1
SB_ARCH_GPT, SB_ARCH_LLAMA = 0, 1
SB_EPI_STORE, SB_EPI_GELU, SB_EPI_RESID, SB_EPI_SWIGLU = 0, 1, 2, 3
SB_RESERVE_MAX, SB_RESERVE_POW2, SB_RESERVE_ORACLE = 0, 1, 2
SB_ATTN_NOALLOC_SCRATCH_BYTES = 64 << 20
(SB_K_GEMM_QKV, SB_K_GEMM_O, SB_K_GEMM_FFN1, SB_K_GEMM_FFN2, SB_K_GEMM_LM, SB_K_ATTN, SB_K_ATTN_COMBINE,
 SB_K_NORM, SB_K_ROPE_APPEND, SB_K_EMBED, SB_K_ARGMAX, SB_K_COUNT) = range(12)
KERNEL_CLASSES = ["gemm_qkv", "gemm_o", "gemm_ffn1", "gemm_ffn2", "gemm_lm", "attention", "attention_combine",
                  "norm", "rope_append", "embed", "argmax"]

_STATUS = {0: "SB_OK", -1: "SB_ERR_INVALID", -2: "SB_ERR_NO_SLOTS", -3: "SB_ERR_NOT_FOUND", -4: "SB_ERR_TOO_LARGE",
           -5: "SB_ERR_DEVICE", -6: "SB_ERR_WORKSPACE", -7: "SB_ERR_STATE", -8: "SB_ERR_CAPACITY"}


class SBError(RuntimeError):
    def __init__(self, status, func, msg):
        super().__init__(f"{func}: {_STATUS.get(status, status)}: {msg}")
        self.status = status
        self.func = func


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python selective_batching_amd/build.py` "
                      "(or __graft_entry__.build()) first")
# PyTorch carries its own HIP runtime.  Loaded first, it is the one libsb.so binds to (same soname),
# so the library and the streams and memory it is handed share one runtime; loaded after libsb.so,
# a second runtime would come up beside the system one the library had bound, and the library's
# calls would not see the device.
import torch  # noqa: F401,E402
lib = C.CDLL(LIB_PATH)

i32, i64, f32, f64, vp, sz = C.c_int32, C.c_int64, C.c_float, C.c_double, C.c_void_p, C.c_size_t
P = C.POINTER


class sb_model_dims(C.Structure):
    _fields_ = [("arch", i32), ("dtype", i32), ("n_layers", i32), ("hidden", i32), ("n_heads", i32),
                ("n_kv_heads", i32), ("head_dim", i32), ("ffn", i32), ("vocab", i32), ("max_pos", i32),
                ("eps", f32), ("rope_theta", f32)]


class sb_layer_weights(C.Structure):
    _fields_ = [(n, vp) for n in ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o", "ln2_g", "ln2_b",
                                  "w1", "b1", "w2", "b2")]


class sb_model_weights(C.Structure):
    _fields_ = [(n, vp) for n in ("tok_emb", "pos_emb", "lnf_g", "lnf_b", "w_lm")]


class sb_ragged(C.Structure):
    _fields_ = [("n_req", i32), ("n_tokens", i32), ("n_items", i32), ("n_partials", i32), ("n_groups", i32),
                ("max_new", i32), ("cu_seqlens", vp), ("ctx_lens", vp), ("last_row", vp), ("tok_pos", vp),
                ("tok_slot", vp), ("tok_ids", vp), ("items", vp), ("groups", vp)]


# name -> (restype, argtypes); restype int means a status code
_PROTOS = {
    "sb_last_error": (C.c_char_p, []),
    "sb_kv_arena_slots": (i64, [i64, i32]),
    "sb_kv_arena_bytes": (sz, [i64, i32, i32, i32, i32]),
    "sb_kv_create": (C.c_int, [i64, i64, i32, i32, i32, i32, vp, vp, P(vp)]),
    "sb_kv_set_stream": (C.c_int, [vp, vp]),
    "sb_kv_reserve": (C.c_int, [vp, i64, i32, P(i64)]),
    "sb_kv_free": (C.c_int, [vp, i64]),
    "sb_kv_lookup": (C.c_int, [vp, i64, P(i64), P(i32)]),
    "sb_kv_stats": (C.c_int, [vp, P(i64), P(i64), P(i64), P(i64)]),
    "sb_kv_layer_ptrs": (C.c_int, [vp, i32, P(vp), P(vp)]),
    "sb_kv_write": (C.c_int, [vp, i32, i32, vp, vp, vp, vp]),
    "sb_kv_read": (C.c_int, [vp, i32, i32, vp, vp, vp, vp]),
    "sb_kv_destroy": (None, [vp]),
    "sb_sched_create": (C.c_int, [i32, vp, P(vp)]),
    "sb_sched_add": (C.c_int, [vp, i64, f64, i32, vp, i32, i32]),
    "sb_sched_add_running": (C.c_int, [vp, i64, f64, i32, vp, i32, i32, i32, i32]),
    "sb_select_batch": (C.c_int, [vp, i32, vp, vp, vp, vp, P(i32)]),
    "sb_batch_tokens": (C.c_int, [vp, i32, vp, i32, vp, P(i32)]),
    "sb_sched_complete": (C.c_int, [vp, i32, vp, vp, P(i32), vp]),
    "sb_sched_set_chunking": (C.c_int, [vp, i32, i32]),
    "sb_sched_set_request_level": (C.c_int, [vp, i32]),
    "sb_reservation_tokens": (C.c_int, [i32, i32, i32, i32, P(i32)]),
    "sb_kv_usage": (C.c_int, [vp, P(i64), P(i64)]),
    "sb_sched_complete_deferred": (C.c_int, [vp, i32, vp, P(i32), vp, P(i64)]),
    "sb_sched_set_tokens": (C.c_int, [vp, i64, i32, vp]),
    "sb_batch_token_refs": (C.c_int, [vp, i32, vp, i32, vp, P(i32), P(i64)]),
    "sb_sched_output": (C.c_int, [vp, i64, i32, vp, P(i32)]),
    "sb_sched_stats": (C.c_int, [vp, P(i32), P(i64), P(i64)]),
    "sb_sched_destroy": (None, [vp]),
    "sb_ragged_bytes": (sz, [P(sb_model_dims), i32, i32, i64]),
    "sb_attn_max_partials": (i64, [P(sb_model_dims), i32, i64]),
    "sb_ragged_build": (C.c_int, [P(sb_model_dims), i32, vp, vp, vp, vp, vp, vp, sz, vp, P(sb_ragged)]),
    "sb_layer_workspace_bytes": (sz, [P(sb_model_dims), i32, i32, i32]),
    "sb_embed": (C.c_int, [P(sb_model_dims), P(sb_model_weights), P(sb_ragged), vp, vp]),
    "sb_embed_chained": (C.c_int, [P(sb_model_dims), P(sb_model_weights), P(sb_ragged), vp, i32, vp, vp]),
    "sb_forward": (C.c_int, [P(sb_model_dims), P(sb_model_weights), vp, i32, P(sb_ragged), vp, vp, i32, vp, vp, vp,
                             vp, sz, vp]),
    "sb_layer_step": (C.c_int, [P(sb_model_dims), P(sb_layer_weights), P(sb_ragged), vp, i32, vp, vp, sz, vp]),
    "sb_lm_argmax": (C.c_int, [P(sb_model_dims), P(sb_model_weights), P(sb_ragged), vp, vp, vp, vp, sz, vp]),
    "sb_timing_enable": (C.c_int, [i32]),
    "sb_timing_read": (C.c_int, [i32, P(f64), P(i64)]),
    "sb_timing_reset": (C.c_int, []),
    "sb_op_gemm": (C.c_int, [i32, i32, i32, i32, i32, vp, i64, vp, i64, vp, vp, i64, i32, i32, vp]),
    "sb_op_norm": (C.c_int, [i32, i32, i32, i32, vp, vp, vp, vp, f32, vp, vp]),
    "sb_op_rope_append": (C.c_int, [P(sb_model_dims), P(sb_ragged), vp, i32, vp, vp]),
    "sb_op_attention": (C.c_int, [P(sb_model_dims), P(sb_ragged), vp, i32, vp, vp, vp, sz, vp]),
    "sb_op_attention_noalloc": (C.c_int, [P(sb_model_dims), P(sb_ragged), vp, i32, vp, vp, vp]),
    "sb_op_argmax": (C.c_int, [i32, i32, vp, vp, vp]),
}

for _name, (_res, _args) in _PROTOS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def last_error() -> str:
    return lib.sb_last_error().decode(errors="replace")


def check(status, func):
    if status != SB_OK:
        raise SBError(status, func, last_error())
    return status


def call(name, *args):
    """Call a status-returning entry point and raise SBError on failure."""
    return check(getattr(lib, name)(*args), name)
