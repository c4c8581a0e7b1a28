"""Python wrappers with the names of the C entry points (include/sb.h, include/sb_ops.h).

Only argument marshalling: numpy arrays in and out for host arrays, integer
addresses for device buffers and streams.  Errors raise SBError.
"""
import ctypes as C

import numpy as np

from ._lib import call, lib, sb_model_dims, sb_model_weights, sb_layer_weights, sb_ragged  # noqa: F401

_i32p = C.POINTER(C.c_int32)
_i64p = C.POINTER(C.c_int64)


def _ptr(a):
    return a.ctypes.data_as(C.c_void_p) if a is not None else None


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _i64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


# ---------------------------------------------------------------- K/V manager
def sb_kv_arena_slots(n_slots, max_live):
    return int(lib.sb_kv_arena_slots(n_slots, max_live))


def sb_kv_arena_bytes(arena_slots, n_layers, n_kv_heads, head_dim, dtype):
    return int(lib.sb_kv_arena_bytes(arena_slots, n_layers, n_kv_heads, head_dim, dtype))


def sb_kv_create(n_slots, arena_slots, n_layers, n_kv_heads, head_dim, dtype, k_arena=None, v_arena=None):
    h = C.c_void_p()
    call("sb_kv_create", n_slots, arena_slots, n_layers, n_kv_heads, head_dim, dtype, k_arena, v_arena, C.byref(h))
    return h.value


def sb_kv_set_stream(kv, stream):
    call("sb_kv_set_stream", kv, stream)


def sb_kv_reserve(kv, req_id, max_tokens):
    b = C.c_int64()
    call("sb_kv_reserve", kv, req_id, max_tokens, C.byref(b))
    return b.value


def sb_kv_free(kv, req_id):
    call("sb_kv_free", kv, req_id)


def sb_kv_lookup(kv, req_id):
    b, m = C.c_int64(), C.c_int32()
    call("sb_kv_lookup", kv, req_id, C.byref(b), C.byref(m))
    return b.value, m.value


def sb_kv_stats(kv):
    a, b, c, d = C.c_int64(), C.c_int64(), C.c_int64(), C.c_int64()
    call("sb_kv_stats", kv, C.byref(a), C.byref(b), C.byref(c), C.byref(d))
    return {"n_rsrv": a.value, "n_slots": b.value, "n_live": c.value, "n_compactions": d.value}


def sb_kv_layer_ptrs(kv, layer):
    k, v = C.c_void_p(), C.c_void_p()
    call("sb_kv_layer_ptrs", kv, layer, C.byref(k), C.byref(v))
    return k.value, v.value


def sb_kv_write(kv, layer, n, slots_dev, k_dev, v_dev, stream=None):
    call("sb_kv_write", kv, layer, n, slots_dev, k_dev, v_dev, stream)


def sb_kv_read(kv, layer, n, slots_dev, k_dev, v_dev, stream=None):
    call("sb_kv_read", kv, layer, n, slots_dev, k_dev, v_dev, stream)


def sb_kv_destroy(kv):
    lib.sb_kv_destroy(kv)


# ---------------------------------------------------------------- scheduler
def sb_sched_create(max_bs, kv):
    h = C.c_void_p()
    call("sb_sched_create", max_bs, kv, C.byref(h))
    return h.value


def sb_sched_add(s, req_id, arrival, prompt_tokens, out_len, max_tokens, prompt_len=None):
    toks = None if prompt_tokens is None else _i32(prompt_tokens)
    plen = len(toks) if toks is not None else int(prompt_len)
    call("sb_sched_add", s, req_id, float(arrival), plen, _ptr(toks), out_len, max_tokens)


def sb_sched_add_running(s, req_id, arrival, prompt_len, out_len, max_tokens, generated, last_token, prompt_tokens=None):
    toks = None if prompt_tokens is None else _i32(prompt_tokens)
    call("sb_sched_add_running", s, req_id, float(arrival), prompt_len, _ptr(toks), out_len, max_tokens, generated,
         last_token)


def sb_reservation_tokens(policy, prompt_len, out_len, max_out):
    v = C.c_int32()
    call("sb_reservation_tokens", policy, prompt_len, out_len, max_out, C.byref(v))
    return v.value


def sb_kv_usage(s):
    r, st = C.c_int64(), C.c_int64()
    call("sb_kv_usage", s, C.byref(r), C.byref(st))
    return r.value, st.value


def sb_sched_set_request_level(s, on):
    call("sb_sched_set_request_level", s, 1 if on else 0)


def sb_sched_set_chunking(s, token_budget, chunk):
    call("sb_sched_set_chunking", s, token_budget, chunk)


def sb_select_batch(s, cap):
    ids = np.zeros(cap, np.int64)
    n_new = np.zeros(cap, np.int32)
    ctx = np.zeros(cap, np.int32)
    base = np.zeros(cap, np.int64)
    n = C.c_int32()
    call("sb_select_batch", s, cap, _ptr(ids), _ptr(n_new), _ptr(ctx), _ptr(base), C.byref(n))
    k = n.value
    return ids[:k].copy(), n_new[:k].copy(), ctx[:k].copy(), base[:k].copy()


def sb_batch_tokens(s, ids, cap):
    ids = _i64(ids)
    out = np.zeros(max(cap, 1), np.int32)
    n = C.c_int32()
    call("sb_batch_tokens", s, len(ids), _ptr(ids), cap, _ptr(out), C.byref(n))
    return out[:n.value].copy()


def sb_sched_complete(s, ids, new_tokens):
    ids = _i64(ids)
    toks = _i32(new_tokens)
    fin = np.zeros(max(len(ids), 1), np.int64)
    nf = C.c_int32()
    call("sb_sched_complete", s, len(ids), _ptr(ids), _ptr(toks), C.byref(nf), _ptr(fin))
    return fin[:nf.value].copy()


def sb_sched_complete_deferred(s, ids):
    """Count-based Complete with the token values left pending; returns (finished ids, ticket)."""
    ids = _i64(ids)
    fin = np.zeros(max(len(ids), 1), np.int64)
    nf = C.c_int32()
    ticket = C.c_int64()
    call("sb_sched_complete_deferred", s, len(ids), _ptr(ids), C.byref(nf), _ptr(fin), C.byref(ticket))
    return fin[:nf.value].copy(), ticket.value


def sb_sched_set_tokens(s, ticket, tokens):
    toks = _i32(tokens)
    call("sb_sched_set_tokens", s, ticket, len(toks), _ptr(toks))


def sb_batch_token_refs(s, ids, cap):
    """Token ids of the batch, pending ones as references -(1 + row); returns (tokens, ticket or -1)."""
    ids = _i64(ids)
    out = np.zeros(max(cap, 1), np.int32)
    n = C.c_int32()
    ticket = C.c_int64()
    call("sb_batch_token_refs", s, len(ids), _ptr(ids), cap, _ptr(out), C.byref(n), C.byref(ticket))
    return out[:n.value].copy(), ticket.value


def sb_sched_output(s, req_id, cap=1 << 16):
    out = np.zeros(cap, np.int32)
    n = C.c_int32()
    call("sb_sched_output", s, req_id, cap, _ptr(out), C.byref(n))
    return out[:n.value].copy()


def sb_sched_stats(s):
    p, r, f = C.c_int32(), C.c_int64(), C.c_int64()
    call("sb_sched_stats", s, C.byref(p), C.byref(r), C.byref(f))
    return {"pool": p.value, "n_rsrv": r.value, "n_finished": f.value}


def sb_sched_destroy(s):
    lib.sb_sched_destroy(s)


# ---------------------------------------------------------------- ragged batch
def sb_ragged_bytes(dims, max_req, max_tokens, max_keys_total):
    return int(lib.sb_ragged_bytes(C.byref(dims), max_req, max_tokens, max_keys_total))


def sb_attn_max_partials(dims, max_req, max_keys_total):
    return int(lib.sb_attn_max_partials(C.byref(dims), max_req, max_keys_total))


def sb_ragged_build(dims, n_new, ctx, slot_base, token_ids, host_staging, dev_meta, nbytes, stream=None):
    n_new, ctx, base = _i32(n_new), _i32(ctx), _i64(slot_base)
    toks = None if token_ids is None else _i32(token_ids)
    rg = sb_ragged()
    call("sb_ragged_build", C.byref(dims), len(n_new), _ptr(n_new), _ptr(ctx), _ptr(base), _ptr(toks), host_staging,
         dev_meta, nbytes, stream, C.byref(rg))
    return rg


# ---------------------------------------------------------------- device steps
def sb_layer_workspace_bytes(dims, max_tokens, max_req, max_partials):
    return int(lib.sb_layer_workspace_bytes(C.byref(dims), max_tokens, max_req, max_partials))


def sb_embed(dims, mw, rg, x, stream=None):
    call("sb_embed", C.byref(dims), C.byref(mw), C.byref(rg), x, stream)


def sb_embed_chained(dims, mw, rg, prev_ids, prev_n, x, stream=None):
    call("sb_embed_chained", C.byref(dims), C.byref(mw), C.byref(rg), prev_ids, prev_n, x, stream)


def sb_forward(dims, mw, layer_array, n_layers, rg, kv, prev_ids, prev_n, x, logits, out_ids, ws, ws_bytes,
               stream=None):
    """layer_array: a ctypes array of sb_layer_weights (kept by the caller)."""
    call("sb_forward", C.byref(dims), C.byref(mw), C.cast(layer_array, C.c_void_p) if layer_array is not None else None,
         n_layers, C.byref(rg), kv, prev_ids, prev_n, x, logits, out_ids, ws, ws_bytes, stream)


def sb_layer_step(dims, lw, rg, kv, layer, x, ws, ws_bytes, stream=None):
    call("sb_layer_step", C.byref(dims), C.byref(lw), C.byref(rg), kv, layer, x, ws, ws_bytes, stream)


def sb_lm_argmax(dims, mw, rg, x, logits, out_ids, ws, ws_bytes, stream=None):
    call("sb_lm_argmax", C.byref(dims), C.byref(mw), C.byref(rg), x, logits, out_ids, ws, ws_bytes, stream)


def sb_timing_enable(on, classes=None):
    """on=False: off; on=True: every class, or only the kernel-class indices in ``classes``."""
    global timing_mask
    mask = 0
    if on:
        mask = -1 if classes is None else sum(1 << k for k in classes)
    call("sb_timing_enable", mask)
    timing_mask = mask


timing_mask = 0     # the class mask last set through sb_timing_enable


def sb_timing_read(k):
    ms, n = C.c_double(), C.c_int64()
    call("sb_timing_read", k, C.byref(ms), C.byref(n))
    return ms.value, n.value


def sb_timing_reset():
    call("sb_timing_reset")


# ---------------------------------------------------------------- op-level entry points
def sb_op_gemm(dtype, epilogue, M, N, K, A, lda, W, ldw, bias, Cout, ldc, out_f32=0, F=0, stream=None):
    call("sb_op_gemm", dtype, epilogue, M, N, K, A, lda, W, ldw, bias, Cout, ldc, out_f32, F, stream)


def sb_op_norm(dtype, kind, rows, hidden, x, row_map, g, b, eps, out, stream=None):
    call("sb_op_norm", dtype, kind, rows, hidden, x, row_map, g, b, eps, out, stream)


def sb_op_rope_append(dims, rg, kv, layer, qkv, stream=None):
    call("sb_op_rope_append", C.byref(dims), C.byref(rg), kv, layer, qkv, stream)


def sb_op_attention(dims, rg, kv, layer, qkv, o, ws, ws_bytes, stream=None):
    call("sb_op_attention", C.byref(dims), C.byref(rg), kv, layer, qkv, o, ws, ws_bytes, stream)


def sb_op_attention_noalloc(dims, rg, kv, layer, qkv, o, stream=None):
    call("sb_op_attention_noalloc", C.byref(dims), C.byref(rg), kv, layer, qkv, o, stream)


def sb_op_argmax(rows, V, logits, out, stream=None):
    call("sb_op_argmax", rows, V, logits, out, stream)
