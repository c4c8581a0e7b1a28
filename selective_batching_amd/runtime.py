"""Device memory and the iteration loop around the C ABI.

PyTorch provides device memory (weights, K/V arenas, workspace, activations,
pinned staging) and the HIP stream; every computation is a libsb call.  One
iteration (``Engine.step``) follows the scheduling loop of Algorithm 1 with a
single worker ("连续批处理完全拆解"; "CS349D Lecture 2", section 4.1): select a
batch, build the ragged metadata, run embed -> layers -> LM head/argmax on the
flattened batch, bring the B new token ids back, complete the iteration.
"""
import ctypes as C
import time

import numpy as np
import torch

from . import api as A
from ._lib import (SB_ARCH_GPT, SB_ARCH_LLAMA, SB_BF16, SB_F32, sb_layer_weights, sb_model_dims,
                   sb_model_weights)

TORCH_DT = {SB_F32: torch.float32, SB_BF16: torch.bfloat16}
DT_CODE = {"fp32": SB_F32, "bf16": SB_BF16}


def stream_handle():
    return torch.cuda.current_stream().cuda_stream


def make_dims(m, dtype: str) -> sb_model_dims:
    """ABI model shape from any object with arch, n_layers, H, nq, nkv, d, F, V, max_pos, eps, rope_theta."""
    return sb_model_dims(arch=SB_ARCH_GPT if m.arch == "gpt" else SB_ARCH_LLAMA, dtype=DT_CODE[dtype],
                         n_layers=m.n_layers, hidden=m.H, n_heads=m.nq, n_kv_heads=m.nkv, head_dim=m.d, ffn=m.F,
                         vocab=m.V, max_pos=m.max_pos, eps=m.eps, rope_theta=m.rope_theta)


def _addr(t):
    return None if t is None else t.data_ptr()


LAYER_KEYS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o", "ln2_g", "ln2_b", "w1", "b1", "w2", "b2")
MODEL_KEYS = ("tok_emb", "pos_emb", "lnf_g", "lnf_b", "w_lm")


class DeviceWeights:
    """Weights resident in HBM in the model dtype, plus the ABI structs pointing at them.

    ``host``: dict of numpy arrays (layout of ``synth.make_weights``), copied
    exactly; or None with ``seed``: random init on the device (matrices
    N(0, min(0.02, fan_in^-1/2)^2), embeddings and biases N(0, 0.02^2), gains
    1 + N(0, 0.1^2)) for runs that do not compare against the oracle.
    """

    def __init__(self, m, dtype: str, host=None, seed=0, device="cuda", layers=None, with_head=True):
        self.m, self.dtype = m, dtype
        tdt = TORCH_DT[DT_CODE[dtype]]
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)

        def put(arr):
            return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device=device).to(tdt)

        def wstd(fan_in):
            return min(0.02, fan_in ** -0.5)

        def rnd(shape, std, mean=0.0):
            t = torch.empty(shape, dtype=tdt, device=device)
            t.normal_(mean, std, generator=gen)
            return t

        gpt = m.arch == "gpt"
        n_layers = m.n_layers if layers is None else layers
        self.layers = []
        for l in range(n_layers):
            if host is not None:
                hw = host["layers"][l]
                t = {k: (put(hw[k]) if k in hw else None) for k in LAYER_KEYS}
            else:
                f1 = m.F if gpt else 2 * m.F
                t = {"ln1_g": rnd((m.H,), 0.1, 1.0), "w_qkv": rnd((m.qkv_out, m.H), wstd(m.H)),
                     "w_o": rnd((m.H, m.nq * m.d), wstd(m.nq * m.d)), "ln2_g": rnd((m.H,), 0.1, 1.0),
                     "w1": rnd((f1, m.H), wstd(m.H)), "w2": rnd((m.H, m.F), wstd(m.F))}
                for k in ("ln1_b", "b_qkv", "b_o", "ln2_b", "b1", "b2"):
                    t[k] = None
                if gpt:
                    t.update({"ln1_b": rnd((m.H,), 0.02), "b_qkv": rnd((m.qkv_out,), 0.02),
                              "b_o": rnd((m.H,), 0.02), "ln2_b": rnd((m.H,), 0.02), "b1": rnd((m.F,), 0.02),
                              "b2": rnd((m.H,), 0.02)})
            self.layers.append(t)
        self.model = {k: None for k in MODEL_KEYS}
        if with_head and m.V > 0:
            if host is not None:
                self.model = {k: (put(host[k]) if k in host else None) for k in MODEL_KEYS}
            else:
                self.model = {"tok_emb": rnd((m.V, m.H), 0.02), "w_lm": rnd((m.V, m.H), wstd(m.H)),
                              "lnf_g": rnd((m.H,), 0.1, 1.0), "lnf_b": rnd((m.H,), 0.02) if gpt else None,
                              "pos_emb": rnd((m.max_pos, m.H), 0.02) if gpt else None}
        self.layer_structs = [sb_layer_weights(**{k: _addr(t[k]) for k in LAYER_KEYS}) for t in self.layers]
        self.layer_array = (sb_layer_weights * max(len(self.layer_structs), 1))(*self.layer_structs)
        self.model_struct = sb_model_weights(**{k: _addr(self.model[k]) for k in MODEL_KEYS})


class Engine:
    """K/V manager + scheduler + device buffers for one model on one GPU."""

    def __init__(self, m, dtype: str, weights: DeviceWeights, n_slots: int, max_bs: int, max_tokens: int,
                 max_keys_total: int = None, device="cuda", zero_arena=True, chunking=None, request_level=False,
                 graphs=False):
        """``max_tokens``: most tokens one iteration feeds (with ``chunking`` = (token budget, chunk) the
        budget bounds it).  ``request_level``: static batching (the baseline) instead of Algorithm 1.
        ``graphs``: replay the device side of an iteration from a HIP graph when an iteration of the same
        shape has run before (see ``forward``)."""
        self.m, self.dtype, self.w = m, dtype, weights
        self.graphs = graphs
        # per-iteration timing for logs: host time of each launch (Select, metadata, enqueue) and, when
        # record_events is set, the device time of its work from a pair of HIP events on the stream
        self.record_events = False
        self._graph_seen = {}          # iteration shape -> times seen (captured on the second)
        self._graph_cache = {}         # iteration shape -> captured torch.cuda.CUDAGraph
        self.dims = make_dims(m, dtype)
        self.max_bs, self.max_tokens = max_bs, max_tokens
        self.device = device
        L = len(weights.layers)
        self.n_layers = L
        L = max(L, 1)          # the K/V manager needs at least one layer plane
        self.arena_slots = A.sb_kv_arena_slots(n_slots, max_bs)
        nbytes = A.sb_kv_arena_bytes(self.arena_slots, L, m.nkv, m.d, self.dims.dtype)
        alloc = torch.zeros if zero_arena else torch.empty
        self.k_arena = alloc(nbytes, dtype=torch.uint8, device=device)
        self.v_arena = alloc(nbytes, dtype=torch.uint8, device=device)
        self.kv = A.sb_kv_create(n_slots, self.arena_slots, L, m.nkv, m.d, self.dims.dtype,
                                 self.k_arena.data_ptr(), self.v_arena.data_ptr())
        A.sb_kv_set_stream(self.kv, stream_handle())
        self.sched = A.sb_sched_create(max_bs, self.kv)
        if chunking is not None:
            A.sb_sched_set_chunking(self.sched, *chunking)
        if request_level:
            A.sb_sched_set_request_level(self.sched, True)
        self.max_keys_total = max_keys_total if max_keys_total is not None else max_bs * (n_slots + 1)
        self.meta_bytes = A.sb_ragged_bytes(self.dims, max_bs, max_tokens, self.max_keys_total)
        # two host staging buffers (and two host id buffers): the host can build iteration k+1's
        # metadata while iteration k's copy from the other buffer is still queued on the stream
        self.staging_bufs = [torch.empty(self.meta_bytes, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
        self.staging = self.staging_bufs[0]
        self.meta = torch.empty(self.meta_bytes, dtype=torch.uint8, device=device)
        self.max_partials = A.sb_attn_max_partials(self.dims, max_bs, self.max_keys_total)
        self.ws_bytes = A.sb_layer_workspace_bytes(self.dims, max_tokens, max_bs, self.max_partials)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.x = torch.empty(max_tokens * m.H, dtype=torch.float32, device=device)
        # one device id buffer per staging buffer: a chained launch reads the previous iteration's ids
        # from the other buffer while writing its own
        self.ids_dev_bufs = [torch.empty(max_bs, dtype=torch.int32, device=device) for _ in range(2)]
        self.ids_dev = self.ids_dev_bufs[0]
        self.ids_host_bufs = [torch.empty(max_bs, dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self.ids_host = self.ids_host_bufs[0]
        self.logits = torch.empty(max_bs * max(m.V, 1), dtype=torch.float32, device=device) if m.V > 0 else None

    def close(self):
        if self.sched:
            A.sb_sched_destroy(self.sched)
            self.sched = None
        if self.kv:
            A.sb_kv_destroy(self.kv)
            self.kv = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------ requests
    def add(self, rid, arrival, prompt, out_len, max_tokens):
        A.sb_sched_add(self.sched, rid, arrival, prompt, out_len, max_tokens)

    def add_running(self, rid, arrival, prompt_len, out_len, max_tokens, generated, last_token):
        A.sb_sched_add_running(self.sched, rid, arrival, prompt_len, out_len, max_tokens, generated, last_token)

    # ------------------------------------------------------------ device passes
    def build(self, n_new, ctx, slot_base, tokens, buf=0):
        return A.sb_ragged_build(self.dims, n_new, ctx, slot_base, tokens, self.staging_bufs[buf].data_ptr(),
                                 self.meta.data_ptr(), self.meta_bytes, stream_handle())

    def forward(self, rg, layer_outputs=None, x_in=None, head=True, buf=0, prev=None):
        """embed (or x_in) -> every layer -> final norm / LM head / argmax on the ragged batch ``rg``.
        ``prev``: (device ids tensor, count) of the previous iteration, for token references; the new
        ids go to id buffer ``buf``."""
        s = stream_handle()
        T, H = rg.n_tokens, self.m.H
        xv = self.x[:T * H]
        ids_dev = self.ids_dev_bufs[buf]
        if x_in is None and layer_outputs is None and head:
            # the common case: the whole device side of the iteration in one library call
            ptrs = (prev[0].data_ptr() if prev is not None else None, prev[1] if prev is not None else 0,
                    xv.data_ptr(), self.logits.data_ptr(), ids_dev.data_ptr())
            if self.graphs and A.timing_mask == 0:
                self._forward_graph(rg, ptrs)
            else:
                self._sb_forward(rg, ptrs, s)
            return ids_dev[:rg.n_req]
        if x_in is not None:
            xv.copy_(x_in.reshape(-1))
        elif prev is not None:
            A.sb_embed_chained(self.dims, self.w.model_struct, rg, prev[0].data_ptr(), prev[1], xv.data_ptr(), s)
        else:
            A.sb_embed(self.dims, self.w.model_struct, rg, xv.data_ptr(), s)
        for l in range(self.n_layers):
            A.sb_layer_step(self.dims, self.w.layer_structs[l], rg, self.kv, l, xv.data_ptr(), self.ws.data_ptr(),
                            self.ws_bytes, s)
            if layer_outputs is not None:
                layer_outputs.append(xv.view(T, H).clone())
        if not head:
            return None
        A.sb_lm_argmax(self.dims, self.w.model_struct, rg, xv.data_ptr(), self.logits.data_ptr(),
                       ids_dev.data_ptr(), self.ws.data_ptr(), self.ws_bytes, s)
        return ids_dev[:rg.n_req]

    def _sb_forward(self, rg, ptrs, stream):
        prev_ids, prev_n, x, logits, ids = ptrs
        A.sb_forward(self.dims, self.w.model_struct, self.w.layer_array, self.n_layers, rg, self.kv, prev_ids, prev_n,
                     x, logits, ids, self.ws.data_ptr(), self.ws_bytes, stream)

    # graphs kept per engine; beyond this many shapes the cache starts over
    MAX_GRAPHS = 16

    def _forward_graph(self, rg, ptrs):
        """The launches of sb_forward depend only on the host fields of ``rg`` (counts and the device
        addresses of its arrays) and on the buffers in ``ptrs``; what the kernels read from those
        buffers (metadata, ids, K/V) may change freely.  So an iteration whose shape key matches a
        captured one replays that graph: one launch instead of one per kernel (a decode loop at a
        steady batch is launch-bound).  A shape is captured the second time it is seen, so a stream
        of ever-new shapes (arrivals) runs eagerly and pays no capture.  sb_forward issues kernel
        launches only (no memsets, copies or host waits), which is what makes it capturable."""
        key = (tuple(getattr(rg, f) for f, _ in rg._fields_), ptrs)
        g = self._graph_cache.get(key)
        if g is None:
            seen = self._graph_seen.get(key, 0) + 1
            self._graph_seen[key] = seen
            if seen < 2:
                self._sb_forward(rg, ptrs, stream_handle())
                return
            if len(self._graph_cache) >= self.MAX_GRAPHS:
                self._graph_cache.clear()
                self._graph_seen = {key: seen}
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._sb_forward(rg, ptrs, stream_handle())
            self._graph_cache[key] = g
        g.replay()

    def launch(self, sched=None, buf=0, keep=False, chain=None):
        """Select the next iteration from ``sched`` (default: this engine's scheduler), build its
        metadata in staging buffer ``buf`` and enqueue all of its GPU work, without waiting.  Returns
        None for an empty pool, else the pending iteration for ``finish``.  Two iterations may be in
        flight when they use different ``buf``; their GPU work runs in stream order.

        ``chain``: the previous iteration, already completed with ``complete_counts`` but whose token
        values may still be on the device: members that continue from it embed its ids straight from
        its device buffer (the other ``buf``), so this launch never waits for them."""
        sched = self.sched if sched is None else sched
        h0 = time.perf_counter()
        ids, n_new, ctx, base = A.sb_select_batch(sched, self.max_bs)
        if len(ids) == 0:
            return None
        n_rsrv = A.sb_sched_stats(sched)["n_rsrv"]
        prev = None
        if chain is not None:
            toks, ticket = A.sb_batch_token_refs(sched, ids, self.max_tokens)
            if ticket >= 0:
                assert ticket == chain["ticket"] and chain["buf"] != buf
                prev = (self.ids_dev_bufs[chain["buf"]], len(chain["ids"]))
        else:
            toks = A.sb_batch_tokens(sched, ids, self.max_tokens)
        rg = self.build(n_new, ctx, base, toks, buf)
        outs = [] if keep else None
        start = None
        if self.record_events:
            start = torch.cuda.Event(enable_timing=True)
            start.record()
        ids_dev = self.forward(rg, layer_outputs=outs, buf=buf, prev=prev)
        B = len(ids)
        self.ids_host_bufs[buf][:B].copy_(ids_dev[:B], non_blocking=True)
        done = torch.cuda.Event(enable_timing=self.record_events)
        done.record()
        return {"sched": sched, "buf": buf, "ids": ids, "n_new": n_new, "ctx": ctx, "slot_base": base,
                "event": done, "start": start, "outs": outs, "ticket": None, "n_rsrv": n_rsrv,
                "host_ms": 1e3 * (time.perf_counter() - h0)}

    def _result(self, p, new):
        res = {"ids": p["ids"], "n_new": p["n_new"], "ctx": p["ctx"], "slot_base": p["slot_base"], "tokens": new,
               "finished": p.get("finished"), "n_rsrv": p["n_rsrv"], "host_ms": p["host_ms"]}
        if p.get("start") is not None:
            res["gpu_ms"] = p["start"].elapsed_time(p["event"])
        if p["outs"] is not None:
            B = len(p["ids"])
            res["layer_outputs"] = [o.cpu() for o in p["outs"]]
            res["logits"] = self.logits[:B * self.m.V].view(B, self.m.V).cpu()
        return res

    def finish(self, p):
        """Wait for a launched iteration, hand its new tokens to its scheduler (Complete)."""
        p["event"].synchronize()
        B = len(p["ids"])
        new = self.ids_host_bufs[p["buf"]][:B].numpy().copy()
        p["finished"] = A.sb_sched_complete(p["sched"], p["ids"], new)
        return self._result(p, new)

    def complete_counts(self, p):
        """Complete a launched iteration without waiting for it: every member advances one token,
        finished ones free their slots (counts only); the values follow in ``settle``."""
        p["finished"], p["ticket"] = A.sb_sched_complete_deferred(p["sched"], p["ids"])

    def settle(self, p):
        """Wait for an iteration completed by ``complete_counts`` and record its token values."""
        p["event"].synchronize()
        B = len(p["ids"])
        new = self.ids_host_bufs[p["buf"]][:B].numpy().copy()
        A.sb_sched_set_tokens(p["sched"], p["ticket"], new)
        return self._result(p, new)

    def step(self, keep=False):
        """One scheduler iteration; returns None for an empty pool, else a dict of the batch and its results."""
        p = self.launch(keep=keep)
        return None if p is None else self.finish(p)

    def run_chained(self, reqs=(), on_iteration=None, max_iters=None):
        """Serve ``reqs`` (objects with rid, arrival, prompt, out_len, max_tokens) and whatever is already
        in the pool until all are done, one iteration ahead of the host: iteration t+1 is selected and
        launched -- its decodes embedding iteration t's ids on the device -- before the host waits for
        iteration t's ids.  Arrivals follow the iteration clock: a request joins the pool at the first
        iteration t >= its arrival; an idle clock jumps to the next arrival.  ``on_iteration(result)``
        receives each settled iteration (with its clock in result["t"]).  ``max_iters``: stop launching
        after that many iterations (the requests still in the pool stay there).  Returns the iteration count."""
        import math
        pending = sorted(reqs, key=lambda r: (r.arrival, r.rid))
        i, clock, n_iter, prev = 0, 0, 0, None
        while True:
            if prev is not None:
                self.complete_counts(prev)
            while i < len(pending) and pending[i].arrival <= clock:
                r = pending[i]
                self.add(r.rid, r.arrival, r.prompt, r.out_len, r.max_tokens)
                i += 1
            p = self.launch(buf=n_iter % 2, chain=prev) if max_iters is None or n_iter < max_iters else None
            if prev is not None:
                res = self.settle(prev)
                res["t"] = prev["t"]
                if on_iteration is not None:
                    on_iteration(res)
            if p is None:
                if i >= len(pending) or (max_iters is not None and n_iter >= max_iters):
                    return n_iter
                clock, prev = int(math.ceil(pending[i].arrival)), None
                continue
            p["t"] = clock
            prev, n_iter, clock = p, n_iter + 1, clock + 1

    def output(self, rid):
        return A.sb_sched_output(self.sched, rid)
