"""Request mixes of the workloads (seeded, synthetic).

A batch entry is ``(n_new, ctx)``: the number of tokens a request feeds this
iteration and the number of its tokens already held by the K/V manager.  A
prefill is ``(L, 0)``, a decode ``(1, ctx)``, a chunk of a split prefill
``(L, ctx)`` with both positive.
"""
from dataclasses import dataclass, field
from typing import List

import numpy as np

from .gen import normal, rng_for, uniform_int


@dataclass
class Req:
    rid: int
    arrival: float
    prompt: List[int]
    out_len: int
    max_tokens: int
    generated: List[int] = field(default_factory=list)


def figure5_requests(seed: int = 0, vocab: int = 256, out_len: int = 8, extra: int = 8):
    """Four requests that produce the Figure-5 batch at iteration 1.

    x1 (3-token prompt) and x2 (1-token prompt) arrive at t=0, x3 (2 tokens)
    and x4 (3 tokens) at t=1.  At iteration 1 the batch is x1 decode with 3
    cached tokens, x2 decode with 1 cached, x3 prefill 2, x4 prefill 3: seven
    tokens.  ``max_tokens = prompt + extra``.
    """
    lens = [3, 1, 2, 3]
    arrivals = [0.0, 0.0, 1.0, 1.0]
    ids = uniform_int(seed, "fig5.prompts", 0, vocab - 1, sum(lens)).tolist()
    reqs, o = [], 0
    for i, (n, a) in enumerate(zip(lens, arrivals)):
        reqs.append(Req(i, a, ids[o:o + n], out_len, n + extra))
        o += n
    return reqs


def p4_grid_requests(seed: int = 0, vocab: int = 256):
    """Six requests of the lecture's continuous-batching timeline (max_bs = 3).

    Arrival iterations (0, 0, 1, 2, 3, 6), output lengths (6, 3, 9, 2, 5, 3).
    Prompt lengths are not given by the lecture; they do not affect the
    schedule, so short random prompts are used.
    """
    arrivals = [0, 0, 1, 2, 3, 6]
    outs = [6, 3, 9, 2, 5, 3]
    plen = uniform_int(seed, "p4.plen", 1, 6, 6).tolist()
    reqs = []
    for i in range(6):
        p = uniform_int(seed, f"p4.prompt{i}", 0, vocab - 1, plen[i]).tolist()
        reqs.append(Req(i, float(arrivals[i]), p, outs[i], plen[i] + outs[i]))
    return reqs


def exercise4_batch():
    """(n_new, ctx) of the lecture's exercise-4 step: prefills 37 and 9, decodes at ctx 120, 15, 64."""
    return [(37, 0), (9, 0), (1, 120), (1, 15), (1, 64)]


def mini_decode_batch(seed: int = 0, n: int = 64, ctx_lo: int = 16, ctx_hi: int = 256):
    """64 decodes with cached lengths uniform in [16, 256]."""
    ctx = uniform_int(seed, "mini.ctx", ctx_lo, ctx_hi, n).tolist()
    return [(1, c) for c in ctx]


def llama_mixed_batch(seed: int = 0, n_dec: int = 240, n_pre: int = 16):
    """240 decodes (ctx uniform [128, 2048]) then 16 prefills (prompt uniform [32, 512])."""
    ctx = uniform_int(seed, "llama.ctx", 128, 2048, n_dec).tolist()
    pl = uniform_int(seed, "llama.plen", 32, 512, n_pre).tolist()
    return [(1, c) for c in ctx] + [(L, 0) for L in pl]


def gpt175b_mixed_batch(seed: int = 0, n_dec: int = 96, n_pre: int = 32):
    """96 decodes (ctx uniform [512, 2048]) then 32 prefills (prompt uniform [128, 1024])."""
    ctx = uniform_int(seed, "g175.ctx", 512, 2048, n_dec).tolist()
    pl = uniform_int(seed, "g175.plen", 128, 1024, n_pre).tolist()
    return [(1, c) for c in ctx] + [(L, 0) for L in pl]


def random_ragged_batch(seed: int, n_req: int, max_ctx: int, max_new: int, name: str = "rag"):
    """Mixed batch of decodes, prefills and prefill chunks (ctx > 0, n_new > 1)."""
    g = rng_for(seed, name)
    out = []
    for _ in range(n_req):
        kind = g.integers(0, 3)
        if kind == 0:
            out.append((1, int(g.integers(0, max_ctx + 1))))
        elif kind == 1:
            out.append((int(g.integers(1, max_new + 1)), 0))
        else:
            out.append((int(g.integers(1, max_new + 1)), int(g.integers(1, max_ctx + 1))))
    return out


def poisson_trace(seed: int = 0, n: int = 2000, rate: float = 0.5, vocab: int = 128256,
                  plo: int = 32, phi: int = 512, olo: int = 1, ohi: int = 512, reserve_out: int = 512,
                  with_prompts: bool = False):
    """Poisson arrivals on the iteration clock (rate requests per iteration).

    prompt ~ U[plo, phi], out_len ~ U[olo, ohi], max_tokens = prompt + reserve_out.
    Prompt token ids are drawn only when ``with_prompts`` (they do not affect
    scheduling).
    """
    g = rng_for(seed, "trace.gaps")
    gaps = g.exponential(1.0 / rate, size=n)
    arrivals = np.cumsum(gaps)
    pl = uniform_int(seed, "trace.plen", plo, phi, n).tolist()
    ol = uniform_int(seed, "trace.olen", olo, ohi, n).tolist()
    reqs = []
    for i in range(n):
        prompt = (uniform_int(seed, f"trace.prompt{i}", 0, vocab - 1, pl[i]).tolist()
                  if with_prompts else [0] * pl[i])
        reqs.append(Req(i, float(arrivals[i]), prompt, int(ol[i]), int(pl[i]) + reserve_out))
    return reqs


def synthetic_kv(seed: int, name: str, n_tok: int, nkv: int, d: int, std: float, dtype: str):
    """Cached K and V rows ``[n_tok, nkv, d]`` for a request whose history is synthetic."""
    k = normal(seed, name + ".k", (n_tok, nkv, d), std=std, dtype=dtype)
    v = normal(seed, name + ".v", (n_tok, nkv, d), std=std, dtype=dtype)
    return k, v
