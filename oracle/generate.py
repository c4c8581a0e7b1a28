"""Greedy generation, one request at a time and under continuous batching.

The prefill iteration processes the whole prompt and yields the first token;
every later iteration feeds the last generated token and yields one more
("连续批处理完全拆解", Figure 3; "从静态批处理到连续批处理", Prefill/Decode).
Continuous batching changes only when each token is computed, so both
functions must return the same tokens ("CS349D Lecture 2", section 4.1 and
common pitfall 3).
"""
import numpy as np

from . import model as M
from . import flat as FL
from .scheduler import replay


def generate_one_at_a_time(m, W, prompt, out_len, store=None):
    """Returns (tokens, margins): ``out_len`` greedy tokens for one request run alone."""
    cache = M.new_cache(m)
    toks, margins = [], []
    _, logits = M.forward_request(m, W, list(prompt), 0, cache, store)
    toks.append(M.greedy(logits))
    margins.append(M.top2_margin(logits))
    ctx = len(prompt)
    while len(toks) < out_len:
        _, logits = M.forward_request(m, W, [toks[-1]], ctx, cache, store)
        toks.append(M.greedy(logits))
        margins.append(M.top2_margin(logits))
        ctx += 1
    return toks, margins


def generate_continuous(m, W, reqs, max_bs, n_slots, record=None, store=None, budget=None, chunk=None):
    """Greedy generation of ``reqs`` under the iteration-level scheduler.

    Each iteration runs the flattened selective-batched forward over the
    batch.  ``record`` (a list) receives per-iteration dicts with the batch
    work list, the flattened layer outputs and the last-row logits.
    Returns (tokens per rid, scheduler log).
    """
    by_id = {r.rid: r for r in reqs}
    toks = {r.rid: [] for r in reqs}
    caches = {r.rid: M.new_cache(m) for r in reqs}

    def engine(t, work):
        batch = [(n_new, ctx) for _, n_new, ctx in work]
        ids = []
        for rid, n_new, ctx in work:
            prompt = list(by_id[rid].prompt)
            # a prompt (or a chunk of it) with the tokens before it cached, else the last generated token
            ids.append(prompt[ctx:ctx + n_new] if ctx < len(prompt) else [toks[rid][-1]])
        outs, logits = FL.forward_flat(m, W, ids, batch, [caches[rid] for rid, _, _ in work], store)
        for i, (rid, n_new, ctx) in enumerate(work):
            if ctx + n_new >= len(by_id[rid].prompt):      # a chunk that ends short of the prompt yields nothing
                toks[rid].append(M.greedy(logits[i]))
        if record is not None:
            record.append({"t": t, "work": work, "ids": ids, "outs": outs, "logits": logits})

    log = replay(reqs, max_bs, n_slots, engine, budget, chunk)
    return toks, log
