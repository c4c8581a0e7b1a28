"""Selective batching in numpy: token-wise operators on ``[sum L_i, H]``,
Split by request offsets around attention, Merge back.

Sources: "连续批处理完全拆解" (section 观察 and the Figure 5 walk-through: the
non-attention operators run on the flattened tensor; attention runs per
request against the K/V manager's history; outputs are merged back),
"CS349D Lecture 2" section 3.2 (padding counts) and exercise 4 (useful versus
padded (query, key) pairs).

This module is the oracle's self-check of the offset arithmetic: its layer
output must equal ``model.layer_forward`` run request by request, to fp64
round-off.
"""
import numpy as np

from . import model as M
from .precision import store as _store

F64 = np.float64


def cu_seqlens(batch):
    """Prefix sums of the per-request new-token counts: request i owns rows cu[i]..cu[i+1]-1."""
    cu = [0]
    for n_new, _ in batch:
        cu.append(cu[-1] + n_new)
    return cu


def positions(batch):
    """Position of every flattened row: ctx_i + j for the j-th new token of request i."""
    return [ctx + j for n_new, ctx in batch for j in range(n_new)]


def last_rows(batch):
    """Row of each request's last new token (the one whose logits pick its next token)."""
    cu = cu_seqlens(batch)
    return [cu[i + 1] - 1 for i in range(len(batch))]


def useful_pairs(batch):
    """(query, key) pairs the causal mask allows: query j of request i sees ctx_i + j + 1 keys."""
    return sum(sum(ctx + j + 1 for j in range(n_new)) for n_new, ctx in batch)


def padded_tokens(batch):
    """Rows of the padded [B, max L, H] layout."""
    return len(batch) * max(n for n, _ in batch)


def padded_pairs(batch):
    """(query, key) pairs when every request is padded to max L queries and max (ctx+L) keys."""
    return len(batch) * max(n for n, _ in batch) * max(n + c for n, c in batch)


def layer_forward_flat(m, w, x, batch, caches, store=None):
    """One layer over the flattened batch.

    x: [T, H] rows of all requests' new tokens in batch order; batch: list of
    (n_new, ctx); caches: per-request dicts 'k','v' of this layer, extended in place;
    store: storage dtype of the tensors handed between operators (None: exact).
    """
    x = np.asarray(x, F64)
    T = x.shape[0]
    cu = cu_seqlens(batch)
    assert cu[-1] == T
    pos = np.asarray(positions(batch))
    # token-wise: norm + QKV projection on all T rows at once
    q, k, v = M.qkv_project(m, w, _store(M.norm1(m, w, x), store), pos, store)
    o = np.empty((T, m.nq, m.d), F64)
    # Split -> per-request attention against that request's own history -> Merge
    for i, (n_new, ctx) in enumerate(batch):
        rows = slice(cu[i], cu[i + 1])
        c = caches[i]
        assert c["k"].shape[0] == ctx
        c["k"] = np.concatenate([c["k"], k[rows]], axis=0)
        c["v"] = np.concatenate([c["v"], v[rows]], axis=0)
        o[rows] = M.attention(q[rows], c["k"], c["v"], ctx, m.group)
    # token-wise again on the merged tensor
    x = x + M.linear(_store(o, store).reshape(T, m.nq * m.d), w["w_o"], w.get("b_o"))
    x = x + M.ffn(m, w, _store(M.norm2(m, w, x), store), store)
    return x


def forward_flat(m, W, batch_ids, batch, caches, store=None):
    """Whole model over a flattened batch.

    batch_ids: per-request lists of new token ids; caches[i][layer] per request.
    Returns (list of per-layer [T, H] outputs, [B, V] logits of each request's last row).
    """
    ids = np.concatenate([np.asarray(t, np.int64) for t in batch_ids])
    pos = np.asarray(positions(batch))
    x = np.asarray(W["tok_emb"], F64)[ids]
    if m.arch == "gpt":
        x = x + np.asarray(W["pos_emb"], F64)[pos]
    outs = []
    for l, w in enumerate(W["layers"]):
        x = layer_forward_flat(m, w, x, batch, [c[l] for c in caches], store)
        outs.append(x)
    lr = last_rows(batch)
    logits = M.linear(_store(M.final_norm(m, W, x[lr]), store), W["w_lm"])
    return outs, logits
