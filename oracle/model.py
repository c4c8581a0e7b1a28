"""The plain per-request Transformer decoder, in fp64 numpy.

One request is run alone: its new tokens at positions ``ctx .. ctx+L-1``
attend to the ``ctx`` keys/values its earlier iterations left in its own
cache plus the new ones (causal, including itself).  This is the result
selective batching must reproduce ("连续批处理完全拆解", sections 观察 and
Figure 5; "CS349D Lecture 2", section 4.2).

The pages name the operators (Linear, LayerNorm/RMSNorm, GeLU, residual Add,
attention) but not the model's details; the readings used here are:
  * pre-norm blocks; LayerNorm / RMSNorm epsilon 1e-5 inside the square root;
  * GeLU is the exact x * Phi(x) (erf form); SwiGLU is SiLU(gate) * up;
  * attention scores are scaled by 1/sqrt(head_dim); query head h reads K/V
    head h // (nq / nkv);
  * GPT-style: learned absolute positions added to the token embedding;
    Llama-style: rotary embedding of q and k (rotate-half form, base theta),
    no biases;
  * the LM head is its own matrix (not tied to the embedding); greedy
    decoding takes the first index of the maximum logit.
"""
import numpy as np
from scipy.special import erf

from .precision import store as _store

F64 = np.float64


def layer_norm(x, g, b, eps):
    """(x - mean) / sqrt(var + eps) * g + b over the last axis (population variance)."""
    x = np.asarray(x, F64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(g, F64) + np.asarray(b, F64)


def rms_norm(x, g, eps):
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    x = np.asarray(x, F64)
    ms = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, F64)


def gelu(x):
    """Exact GeLU: x * Phi(x) with Phi the standard normal CDF."""
    x = np.asarray(x, F64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def silu(x):
    x = np.asarray(x, F64)
    return x / (1.0 + np.exp(-x))


def rope(x, pos, theta):
    """Rotary position embedding, rotate-half form.

    x: [L, heads, d]; pos: [L] integer positions.  Dimension pair (i, i + d/2)
    is rotated by angle pos * theta^(-2i/d).
    """
    x = np.asarray(x, F64)
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-(np.arange(half, dtype=F64) * 2.0) / d)
    ang = np.asarray(pos, F64)[:, None] * inv[None, :]          # [L, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(q, K, V, ctx, group):
    """Causal attention of one request.

    q: [L, nq, d] queries of the new tokens (positions ctx..ctx+L-1);
    K, V: [ctx+L, nkv, d] the request's whole history including the new tokens.
    Query j sees keys 0..ctx+j.  Returns [L, nq, d].
    """
    q = np.asarray(q, F64)
    K = np.asarray(K, F64)
    V = np.asarray(V, F64)
    L, nq, d = q.shape
    n = K.shape[0]
    assert n == ctx + L
    out = np.empty((L, nq, d), F64)
    visible = np.arange(n)[None, :] <= (ctx + np.arange(L))[:, None]   # [L, n]
    scale = 1.0 / np.sqrt(d)
    for h in range(nq):
        kh = h // group
        s = (q[:, h, :] @ K[:, kh, :].T) * scale
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ V[:, kh, :]
    return out


def norm1(m, w, x):
    if m.arch == "gpt":
        return layer_norm(x, w["ln1_g"], w["ln1_b"], m.eps)
    return rms_norm(x, w["ln1_g"], m.eps)


def norm2(m, w, x):
    if m.arch == "gpt":
        return layer_norm(x, w["ln2_g"], w["ln2_b"], m.eps)
    return rms_norm(x, w["ln2_g"], m.eps)


def final_norm(m, W, x):
    if m.arch == "gpt":
        return layer_norm(x, W["lnf_g"], W["lnf_b"], m.eps)
    return rms_norm(x, W["lnf_g"], m.eps)


def linear(x, w, b=None):
    y = np.asarray(x, F64) @ np.asarray(w, F64).T
    if b is not None:
        y = y + np.asarray(b, F64)
    return y


def qkv_project(m, w, h, pos, store=None):
    """q [L,nq,d], k [L,nkv,d], v [L,nkv,d] of the new tokens (RoPE applied for Llama).

    ``store``: storage dtype of the projection and of the rotated q, k (None: exact)."""
    L = h.shape[0]
    qkv = _store(linear(h, w["w_qkv"], w.get("b_qkv")), store)
    nq_d, nkv_d = m.nq * m.d, m.nkv * m.d
    q = qkv[:, :nq_d].reshape(L, m.nq, m.d)
    k = qkv[:, nq_d:nq_d + nkv_d].reshape(L, m.nkv, m.d)
    v = qkv[:, nq_d + nkv_d:].reshape(L, m.nkv, m.d)
    if m.arch == "llama":
        q = _store(rope(q, pos, m.rope_theta), store)
        k = _store(rope(k, pos, m.rope_theta), store)
    return q, k, v


def ffn(m, w, h, store=None):
    """Feed-forward block; the activation output (the second linear's input) is stored in ``store``."""
    if m.arch == "gpt":
        g = gelu(linear(h, w["w1"], w["b1"]))
        return linear(_store(g, store), w["w2"], w["b2"])
    gu = linear(h, w["w1"])
    g = silu(gu[:, :m.F]) * gu[:, m.F:]
    return linear(_store(g, store), w["w2"])


def layer_forward(m, w, x, ctx, cache, store=None):
    """One decoder layer for one request.

    x: [L, H] hidden rows of the new tokens; cache: dict with 'k', 'v' arrays
    [ctx, nkv, d] of this layer (extended in place with the new rows).
    ``store``: storage dtype of the tensors handed between operators (None: exact).
    Returns the layer's output rows [L, H].
    """
    x = np.asarray(x, F64)
    L = x.shape[0]
    assert cache["k"].shape[0] == ctx
    pos = ctx + np.arange(L)
    q, k, v = qkv_project(m, w, _store(norm1(m, w, x), store), pos, store)
    cache["k"] = np.concatenate([cache["k"], k], axis=0)
    cache["v"] = np.concatenate([cache["v"], v], axis=0)
    o = _store(attention(q, cache["k"], cache["v"], ctx, m.group), store)
    x = x + linear(o.reshape(L, m.nq * m.d), w["w_o"], w.get("b_o"))
    x = x + ffn(m, w, _store(norm2(m, w, x), store), store)
    return x


def new_cache(m, n_layers=None):
    n = m.n_layers if n_layers is None else n_layers
    return [{"k": np.zeros((0, m.nkv, m.d), F64), "v": np.zeros((0, m.nkv, m.d), F64)} for _ in range(n)]


def embed(m, W, ids, ctx):
    x = np.asarray(W["tok_emb"], F64)[np.asarray(ids)]
    if m.arch == "gpt":
        x = x + np.asarray(W["pos_emb"], F64)[ctx + np.arange(len(ids))]
    return x


def lm_logits(m, W, x_last, store=None):
    return linear(_store(final_norm(m, W, np.asarray(x_last, F64)[None, :]), store), W["w_lm"])[0]


def greedy(logits):
    """First index of the maximum."""
    return int(np.argmax(logits))


def forward_request(m, W, ids, ctx, cache, store=None):
    """All layers for one request's new tokens; returns (layer outputs, logits of the last token)."""
    x = embed(m, W, ids, ctx)
    outs = []
    for l, w in enumerate(W["layers"]):
        x = layer_forward(m, w, x, ctx, cache[l], store)
        outs.append(x)
    return outs, lm_logits(m, W, x[-1], store)


def top2_margin(logits):
    """Gap between the largest and second-largest logit (how safe the argmax is)."""
    s = np.sort(np.asarray(logits, F64))
    return float(s[-1] - s[-2]) if s.size > 1 else float("inf")
