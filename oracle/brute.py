"""Attention by explicit loops, for tiny inputs.

Scaled dot-product attention of one request with a causal mask, computed one
(query, head) at a time with ``math.exp`` and Python sums, independently of
the vectorised ``model.attention``.  Query j of a request with ``ctx`` cached
tokens sees keys 0..ctx+j ("CS349D Lecture 2", exercise 4: the causal mask
allows ctx + j + 1 keys for the j-th new token).
"""
import math


def attention_loops(q, K, V, ctx, group):
    """q: [L][nq][d], K, V: [ctx+L][nkv][d] nested lists or arrays; returns [L][nq][d] lists."""
    L = len(q)
    nq = len(q[0])
    d = len(q[0][0])
    out = []
    for j in range(L):
        row = []
        for h in range(nq):
            kh = h // group
            n_vis = ctx + j + 1
            scores = []
            for t in range(n_vis):
                s = 0.0
                for e in range(d):
                    s += float(q[j][h][e]) * float(K[t][kh][e])
                scores.append(s / math.sqrt(d))
            mx = max(scores)
            ws = [math.exp(s - mx) for s in scores]
            z = sum(ws)
            o = []
            for e in range(d):
                acc = 0.0
                for t in range(n_vis):
                    acc += ws[t] * float(V[t][kh][e])
                o.append(acc / z)
            row.append(o)
        out.append(row)
    return out
