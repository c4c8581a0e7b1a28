"""Pins of the oracle's Transformer pieces: closed forms, brute force, structure, invariants."""
import math

import numpy as np
import pytest

from golden import load
from oracle import brute, flat as FL, generate as G, model as M
from synth import TOY, ModelDims, figure5_requests, make_weights, normal, p4_grid_requests, random_ragged_batch

TINY_GPT = ModelDims("tiny-gpt", "gpt", n_layers=2, H=16, nq=4, nkv=4, d=4, F=32, V=40, max_pos=64)
TINY_LLAMA = ModelDims("tiny-llama", "llama", n_layers=2, H=16, nq=4, nkv=2, d=4, F=24, V=40, max_pos=0,
                       rope_theta=10000.0)


# ---------------------------------------------------------------- scalar functions
def test_gelu_values():
    # Phi(1) = 0.8413447460685429, Phi(-1) = 0.15865525393145707 (standard normal CDF tables)
    assert M.gelu(1.0) == pytest.approx(0.8413447460685429, abs=1e-15)
    assert M.gelu(-1.0) == pytest.approx(-0.15865525393145707, abs=1e-15)
    assert M.gelu(0.0) == 0.0
    # Phi(2) = 0.9772498680518208
    assert M.gelu(2.0) == pytest.approx(2 * 0.9772498680518208, abs=1e-14)
    assert M.gelu(40.0) == pytest.approx(40.0)


def test_silu_values():
    assert M.silu(0.0) == 0.0
    assert M.silu(1.0) == pytest.approx(0.7310585786300049, abs=1e-15)   # 1 / (1 + e^-1)
    assert M.silu(-1.0) == pytest.approx(-0.2689414213699951, abs=1e-15)


def test_layer_norm_closed_forms():
    eps = 1e-5
    y = M.layer_norm(np.array([[1.0, -1.0]]), np.ones(2), np.zeros(2), eps)
    np.testing.assert_allclose(y, [[1 / math.sqrt(1 + eps), -1 / math.sqrt(1 + eps)]], rtol=1e-15)
    # constant row -> the shift only
    y = M.layer_norm(np.full((1, 5), 3.0), np.full(5, 7.0), np.arange(5.0), eps)
    np.testing.assert_allclose(y, [np.arange(5.0)], atol=1e-12)
    # gain and shift act per feature after normalisation: [3, 5] -> [-1, 1] (up to eps)
    y = M.layer_norm(np.array([[3.0, 5.0]]), np.array([2.0, 10.0]), np.array([0.5, -0.5]), 0.0)
    np.testing.assert_allclose(y, [[-1.5, 9.5]], atol=1e-15)
    x = normal(0, "ln", (7, 33), std=3.0, mean=1.5).astype(np.float64)
    y = M.layer_norm(x, np.ones(33), np.zeros(33), 0.0)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-13)
    np.testing.assert_allclose((y * y).mean(axis=1), 1, atol=1e-12)


def test_rms_norm_closed_forms():
    y = M.rms_norm(np.array([[3.0, 4.0]]), np.ones(2), 0.0)
    r = math.sqrt(12.5)
    np.testing.assert_allclose(y, [[3 / r, 4 / r]], rtol=1e-15)
    y = M.rms_norm(np.array([[3.0, 4.0]]), np.array([2.0, -1.0]), 0.0)
    np.testing.assert_allclose(y, [[6 / r, -4 / r]], rtol=1e-15)
    x = normal(1, "rms", (5, 40), std=2.0).astype(np.float64)
    y = M.rms_norm(x, np.ones(40), 0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(axis=1)), 1, atol=1e-13)


def test_linear_orientation():
    # weights are [out, in]: y_o = sum_i x_i w[o, i] + b_o
    x = np.array([[1.0, 2.0]])
    w = np.array([[1.0, 0.0], [0.0, 0.0], [0.0, 1.0], [3.0, -1.0]])
    np.testing.assert_array_equal(M.linear(x, w, np.array([0, 0, 0, 0.5])), [[1.0, 0.0, 2.0, 1.5]])


def test_rope_closed_forms():
    # d = 2: one pair rotated by angle pos * theta^0 = pos
    x = np.array([[[1.0, 0.0]]])
    y = M.rope(x, np.array([1]), 10000.0)
    np.testing.assert_allclose(y, [[[math.cos(1), math.sin(1)]]], rtol=1e-15)
    # position 0 is the identity
    x = normal(2, "rope", (3, 2, 8)).astype(np.float64)
    np.testing.assert_array_equal(M.rope(x, np.zeros(3, int), 500000.0), x)
    # d = 4, theta = 100: pairs (0,2) at angle pos, (1,3) at angle pos / 10
    x = np.array([[[1.0, 1.0, 0.0, 0.0]]])
    y = M.rope(x, np.array([2]), 100.0)
    np.testing.assert_allclose(y, [[[math.cos(2), math.cos(0.2), math.sin(2), math.sin(0.2)]]], rtol=1e-15)
    # rotation: norms preserved, and q.k depends only on the position difference
    q = normal(3, "rq", (1, 1, 16)).astype(np.float64)
    k = normal(3, "rk", (1, 1, 16)).astype(np.float64)
    np.testing.assert_allclose(np.linalg.norm(M.rope(q, np.array([37]), 500000.0)), np.linalg.norm(q))
    a = (M.rope(q, np.array([5]), 500000.0) * M.rope(k, np.array([2]), 500000.0)).sum()
    b = (M.rope(q, np.array([105]), 500000.0) * M.rope(k, np.array([102]), 500000.0)).sum()
    assert a == pytest.approx(b, rel=1e-12)


def test_greedy_ties_take_first():
    assert M.greedy(np.array([1.0, 3.0, 3.0, -1.0])) == 1


# ---------------------------------------------------------------- attention
def _rand_qkv(seed, L, ctx, nq, nkv, d):
    q = normal(seed, "q", (L, nq, d)).astype(np.float64)
    K = normal(seed, "k", (ctx + L, nkv, d)).astype(np.float64)
    V = normal(seed, "v", (ctx + L, nkv, d)).astype(np.float64)
    return q, K, V


@pytest.mark.parametrize("L,ctx,nq,nkv", [(1, 0, 2, 2), (1, 5, 4, 2), (3, 0, 2, 1), (4, 3, 4, 4), (2, 6, 6, 2)])
def test_attention_matches_brute_force(L, ctx, nq, nkv):
    q, K, V = _rand_qkv(L * 100 + ctx, L, ctx, nq, nkv, 5)
    got = M.attention(q, K, V, ctx, nq // nkv)
    want = np.array(brute.attention_loops(q.tolist(), K.tolist(), V.tolist(), ctx, nq // nkv))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_attention_single_token_no_history_is_v():
    q, K, V = _rand_qkv(7, 1, 0, 4, 2, 8)
    got = M.attention(q, K, V, 0, 2)
    np.testing.assert_allclose(got[0], V[0][[0, 0, 1, 1]], rtol=1e-15)


def test_attention_equal_keys_is_running_mean():
    L, ctx, d = 3, 4, 6
    q = normal(8, "q", (L, 1, d)).astype(np.float64)
    K = np.ones((ctx + L, 1, d))
    V = normal(8, "v", (ctx + L, 1, d)).astype(np.float64)
    got = M.attention(q, K, V, ctx, 1)
    for j in range(L):
        np.testing.assert_allclose(got[j, 0], V[:ctx + j + 1, 0].mean(axis=0), rtol=1e-13)


def test_attention_scale_is_inverse_sqrt_d():
    # d = 4, q = k1 = (1,1,1,1): score 4 / sqrt(4) = 2; k0 = 0: score 0.
    q = np.ones((1, 1, 4))
    K = np.array([[[0.0] * 4], [[1.0] * 4]])
    V = np.array([[[1.0, 0, 0, 0]], [[0.0, 1, 0, 0]]])
    got = M.attention(q, K, V, 1, 1)
    w1 = math.exp(2) / (1 + math.exp(2))
    np.testing.assert_allclose(got[0, 0], [1 - w1, w1, 0, 0], rtol=1e-14)


def test_attention_gqa_head_mapping():
    # kv head g holds constant value g: query head h must read kv head h // (nq / nkv)
    nq, nkv, d = 8, 2, 3
    q = normal(9, "q", (2, nq, d)).astype(np.float64)
    K = normal(9, "k", (5, nkv, d)).astype(np.float64)
    V = np.zeros((5, nkv, d))
    V[:, 1, :] = 1.0
    got = M.attention(q, K, V, 3, nq // nkv)
    np.testing.assert_allclose(got[:, :4], 0.0)
    np.testing.assert_allclose(got[:, 4:], 1.0, rtol=1e-15)


# ---------------------------------------------------------------- layer structure
def _zero_layer(m):
    from synth import make_layer_weights
    w = make_layer_weights(m, 0, 0, "fp32")
    return {k: np.zeros_like(v, dtype=np.float64) for k, v in w.items()}


@pytest.mark.parametrize("m", [TINY_GPT, TINY_LLAMA])
def test_layer_zero_weights_is_identity(m):
    w = _zero_layer(m)
    x = normal(10, "x", (3, m.H)).astype(np.float64)
    y = M.layer_forward(m, w, x, 0, M.new_cache(m, 1)[0])
    np.testing.assert_array_equal(y, x)


def test_layer_bias_paths_gpt():
    m = TINY_GPT
    w = _zero_layer(m)
    w["b_o"] = normal(11, "bo", (m.H,)).astype(np.float64)
    w["b1"] = normal(11, "b1", (m.F,)).astype(np.float64)
    w["b2"] = normal(11, "b2", (m.H,)).astype(np.float64)
    w["w2"][np.arange(m.H), np.arange(m.H)] = 1.0          # w2 selects the first H FFN features
    x = normal(11, "x", (2, m.H)).astype(np.float64)
    y = M.layer_forward(m, w, x, 0, M.new_cache(m, 1)[0])
    np.testing.assert_allclose(y, x + w["b_o"] + M.gelu(w["b1"][:m.H]) + w["b2"], rtol=1e-14)


@pytest.mark.parametrize("m", [TINY_GPT, TINY_LLAMA])
def test_layer_value_path_and_second_norm_input(m):
    """V = first norm's output, K = 0 (uniform attention), W_o = I: the attention adds the causal
    mean of the normalised rows; the feed-forward must then see x + that mean."""
    w = _zero_layer(m)
    w["ln1_g"] = np.ones(m.H)
    w["ln2_g"] = np.ones(m.H)
    v0 = (m.nq + m.nkv) * m.d
    # V block = identity on the first nkv*d features; W_o maps q-head features back (GQA copies)
    w["w_qkv"][v0 + np.arange(m.nkv * m.d), np.arange(m.nkv * m.d)] = 1.0
    for h in range(m.nq):
        g = h // m.group
        for e in range(m.d):
            if h % m.group == 0:
                w["w_o"][g * m.d + e, h * m.d + e] = 1.0
    # FFN: identity through the activation on the first H features
    if m.arch == "gpt":
        w["w1"][np.arange(m.H), np.arange(m.H)] = 1.0
    else:
        w["w1"][np.arange(m.H), np.arange(m.H)] = 1.0            # gate
        w["w1"][m.F + np.arange(m.H), np.arange(m.H)] = 1.0      # up
    w["w2"][np.arange(m.H), np.arange(m.H)] = 1.0
    x = normal(12, "x", (4, m.H), std=2.0).astype(np.float64)
    y = M.layer_forward(m, w, x, 0, M.new_cache(m, 1)[0])
    n1 = (M.layer_norm(x, np.ones(m.H), np.zeros(m.H), m.eps) if m.arch == "gpt"
          else M.rms_norm(x, np.ones(m.H), m.eps))
    kv = m.nkv * m.d
    mean = np.cumsum(n1[:, :kv], axis=0) / np.arange(1, 5)[:, None]
    x1 = x.copy()
    x1[:, :kv] += mean
    n2 = (M.layer_norm(x1, np.ones(m.H), np.zeros(m.H), m.eps) if m.arch == "gpt"
          else M.rms_norm(x1, np.ones(m.H), m.eps))
    act = M.gelu(n2) if m.arch == "gpt" else M.silu(n2) * n2
    np.testing.assert_allclose(y, x1 + act, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("m", [TINY_GPT, TINY_LLAMA])
def test_layer_is_causal(m):
    W = make_weights(m, 3, "fp32")
    x = normal(13, "x", (5, m.H)).astype(np.float64)
    y = M.layer_forward(m, W["layers"][0], x, 0, M.new_cache(m, 1)[0])
    x2 = x.copy()
    x2[3:] += 1.0
    y2 = M.layer_forward(m, W["layers"][0], x2, 0, M.new_cache(m, 1)[0])
    np.testing.assert_array_equal(y[:3], y2[:3])
    assert not np.allclose(y[3:], y2[3:])


@pytest.mark.parametrize("m", [TINY_GPT, TINY_LLAMA])
def test_decode_equals_last_row_of_full_prefill(m):
    """The K/V history of earlier iterations must reproduce the full-sequence result."""
    W = make_weights(m, 4, "fp32")
    ids = [3, 17, 5, 9, 22, 1]
    full, logits_full = M.forward_request(m, W, ids, 0, M.new_cache(m))
    cache = M.new_cache(m)
    M.forward_request(m, W, ids[:4], 0, cache)
    M.forward_request(m, W, ids[4:5], 4, cache)
    outs, logits = M.forward_request(m, W, ids[5:], 5, cache)
    for l in range(m.n_layers):
        np.testing.assert_allclose(outs[l][-1], full[l][-1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(logits, logits_full, rtol=1e-12, atol=1e-12)


def test_lm_head_uses_final_norm_of_last_row():
    m = ModelDims("t", "gpt", n_layers=0, H=6, nq=1, nkv=1, d=6, F=6, V=6, max_pos=8)
    W = {"lnf_g": np.full(6, 2.0), "lnf_b": np.arange(6.0), "w_lm": np.eye(6), "layers": []}
    x = normal(14, "x", (6,)).astype(np.float64)
    want = M.layer_norm(x[None], np.ones(6), np.zeros(6), m.eps)[0] * 2.0 + np.arange(6.0)
    np.testing.assert_allclose(M.lm_logits(m, W, x), want, rtol=1e-14)


# ---------------------------------------------------------------- ragged metadata (integer pins)
def test_figure5_counts():
    g = load("figure5.txt")
    batch = list(zip(g["n_new"], g["ctx"]))
    assert FL.cu_seqlens(batch) == g["cu_seqlens"]
    assert FL.cu_seqlens(batch)[-1] == g["tokens"][0]
    assert FL.padded_tokens(batch) == g["padded_tokens"][0]
    assert FL.useful_pairs(batch) == g["useful_pairs"][0]
    assert FL.positions(batch) == [3, 1, 0, 1, 0, 1, 2]
    assert FL.last_rows(batch) == [0, 1, 3, 6]


def test_exercise4_counts():
    g = load("exercise4.txt")
    batch = list(zip(g["n_new"], g["ctx"]))
    T = FL.cu_seqlens(batch)[-1]
    assert T == g["tokens"][0]
    assert FL.padded_tokens(batch) == g["padded_tokens"][0]
    assert round(100 * (1 - T / FL.padded_tokens(batch))) == g["padding_waste_percent"][0]
    assert FL.useful_pairs(batch) == g["useful_pairs"][0]
    assert FL.padded_pairs(batch) == g["padded_pairs"][0]
    assert round(10 * FL.padded_pairs(batch) / FL.useful_pairs(batch)) == g["pair_ratio_x10"][0]


# ---------------------------------------------------------------- flattened self-check
def _batch_run(m, W, batch, seed):
    """Per-request reference and flattened forward on the same synthetic histories."""
    rng_ids = []
    caches_a, caches_b = [], []
    for i, (n_new, ctx) in enumerate(batch):
        hist = [int(v) for v in (np.arange(ctx) * 7 + i) % m.V]
        ca, cb = M.new_cache(m), M.new_cache(m)
        if ctx:
            M.forward_request(m, W, hist, 0, ca)
            M.forward_request(m, W, hist, 0, cb)
        caches_a.append(ca)
        caches_b.append(cb)
        rng_ids.append([int(v) for v in (np.arange(n_new) * 13 + 5 * i + seed) % m.V])
    per_req = [M.forward_request(m, W, rng_ids[i], batch[i][1], caches_a[i]) for i in range(len(batch))]
    outs, logits = FL.forward_flat(m, W, rng_ids, batch, caches_b)
    return per_req, outs, logits


@pytest.mark.parametrize("m", [TINY_GPT, TINY_LLAMA])
@pytest.mark.parametrize("which", ["figure5", "exercise4", "random"])
def test_flat_equals_per_request(m, which):
    if which == "figure5":
        batch = [(1, 3), (1, 1), (2, 0), (3, 0)]
    elif which == "exercise4":
        batch = [(n, min(c, 20)) for n, c in [(37, 0), (9, 0), (1, 120), (1, 15), (1, 64)]]
    else:
        batch = random_ragged_batch(5, 6, 12, 7)
    W = make_weights(m, 5, "fp32")
    per_req, outs, logits = _batch_run(m, W, batch, 1)
    cu = FL.cu_seqlens(batch)
    for i in range(len(batch)):
        for l in range(m.n_layers):
            np.testing.assert_allclose(outs[l][cu[i]:cu[i + 1]], per_req[i][0][l], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(logits[i], per_req[i][1], rtol=1e-12, atol=1e-13)


def test_flat_request_isolation():
    m = TINY_LLAMA
    W = make_weights(m, 6, "fp32")
    batch = [(3, 0), (2, 0)]
    caches = [M.new_cache(m), M.new_cache(m)]
    o1, _ = FL.forward_flat(m, W, [[1, 2, 3], [4, 5]], batch, caches)
    caches = [M.new_cache(m), M.new_cache(m)]
    o2, _ = FL.forward_flat(m, W, [[1, 2, 3], [9, 30]], batch, caches)
    np.testing.assert_array_equal(o1[-1][:3], o2[-1][:3])


# ---------------------------------------------------------------- generation invariant
def test_continuous_equals_one_at_a_time_figure5():
    m = TOY
    W = make_weights(m, 0, "fp32")
    reqs = figure5_requests(seed=0, vocab=m.V, out_len=8)
    rec = []
    toks, log = G.generate_continuous(m, W, reqs, max_bs=4, n_slots=64, record=rec)
    # iteration 1 is the Figure-5 batch
    assert [(n, c) for _, n, c in rec[1]["work"]] == [(1, 3), (1, 1), (2, 0), (3, 0)]
    for r in reqs:
        solo, margins = G.generate_one_at_a_time(m, W, r.prompt, r.out_len)
        assert toks[r.rid] == solo
        assert min(margins) > 1e-6


def test_continuous_equals_one_at_a_time_timeline():
    m = TINY_LLAMA
    W = make_weights(m, 1, "fp32")
    reqs = p4_grid_requests(seed=0, vocab=m.V)
    toks, log = G.generate_continuous(m, W, reqs, max_bs=3, n_slots=10**6)
    assert len(log) == 10
    for r in reqs:
        solo, _ = G.generate_one_at_a_time(m, W, r.prompt, r.out_len)
        assert toks[r.rid] == solo


# ---------------------------------------------------------------- storage precision
def test_round_to_bf16_matches_library_and_ties():
    import torch
    from oracle.precision import round_to_bf16, store
    x = np.concatenate([normal(20, "r", (5000,), std=s).astype(np.float64) for s in (1e-30, 1e-3, 1.0, 1e4, 1e30)])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_to_bf16(x), want)
    # halfway cases go to the even neighbour: 1 + 2^-8 -> 1; 1 + 3*2^-8 -> 1 + 2^-6
    np.testing.assert_array_equal(round_to_bf16([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)]),
                                  [1.0, 1 + 2 ** -6, -1.0])
    np.testing.assert_array_equal(store(x, None), x)
    np.testing.assert_array_equal(store(x, "fp32"), x.astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("m", [TINY_GPT, TINY_LLAMA])
def test_storage_mode_fp32_is_exact_and_bf16_is_close(m):
    W = make_weights(m, 7, "bf16")
    batch = [(3, 0), (1, 4)]
    ids = [[1, 2, 3], [7]]
    res = {}
    for st in (None, "fp32", "bf16"):
        caches = [M.new_cache(m), M.new_cache(m)]
        for i, (n, c) in enumerate(batch):
            if c:
                M.forward_request(m, W, list(range(c)), 0, caches[i], st)
        res[st] = FL.forward_flat(m, W, ids, batch, caches, st)
    for l in range(m.n_layers):
        ex = res[None][0][l]
        scale = np.sqrt(np.mean(ex ** 2))
        assert np.max(np.abs(res["fp32"][0][l] - ex)) <= 1e-6 * scale
        err_bf16 = np.max(np.abs(res["bf16"][0][l] - ex))
        assert 1e-5 * scale < err_bf16 <= 5e-2 * scale        # it does round, and only at bf16 level
