"""GPU parity of whole layers, the model step and generation against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import selective_batching_amd as sb
from gpu_util import TDT, TOL, assert_close_attention, assert_close_elem, assert_close_rms, dev, host, print_case
from oracle import flat as FL
from oracle import generate as OG
from oracle import model as M
from synth import (LLAMA8B, MINI, TOY, GPT175B_LAYER, ModelDims, figure5_requests, gpt175b_mixed_batch,
                   llama_mixed_batch, make_layer_weights, make_weights, mini_decode_batch, normal, random_ragged_batch,
                   synthetic_kv, uniform_int, kv_std, init_std)
from synth.workloads import Req
from selective_batching_amd.runtime import DeviceWeights, Engine, stream_handle

pytestmark = pytest.mark.gpu

TINY_LLAMA = ModelDims("tiny-llama", "llama", n_layers=2, H=256, nq=8, nkv=2, d=32, F=512, V=512, max_pos=0,
                       rope_theta=10000.0)
TINY_LLAMA128 = ModelDims("tiny-llama128", "llama", n_layers=1, H=512, nq=8, nkv=2, d=128, F=512, V=512, max_pos=0)


def _history_engine(m, dtype, W, batch, seed, n_extra_slots=64):
    """Engine holding the batch's requests with synthetic K/V history in every layer."""
    eng = Engine(m, dtype, W, n_slots=sum(n + c for n, c in batch) + n_extra_slots, max_bs=len(batch),
                 max_tokens=sum(n for n, _ in batch), max_keys_total=sum(n + c for n, c in batch))
    caches = []
    bases = []
    eng.keep = []                         # device buffers the queued copies read
    for i, (n, c) in enumerate(batch):
        base = sb.sb_kv_reserve(eng.kv, 1000 + i, n + c)
        bases.append(base)
        cache = []
        for l in range(len(W.layers)):
            hk, hv = synthetic_kv(seed, f"L{l}.h{i}", c, m.nkv, m.d, 1.0, dtype)
            cache.append({"k": hk.astype(np.float64), "v": hv.astype(np.float64)})
            if c:
                slots = torch.arange(base, base + c, dtype=torch.int32, device="cuda")
                dk, dv = dev(hk, dtype), dev(hv, dtype)
                eng.keep += [slots, dk, dv]
                sb.sb_kv_write(eng.kv, l, c, slots.data_ptr(), dk.data_ptr(), dv.data_ptr(), stream_handle())
        caches.append(cache)
    return eng, caches, bases


@pytest.mark.parametrize("m,dtype", [(TOY, "fp32"), (MINI.with_layers(2), "fp32"), (MINI.with_layers(2), "bf16"),
                                     (TINY_LLAMA, "bf16"), (TINY_LLAMA, "fp32"), (TINY_LLAMA128, "bf16")])
@pytest.mark.parametrize("which", ["figure5", "exercise4", "random"])
def test_layer_step_matches_oracle(m, dtype, which):
    print_case("layer_step", m.name, dtype, which)
    batch = {"figure5": [(1, 3), (1, 1), (2, 0), (3, 0)],
             "exercise4": [(37, 0), (9, 0), (1, 120), (1, 15), (1, 64)],
             "random": random_ragged_batch(3, 8, 700, 80)}[which]
    Wh = make_weights(m, 11, dtype)
    W = DeviceWeights(m, dtype, host=Wh)
    eng, caches, bases = _history_engine(m, dtype, W, batch, 5)
    try:
        T = sum(n for n, _ in batch)
        x_in = normal(7, "x_in", (T, m.H))
        rg = eng.build([n for n, _ in batch], [c for _, c in batch], bases, None)
        outs = []
        eng.forward(rg, layer_outputs=outs, x_in=torch.from_numpy(x_in).cuda(), head=False)
        torch.cuda.synchronize()
        x = x_in.astype(np.float64)
        import copy
        for l in range(m.n_layers):
            got = host(outs[l])
            # oracle layer on the GPU's own input of this layer: isolates one layer's error
            cs = [copy.deepcopy(c[l]) for c in caches]
            want_store = FL.layer_forward_flat(m, Wh["layers"][l], x, batch, cs, store=dtype)
            want = FL.layer_forward_flat(m, Wh["layers"][l], x, batch, [c[l] for c in caches])
            r1 = float(np.max(np.abs(got - want_store)) / np.sqrt(np.mean(want_store ** 2)))
            r2 = assert_close_rms(got, want, TOL[dtype], f"layer {l} vs exact oracle")
            print(f"[parity] layer {l}: {r1:.2e} (storage oracle), {r2:.2e} (exact oracle)", flush=True)
            x = got
    finally:
        eng.close()


def _prefill_then_step(m, dtype, seed, prompts, max_bs):
    """Run the prompts' prefills as iteration 0, then one decode iteration, on the GPU (keeping every layer's
    output).  The oracle then runs each layer of each iteration on the GPU's own input of that layer (the
    embedding for layer 0), so every layer output is checked on its own; iteration 1 feeds the GPU's
    iteration-0 tokens (in bf16 a near-tie may pick either)."""
    Wh = make_weights(m, seed, dtype)
    W = DeviceWeights(m, dtype, host=Wh)
    reqs = [Req(i, 0.0, p, 2, len(p) + 2) for i, p in enumerate(prompts)]
    T0 = sum(len(p) for p in prompts)
    eng = Engine(m, dtype, W, n_slots=sum(r.max_tokens for r in reqs), max_bs=max_bs, max_tokens=max(T0, max_bs),
                 max_keys_total=sum(r.max_tokens for r in reqs))
    try:
        for r in reqs:
            eng.add(r.rid, r.arrival, r.prompt, r.out_len, r.max_tokens)
        res = [eng.step(keep=True), eng.step(keep=True)]
        assert eng.step() is None
    finally:
        eng.close()
    caches = [M.new_cache(m) for _ in reqs]
    rec = []
    iters = [([list(p) for p in prompts], [(len(p), 0) for p in prompts]),
             ([[int(t)] for t in res[0]["tokens"]], [(1, len(p)) for p in prompts])]
    for it, (ids, batch) in enumerate(iters):
        pos = np.asarray(FL.positions(batch))
        x = np.asarray(Wh["tok_emb"], np.float64)[np.concatenate(ids)]
        if m.arch == "gpt":
            x = x + np.asarray(Wh["pos_emb"], np.float64)[pos]
        outs = []
        for l in range(m.n_layers):
            outs.append(FL.layer_forward_flat(m, Wh["layers"][l], x, batch, [c[l] for c in caches]))
            x = res[it]["layer_outputs"][l].numpy().astype(np.float64)
        lr = FL.last_rows(batch)
        logits = M.linear(M.final_norm(m, Wh, x[lr]), Wh["w_lm"])
        rec.append({"outs": outs, "logits": logits})
    return rec, res


def _compare_iteration(m, dtype, rec_it, res_it, what):
    """Each GPU layer output (and the logits) against the exact oracle on the same layer input: stated bar."""
    for l in range(m.n_layers):
        r = assert_close_rms(res_it["layer_outputs"][l].numpy(), rec_it["outs"][l], TOL[dtype], f"{what} layer {l}")
        print(f"[parity] {what} layer {l}: {r:.2e} vs exact oracle", flush=True)
    assert_close_rms(res_it["logits"].numpy(), rec_it["logits"], TOL[dtype], f"{what} logits")
    want_ids = [M.greedy(r) for r in rec_it["logits"]]
    got_ids = list(res_it["tokens"])
    if dtype == "fp32":
        assert got_ids == want_ids
    else:
        # bf16: an id may differ only where the oracle's top-2 margin is within the logit tolerance
        tol = TOL[dtype] * float(np.sqrt(np.mean(rec_it["logits"] ** 2)))
        for g, w, lg in zip(got_ids, want_ids, rec_it["logits"]):
            assert g == w or lg[w] - lg[g] <= tol


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_mini_model_64_decodes(dtype):
    """The mini model (4 layers, H 256, vocab 4096) with 64 decodes, history from real prefills."""
    print_case("mini 64 decodes", dtype)
    ctx = [c for _, c in mini_decode_batch(seed=0)]
    prompts = [uniform_int(0, f"mini.prompt{i}", 0, MINI.V - 1, c).tolist() for i, c in enumerate(ctx)]
    rec, res = _prefill_then_step(MINI, dtype, 0, prompts, 64)
    assert list(res[1]["n_new"]) == [1] * 64 and list(res[1]["ctx"]) == ctx
    _compare_iteration(MINI, dtype, rec[0], res[0], "prefill iteration")
    _compare_iteration(MINI, dtype, rec[1], res[1], "decode iteration")


def test_llama8b_shape_layer_stepwise():
    """One Llama-3-8B-shaped layer over the 256-request mixed batch, step by step through the op-level
    entry points; every intermediate of sampled requests is checked against the oracle."""
    m, dtype = LLAMA8B, "bf16"
    batch = llama_mixed_batch(seed=0)
    pre = sorted(range(240, 256), key=lambda i: batch[i][0])
    sample = [0, 57, 239] + [pre[0], pre[-1]]             # the shortest and the longest prompt
    print_case("8b stepwise", sample)
    from selective_batching_amd.runtime import make_dims
    wl = make_layer_weights(m, 3, 0, dtype)
    dims = make_dims(m.with_layers(1), dtype)
    T = sum(n for n, _ in batch)
    n_slots = sum(n + c for n, c in batch) + 64
    arena = sb.sb_kv_arena_slots(n_slots, len(batch))
    nb = sb.sb_kv_arena_bytes(arena, 1, m.nkv, m.d, sb.SB_BF16)
    ka = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    va = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    kv = sb.sb_kv_create(n_slots, arena, 1, m.nkv, m.d, sb.SB_BF16, ka.data_ptr(), va.data_ptr())
    keep, caches = [], {}
    try:
        bases = [sb.sb_kv_reserve(kv, i, n + c) for i, (n, c) in enumerate(batch)]
        for i in sample:
            n, c = batch[i]
            hk, hv = synthetic_kv(3, f"h{i}", c, m.nkv, m.d, kv_std(m), dtype)
            caches[i] = (hk.astype(np.float64), hv.astype(np.float64))
            if c:
                slots = torch.arange(bases[i], bases[i] + c, dtype=torch.int32, device="cuda")
                dk, dv = dev(hk, dtype), dev(hv, dtype)
                keep += [slots, dk, dv]
                sb.sb_kv_write(kv, 0, c, slots.data_ptr(), dk.data_ptr(), dv.data_ptr(), stream_handle())
        mb = sb.sb_ragged_bytes(dims, len(batch), T, n_slots)
        staging = torch.empty(mb, dtype=torch.uint8, pin_memory=True)
        meta = torch.empty(mb, dtype=torch.uint8, device="cuda")
        rg = sb.sb_ragged_build(dims, [n for n, _ in batch], [c for _, c in batch], bases, None, staging.data_ptr(),
                                meta.data_ptr(), mb, stream_handle())
        dw = {k: dev(v, dtype) for k, v in wl.items()}
        x_in = normal(3, "x_in", (T, m.H))
        x = torch.from_numpy(x_in).cuda()
        h = torch.empty((T, m.H), dtype=torch.bfloat16, device="cuda")
        qkv = torch.empty((T, m.qkv_out), dtype=torch.bfloat16, device="cuda")
        o = torch.empty((T, m.nq * m.d), dtype=torch.bfloat16, device="cuda")
        g = torch.empty((T, m.F), dtype=torch.bfloat16, device="cuda")
        pw = torch.empty(max(rg.n_partials, 1) * 16 * (m.d + 2) * 4, dtype=torch.uint8, device="cuda")
        s = stream_handle()
        sync = torch.cuda.synchronize
        sb.sb_op_norm(sb.SB_BF16, 1, T, m.H, x.data_ptr(), None, dw["ln1_g"].data_ptr(), None, m.eps, h.data_ptr(), s)
        sync(); h1 = host(h)
        sb.sb_op_gemm(sb.SB_BF16, sb.SB_EPI_STORE, T, m.qkv_out, m.H, h.data_ptr(), m.H, dw["w_qkv"].data_ptr(), m.H,
                      None, qkv.data_ptr(), m.qkv_out, 0, 0, s)
        sync(); qkv_pre = host(qkv)
        sb.sb_op_rope_append(dims, rg, kv, 0, qkv.data_ptr(), s)
        sync(); qkv_rot = host(qkv)
        # the appended (rotated) k and the v of every new token, read back from the K/V manager
        new_slots = torch.from_numpy(np.concatenate([np.arange(bases[i] + c, bases[i] + c + n)
                                                     for i, (n, c) in enumerate(batch)]).astype(np.int32)).cuda()
        k_new = torch.empty((T, m.nkv * m.d), dtype=torch.bfloat16, device="cuda")
        v_new = torch.empty((T, m.nkv * m.d), dtype=torch.bfloat16, device="cuda")
        sb.sb_kv_read(kv, 0, T, new_slots.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), s)
        sync(); k_app, v_app = host(k_new), host(v_new)
        sb.sb_op_attention(dims, rg, kv, 0, qkv.data_ptr(), o.data_ptr(), pw.data_ptr(), pw.numel(), s)
        sync(); o1 = host(o)
        sb.sb_op_gemm(sb.SB_BF16, sb.SB_EPI_RESID, T, m.H, m.nq * m.d, o.data_ptr(), m.nq * m.d, dw["w_o"].data_ptr(),
                      m.nq * m.d, None, x.data_ptr(), m.H, 0, 0, s)
        sync(); x1 = host(x)
        sb.sb_op_norm(sb.SB_BF16, 1, T, m.H, x.data_ptr(), None, dw["ln2_g"].data_ptr(), None, m.eps, h.data_ptr(), s)
        sync(); h2 = host(h)
        sb.sb_op_gemm(sb.SB_BF16, sb.SB_EPI_SWIGLU, T, m.F, m.H, h.data_ptr(), m.H, dw["w1"].data_ptr(), m.H, None,
                      g.data_ptr(), m.F, 0, m.F, s)
        sync(); g1 = host(g)
        sb.sb_op_gemm(sb.SB_BF16, sb.SB_EPI_RESID, T, m.H, m.F, g.data_ptr(), m.F, dw["w2"].data_ptr(), m.F, None,
                      x.data_ptr(), m.H, 0, 0, s)
        sync(); x2 = host(x)
        w64 = {k: v.astype(np.float64) for k, v in wl.items()}
        cu = FL.cu_seqlens(batch)
        nq_d, nkv_d = m.nq * m.d, m.nkv * m.d
        from oracle.precision import store as ostore
        for i in sample:
            # each step is fed the GPU's own input of that step; the oracle step is exact, then stored
            n, c = batch[i]
            r = slice(cu[i], cu[i + 1])
            xi = x_in[r].astype(np.float64)
            assert_close_elem(h1[r], M.rms_norm(xi, w64["ln1_g"], m.eps), dtype, f"req {i} norm1")
            assert_close_elem(qkv_pre[r], M.linear(h1[r], w64["w_qkv"]), dtype, f"req {i} qkv")
            pos = c + np.arange(n)
            q = M.rope(qkv_pre[r, :nq_d].reshape(n, m.nq, m.d), pos, m.rope_theta)
            k = M.rope(qkv_pre[r, nq_d:nq_d + nkv_d].reshape(n, m.nkv, m.d), pos, m.rope_theta)
            assert_close_elem(qkv_rot[r, :nq_d], q.reshape(n, nq_d), dtype, f"req {i} rope q")
            assert_close_elem(k_app[r], k.reshape(n, nkv_d), dtype, f"req {i} rope k (appended)")
            assert np.array_equal(v_app[r], qkv_pre[r, nq_d + nkv_d:]), f"req {i} appended v"
            assert np.array_equal(qkv_rot[r, nq_d:], qkv_pre[r, nq_d:]), f"req {i} qkv k/v parts left as they were"
            qg = qkv_rot[r, :nq_d].reshape(n, m.nq, m.d)
            kg = k_app[r].reshape(n, m.nkv, m.d)
            v = qkv_pre[r, nq_d + nkv_d:].reshape(n, m.nkv, m.d)
            K = np.concatenate([caches[i][0], kg]); V = np.concatenate([caches[i][1], v])
            att = M.attention(qg, K, V, c, m.group).reshape(n, nq_d)
            att_abs = M.attention(qg, K, np.abs(V), c, m.group).reshape(n, nq_d)
            assert_close_attention(o1[r], att, att_abs, dtype, f"req {i} (n {n}, ctx {c}) attention")
            ra = float(np.max(np.abs(o1[r] - att)) / np.sqrt(np.mean(att ** 2)))
            assert_close_rms(x1[r], xi + M.linear(o1[r], w64["w_o"]), 1e-5, f"req {i} x after attention")
            assert_close_elem(h2[r], M.rms_norm(x1[r], w64["ln2_g"], m.eps), dtype, f"req {i} norm2")
            gu = M.linear(h2[r], w64["w1"])
            assert_close_elem(g1[r], M.silu(gu[:, :m.F]) * gu[:, m.F:], dtype, f"req {i} swiglu")
            assert_close_rms(x2[r], x1[r] + M.linear(g1[r], w64["w2"]), 1e-5, f"req {i} x out")
            print(f"[parity] 8b step-wise request {i} (n {n}, ctx {c}): attention {ra:.2e}", flush=True)
    finally:
        sb.sb_kv_destroy(kv)


def _gpu_generate(m, dtype, W, reqs, max_bs, n_slots, chunking=None, request_level=False, graphs=False,
                  stats=None):
    eng = Engine(m, dtype, W, n_slots=n_slots, max_bs=max_bs, max_tokens=sum(len(r.prompt) for r in reqs) + max_bs,
                 max_keys_total=sum(r.max_tokens for r in reqs), chunking=chunking, request_level=request_level,
                 graphs=graphs)
    try:
        import math
        pending = sorted(reqs, key=lambda r: (r.arrival, r.rid))
        i, t, log = 0, 0, []
        while True:
            while i < len(pending) and pending[i].arrival <= t:
                r = pending[i]
                eng.add(r.rid, r.arrival, r.prompt, r.out_len, r.max_tokens)
                i += 1
            res = eng.step()
            if res is None:
                if i >= len(pending):
                    break
                t = int(math.ceil(pending[i].arrival))
                continue
            log.append((t, [(int(a), int(b), int(c)) for a, b, c in zip(res["ids"], res["n_new"], res["ctx"])]))
            t += 1
        if stats is not None:
            stats.update(sb.sb_kv_stats(eng.kv))
        return {r.rid: list(eng.output(r.rid)) for r in reqs}, log
    finally:
        eng.close()


@pytest.mark.parametrize("n_slots", [64, 30])
def test_figure5_generation_continuous_equals_one_at_a_time(n_slots):
    """Toy fp32 model: the Figure-5 requests, 8 tokens each, under continuous batching on the GPU.
    Ids must equal the oracle's (continuous and one at a time) and the GPU's own one-at-a-time run, bitwise."""
    m = TOY
    Wh = make_weights(m, 0, "fp32")
    W = DeviceWeights(m, "fp32", host=Wh)
    reqs = figure5_requests(seed=0, vocab=m.V, out_len=8)
    gpu, log = _gpu_generate(m, "fp32", W, reqs, 4, n_slots)
    if n_slots == 64:
        assert [(n, c) for _, n, c in log[1][1]] == [(1, 3), (1, 1), (2, 0), (3, 0)]   # the Figure-5 batch
    want, olog = OG.generate_continuous(m, Wh, reqs, max_bs=4, n_slots=n_slots)
    assert [w for _, w in log] == [w for _, w, _ in olog]
    for r in reqs:
        solo_oracle, margins = OG.generate_one_at_a_time(m, Wh, r.prompt, r.out_len)
        solo_gpu, _ = _gpu_generate(m, "fp32", W, [Req(r.rid, 0.0, r.prompt, r.out_len, r.max_tokens)], 1, 64)
        assert gpu[r.rid] == want[r.rid] == solo_oracle == solo_gpu[r.rid]
        assert min(margins) > 1e-4


def test_generation_llama_timeline_requests():
    """Continuous batching with GQA + RoPE (bf16): the lecture's six-request timeline, max_bs 3."""
    from synth import p4_grid_requests
    m = TINY_LLAMA
    Wh = make_weights(m, 2, "bf16")
    W = DeviceWeights(m, "bf16", host=Wh)
    reqs = p4_grid_requests(seed=0, vocab=m.V)
    gpu, log = _gpu_generate(m, "bf16", W, reqs, 3, 10**4)
    assert len(log) == 10
    for r in reqs:
        solo_gpu, _ = _gpu_generate(m, "bf16", W, [Req(r.rid, 0.0, r.prompt, r.out_len, r.max_tokens)], 1, 10**4)
        assert gpu[r.rid] == solo_gpu[r.rid]          # batch-invariant kernels: identical ids even in bf16


# ---------------------------------------------------------------- full-size shapes, sampled requests
def _sampled_layer_parity(m, dtype, batch, sample, seed, kv_std):
    print_case("sampled layer", m.name, len(batch), sample)
    wl = make_layer_weights(m, seed, 0, dtype)
    W = DeviceWeights(m.with_layers(1), dtype, host={"layers": [wl]}, with_head=False)
    eng = Engine(m.with_layers(1), dtype, W, n_slots=sum(n + c for n, c in batch) + 64, max_bs=len(batch),
                 max_tokens=sum(n for n, _ in batch), max_keys_total=sum(n + c for n, c in batch), zero_arena=True)
    try:
        bases = [sb.sb_kv_reserve(eng.kv, i, n + c) for i, (n, c) in enumerate(batch)]
        caches = {}
        keep = []
        for i in sample:
            n, c = batch[i]
            hk, hv = synthetic_kv(seed, f"h{i}", c, m.nkv, m.d, kv_std, dtype)
            caches[i] = {"k": hk.astype(np.float64), "v": hv.astype(np.float64)}
            if c:
                slots = torch.arange(bases[i], bases[i] + c, dtype=torch.int32, device="cuda")
                dk, dv = dev(hk, dtype), dev(hv, dtype)
                keep += [slots, dk, dv]
                sb.sb_kv_write(eng.kv, 0, c, slots.data_ptr(), dk.data_ptr(), dv.data_ptr(), stream_handle())
        T = sum(n for n, _ in batch)
        x_in = normal(seed, "x_in", (T, m.H))
        rg = eng.build([n for n, _ in batch], [c for _, c in batch], bases, None)
        outs = []
        eng.forward(rg, layer_outputs=outs, x_in=torch.from_numpy(x_in).cuda(), head=False)
        torch.cuda.synchronize()
        cu = FL.cu_seqlens(batch)
        got_all = outs[0]
        wl = {k: v.astype(np.float64) for k, v in wl.items()}      # convert once for the oracle
        import copy
        for i in sample:
            n, c = batch[i]
            got = host(got_all[cu[i]:cu[i + 1]])
            # layer_forward extends the cache it is given: each call takes its own copy
            want = M.layer_forward(m, wl, x_in[cu[i]:cu[i + 1]], c, copy.deepcopy(caches[i]))
            tol_exact = TOL[dtype]
            r2 = assert_close_rms(got, want, tol_exact, f"{m.name} request {i} (n_new {n}, ctx {c}) exact")
            note = ""
            if n <= 64:          # the storage-precision oracle (reported only) for the short ones: host time
                want_store = M.layer_forward(m, wl, x_in[cu[i]:cu[i + 1]], c, copy.deepcopy(caches[i]), store=dtype)
                note = f"{float(np.max(np.abs(got - want_store)) / np.sqrt(np.mean(want_store ** 2))):.2e} (storage oracle), "
            print(f"[parity] {m.name} request {i} (n_new {n}, ctx {c}): {note}"
                  f"{r2:.2e} (exact oracle, bar {tol_exact})", flush=True)
    finally:
        eng.close()


def test_llama8b_shape_layer_sampled():
    """Llama-3-8B-shaped layer over the 256-request mixed batch (240 decodes + 16 prefills); sampled requests."""
    batch = llama_mixed_batch(seed=0)
    dec = [0, 1, 57, 119, 200, 239]
    pre = sorted(range(240, 256), key=lambda i: batch[i][0])
    # the two shortest prompts, a median one and the longest: the row tiles far past the causal diagonal
    _sampled_layer_parity(LLAMA8B, "bf16", batch, dec + pre[:2] + [pre[len(pre) // 2], pre[-1]], 0, kv_std(LLAMA8B))


def test_llama8b_shape_lm_head_sampled():
    """Final RMSNorm + 128256-way LM head + greedy argmax at the 8B shape, 256 rows, sampled rows checked."""
    m = LLAMA8B
    B = 256
    w = {"lnf_g": normal(0, "lnf_g", (m.H,), std=0.1, mean=1.0, dtype="bf16"),
         "w_lm": normal(0, "w_lm", (m.V, m.H), std=init_std(m.H), dtype="bf16"),
         "tok_emb": np.zeros((1, m.H), np.float32), "layers": []}
    W = DeviceWeights(m.with_layers(0), "bf16", host=w)
    eng = Engine(m.with_layers(0), "bf16", W, n_slots=B * 8, max_bs=B, max_tokens=B, max_keys_total=B * 8)
    try:
        bases = [sb.sb_kv_reserve(eng.kv, i, 1) for i in range(B)]
        rg = eng.build([1] * B, [0] * B, bases, None)
        x_in = normal(1, "x_last", (B, m.H))
        ids = eng.forward(rg, x_in=torch.from_numpy(x_in).cuda())
        torch.cuda.synchronize()
        got_ids = ids.cpu().numpy()
        logits = eng.logits[:B * m.V].view(B, m.V)
        for r in (0, 1, 100, 255):
            want = M.lm_logits(m, w, x_in[r])
            got = host(logits[r])
            assert_close_rms(got, want, TOL["bf16"], f"lm row {r}")
            wi = M.greedy(want)
            assert got_ids[r] == wi or want[wi] - want[got_ids[r]] <= 4 * TOL["bf16"] * float(np.sqrt(np.mean(want ** 2)))
    finally:
        eng.close()


@pytest.mark.timeout(600)
def test_gpt175b_shape_layer_sampled():
    """GPT-175B-shaped layer (H 12288, 96 heads, FFN 49152) over 96 decodes + 32 prefills; sampled requests."""
    batch = gpt175b_mixed_batch(seed=0)
    pre = sorted(range(96, 128), key=lambda i: batch[i][0])
    # the shortest, a median and the longest prompt (1012 tokens: 16 row tiles of 128 past the diagonal)
    _sampled_layer_parity(GPT175B_LAYER, "bf16", batch, [0, 50, 95] + [pre[0], pre[len(pre) // 2], pre[-1]], 0,
                          kv_std(GPT175B_LAYER))


def test_pipelined_launches_match_sequential_steps():
    """Two iterations in flight (launch A, launch B, then finish A, finish B) give the same tokens as
    running them one after the other.  The GPU is kept busy first so that both launches are queued
    before A's metadata copy runs: each launch must keep its own staging and id buffers."""
    m = MINI
    W = DeviceWeights(m, "bf16", host=make_weights(m, 3, "bf16"))
    prompts = {"A": {r: uniform_int(11, f"pipe.A{r}", 0, m.V - 1, 5 + 7 * r).tolist() for r in range(6)},
               "B": {r: uniform_int(12, f"pipe.B{r}", 0, m.V - 1, 40 - 5 * r).tolist() for r in range(6)}}
    n_tok = max(sum(len(p) for p in ps.values()) for ps in prompts.values())
    eng = Engine(m, "bf16", W, n_slots=512, max_bs=8, max_tokens=n_tok, max_keys_total=512)

    def pool(name):
        kv = sb.sb_kv_create(512, eng.arena_slots, m.n_layers, m.nkv, m.d, sb.SB_BF16,
                             eng.k_arena.data_ptr(), eng.v_arena.data_ptr())
        sb.sb_kv_set_stream(kv, stream_handle())
        s = sb.sb_sched_create(8, kv)
        for r, p in prompts[name].items():
            sb.sb_sched_add(s, r, float(r), p, 4, len(p) + 4)
        return kv, s

    def drop(kv, s):
        sb.sb_sched_destroy(s)
        sb.sb_kv_destroy(kv)

    try:
        seq = {}
        for name in ("A", "B"):
            kv, s = pool(name)
            seq[name] = eng.finish(eng.launch(sched=s))["tokens"]
            drop(kv, s)
        (kva, sa), (kvb, sbb) = pool("A"), pool("B")
        x = torch.randn(4096, 4096, device="cuda")
        for _ in range(20):
            x = torch.tanh(x @ x)
        pa = eng.launch(sched=sa, buf=0)
        pb = eng.launch(sched=sbb, buf=1)
        ra, rb = eng.finish(pa), eng.finish(pb)
        drop(kva, sa)
        drop(kvb, sbb)
        assert np.array_equal(ra["tokens"], seq["A"]) and np.array_equal(rb["tokens"], seq["B"])
    finally:
        eng.close()


def _gpu_generate_chained(m, dtype, W, reqs, max_bs, n_slots, chunking=None, request_level=False, graphs=False,
                          stats=None):
    """As _gpu_generate, but one iteration ahead of the host (Engine.run_chained): decodes embed the
    previous iteration's ids straight from its device buffer."""
    eng = Engine(m, dtype, W, n_slots=n_slots, max_bs=max_bs, max_tokens=sum(len(r.prompt) for r in reqs) + max_bs,
                 max_keys_total=sum(r.max_tokens for r in reqs), chunking=chunking, request_level=request_level,
                 graphs=graphs)
    try:
        log = []
        eng.run_chained(reqs, on_iteration=lambda res: log.append(
            (res["t"], [(int(a), int(b), int(c)) for a, b, c in zip(res["ids"], res["n_new"], res["ctx"])])))
        if stats is not None:
            stats.update(sb.sb_kv_stats(eng.kv))
        return {r.rid: list(eng.output(r.rid)) for r in reqs}, log
    finally:
        eng.close()


@pytest.mark.parametrize("n_slots", [64, 30])
def test_figure5_generation_chained_equals_oracle(n_slots):
    """Toy fp32 model, Figure-5 requests: the chained loop schedules and generates exactly as the
    oracle's continuous batching (ids bit-exact) and as the GPU's synchronous loop."""
    m = TOY
    Wh = make_weights(m, 0, "fp32")
    W = DeviceWeights(m, "fp32", host=Wh)
    reqs = figure5_requests(seed=0, vocab=m.V, out_len=8)
    got, log = _gpu_generate_chained(m, "fp32", W, reqs, 4, n_slots)
    want, olog = OG.generate_continuous(m, Wh, reqs, max_bs=4, n_slots=n_slots)
    assert log == [(t, w) for t, w, _ in olog]
    sync, slog = _gpu_generate(m, "fp32", W, reqs, 4, n_slots)
    assert slog == log
    for r in reqs:
        assert got[r.rid] == want[r.rid] == sync[r.rid]


def test_generation_chained_bf16_trace_matches_synchronous():
    """GQA + RoPE bf16 model, a Poisson trace with arrivals during generation, gaps and reservations that
    bind: chained and synchronous loops give identical schedules and identical ids (bitwise)."""
    from synth import poisson_trace
    m = TINY_LLAMA
    W = DeviceWeights(m, "bf16", host=make_weights(m, 4, "bf16"))
    reqs = poisson_trace(seed=3, n=40, rate=0.4, vocab=m.V, plo=1, phi=40, olo=1, ohi=24, reserve_out=24,
                         with_prompts=True)
    n_slots = 300
    st = {}
    got, log = _gpu_generate_chained(m, "bf16", W, reqs, 6, n_slots, stats=st)
    sync, slog = _gpu_generate(m, "bf16", W, reqs, 6, n_slots)
    assert log == slog
    assert got == sync
    print(f"[case] K/V compactions: {st['n_compactions']}", flush=True)


# ---------------------------------------------------------------- binding reservations: K/V compaction
# Traces whose reservations bind (the lecture's Pow2 and Oracle policies, few slots), chosen so that the
# K/V manager has to compact live ranges several times in mid-generation: a request admitted then finds no
# hole, and the histories of requests still decoding are moved to lower slots between two iterations.
BINDING = {"pow2": dict(seed=61, max_bs=10, n_slots=260), "oracle": dict(seed=63, max_bs=12, n_slots=300)}


def _binding_trace(policy, vocab):
    from synth import poisson_trace
    from oracle import scheduler as OS
    code = {"pow2": sb.SB_RESERVE_POW2, "oracle": sb.SB_RESERVE_ORACLE}[policy]
    reqs = poisson_trace(seed=BINDING[policy]["seed"], n=100, rate=1.0, vocab=vocab, plo=1, phi=48, olo=1, ohi=24,
                         reserve_out=24, with_prompts=True)
    for r in reqs:
        r.max_tokens = sb.sb_reservation_tokens(code, len(r.prompt), r.out_len, 24)
        assert r.max_tokens == OS.reservation(policy, len(r.prompt), r.out_len, 24)
    return reqs


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_kv_compaction_moves_history_bitwise(dtype):
    """The manager's device copies: four requests fill a 3-layer arena with distinct K/V rows, two are
    freed, and a reservation that fits the counter but no hole compacts the arena.  Every surviving row,
    read back at the request's new base, equals what was written (K rows and the 8-slot V blocks)."""
    nl, nkv, d = 3, 2, 32
    es = 2 if dtype == "bf16" else 4
    n_slots = 96
    arena = n_slots
    nb = sb.sb_kv_arena_bytes(arena, nl, nkv, d, sb.SB_BF16 if dtype == "bf16" else sb.SB_F32)
    assert nb == arena * nl * nkv * d * es
    ka = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    va = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    kv = sb.sb_kv_create(n_slots, arena, nl, nkv, d, sb.SB_BF16 if dtype == "bf16" else sb.SB_F32,
                         ka.data_ptr(), va.data_ptr())
    sb.sb_kv_set_stream(kv, stream_handle())
    try:
        sizes = {0: 16, 1: 29, 2: 8, 3: 40}          # 16 + 32 + 8 + 40 physical slots = 96
        base = {r: sb.sb_kv_reserve(kv, r, n) for r, n in sizes.items()}
        assert base == {0: 0, 1: 16, 2: 48, 3: 56}
        rows = {}
        keep = []
        for r, n in sizes.items():
            for l in range(nl):
                k = normal(7, f"cmp.k{r}.{l}", (n, nkv, d), dtype=dtype)
                v = normal(7, f"cmp.v{r}.{l}", (n, nkv, d), dtype=dtype)
                rows[r, l] = (k, v)
                slots = torch.arange(base[r], base[r] + n, dtype=torch.int32, device="cuda")
                dk, dv = dev(k, dtype), dev(v, dtype)
                keep += [slots, dk, dv]
                sb.sb_kv_write(kv, l, n, slots.data_ptr(), dk.data_ptr(), dv.data_ptr(), stream_handle())
        sb.sb_kv_free(kv, 0)
        sb.sb_kv_free(kv, 2)                          # holes of 16 and 8 slots; 69 reserved
        sb.sb_kv_reserve(kv, 4, 24)                   # 69 + 24 <= 96, but no hole holds 24
        st = sb.sb_kv_stats(kv)
        assert st["n_compactions"] == 1
        moved = {r: sb.sb_kv_lookup(kv, r)[0] for r in (1, 3)}
        assert moved == {1: 0, 3: 32} and sb.sb_kv_lookup(kv, 4)[0] == 72
        for r in (1, 3):
            n = sizes[r]
            slots = torch.arange(moved[r], moved[r] + n, dtype=torch.int32, device="cuda")
            for l in range(nl):
                gk = torch.empty((n, nkv * d), dtype=TDT[dtype], device="cuda")
                gv = torch.empty((n, nkv * d), dtype=TDT[dtype], device="cuda")
                sb.sb_kv_read(kv, l, n, slots.data_ptr(), gk.data_ptr(), gv.data_ptr(), stream_handle())
                torch.cuda.synchronize()
                k, v = rows[r, l]
                assert np.array_equal(host(gk), k.reshape(n, nkv * d)), f"request {r} layer {l}: K rows"
                assert np.array_equal(host(gv), v.reshape(n, nkv * d)), f"request {r} layer {l}: V rows"
    finally:
        sb.sb_kv_destroy(kv)


@pytest.mark.parametrize("policy", ["pow2", "oracle"])
def test_generation_binding_reservations_matches_oracle(policy):
    """Toy fp32 model on a 100-request Poisson trace under the Pow2 / Oracle reservation policy with few
    slots: compaction moves live K/V several times during generation.  Synchronous and chained loops
    schedule exactly as the oracle's replay and generate the oracle's ids, bit-exact."""
    from oracle import scheduler as OS
    m = TOY
    Wh = make_weights(m, 0, "fp32")
    W = DeviceWeights(m, "fp32", host=Wh)
    reqs = _binding_trace(policy, m.V)
    cfg = BINDING[policy]
    print_case("binding reservations", policy, cfg)
    want, olog = OG.generate_continuous(m, Wh, reqs, max_bs=cfg["max_bs"], n_slots=cfg["n_slots"])
    assert [w for _, w, _ in olog] == [w for _, w, _ in OS.replay(reqs, cfg["max_bs"], cfg["n_slots"])]
    for gen in (_gpu_generate, _gpu_generate_chained):
        st = {}
        got, log = gen(m, "fp32", W, reqs, cfg["max_bs"], cfg["n_slots"], stats=st)
        print(f"[case] {gen.__name__}: {len(log)} iterations, {st['n_compactions']} compactions", flush=True)
        assert st["n_compactions"] >= 3
        assert log == [(t, w) for t, w, _ in olog]
        bad = [r.rid for r in reqs if got[r.rid] != want[r.rid]]
        assert not bad, f"requests {bad[:5]}: gpu {got[bad[0]]} oracle {want[bad[0]]}"


@pytest.mark.parametrize("policy", ["pow2", "oracle"])
def test_generation_binding_reservations_bf16_chained_equals_synchronous(policy):
    """GQA + RoPE bf16 model on the same binding traces: chained and synchronous generation compact the
    K/V arena several times and still give identical schedules and identical ids (bitwise)."""
    m = TINY_LLAMA
    W = DeviceWeights(m, "bf16", host=make_weights(m, 4, "bf16"))
    reqs = _binding_trace(policy, m.V)
    cfg = BINDING[policy]
    print_case("binding reservations bf16", policy, cfg)
    s1, s2 = {}, {}
    got, log = _gpu_generate_chained(m, "bf16", W, reqs, cfg["max_bs"], cfg["n_slots"], stats=s1)
    sync, slog = _gpu_generate(m, "bf16", W, reqs, cfg["max_bs"], cfg["n_slots"], stats=s2)
    assert s1["n_compactions"] >= 3 and s2["n_compactions"] == s1["n_compactions"]
    assert log == slog
    assert got == sync


def test_llama8b_trace_requests_equal_solo_generation():
    """The 8B-shaped model (32 layers, GQA 32/8, SwiGLU 14336, vocab 128256; random init, bf16) on a Poisson
    trace with the serving trace's prompt lengths (U[32,512]) and short outputs, chained: iterations mix
    prefills over hundreds of rows (the FFN1 GEMM on the big tiles, the norms of more than 1024 rows
    streamed by waves) with decodes.  Requests generated again alone afterwards -- a prompt, then single
    rows: the small-problem tiles and a workgroup per norm row -- give bitwise the same ids."""
    from synth import poisson_trace
    m = LLAMA8B
    W = DeviceWeights(m, "bf16", host=None, seed=0)
    reqs = poisson_trace(seed=12, n=24, rate=2.5, vocab=m.V, plo=32, phi=512, olo=2, ohi=10, reserve_out=10,
                         with_prompts=True)
    print_case("8b trace vs solo", len(reqs))
    n_slots = sum(r.max_tokens for r in reqs) + 8 * len(reqs)
    got, log = _gpu_generate_chained(m, "bf16", W, reqs, 16, n_slots)
    rows = [sum(n for _, n, _ in w) for _, w in log]
    assert max(rows) > 1024                          # some iterations took the large-batch kernels
    assert all(len(got[r.rid]) == r.out_len and all(0 <= t < m.V for t in got[r.rid]) for r in reqs)
    for r in (reqs[0], reqs[len(reqs) // 2], reqs[-1]):
        alone = Req(r.rid, 0.0, r.prompt, r.out_len, r.max_tokens)
        solo, _ = _gpu_generate_chained(m, "bf16", W, [alone], 1, n_slots)
        assert solo[r.rid] == got[r.rid], f"request {r.rid}: trace {got[r.rid]} alone {solo[r.rid]}"


@pytest.mark.parametrize("chunking", [(4, 2), (6, 3)])
def test_chunked_prefill_generation_matches_oracle(chunking):
    """Toy fp32 model, Figure-5 requests with prompts fed in chunks under a token budget: the GPU's
    schedule and ids equal the oracle's chunked continuous batching (ids bit-exact), equal one-at-a-time
    generation, and the chained loop gives the same."""
    m = TOY
    Wh = make_weights(m, 0, "fp32")
    W = DeviceWeights(m, "fp32", host=Wh)
    reqs = figure5_requests(seed=0, vocab=m.V, out_len=8)
    gpu, log = _gpu_generate(m, "fp32", W, reqs, 4, 64, chunking)
    want, olog = OG.generate_continuous(m, Wh, reqs, max_bs=4, n_slots=64, budget=chunking[0], chunk=chunking[1])
    assert log == [(t, w) for t, w, _ in olog]
    plen = {r.rid: len(r.prompt) for r in reqs}
    assert any(0 < c < plen[rid] for _, w in log for rid, n, c in w)   # a prompt chunk on top of cached tokens
    chained, clog = _gpu_generate_chained(m, "fp32", W, reqs, 4, 64, chunking)
    assert clog == log
    for r in reqs:
        solo, margins = OG.generate_one_at_a_time(m, Wh, r.prompt, r.out_len)
        assert gpu[r.rid] == want[r.rid] == chained[r.rid] == solo
        assert min(margins) > 1e-4


def test_chunked_prefill_bf16_trace_chained_matches_synchronous():
    """GQA + RoPE bf16, a trace with long prompts split over several iterations: chained == synchronous."""
    from synth import poisson_trace
    m = TINY_LLAMA
    W = DeviceWeights(m, "bf16", host=make_weights(m, 5, "bf16"))
    reqs = poisson_trace(seed=8, n=30, rate=0.5, vocab=m.V, plo=20, phi=120, olo=1, ohi=16, reserve_out=16,
                         with_prompts=True)
    got, log = _gpu_generate_chained(m, "bf16", W, reqs, 6, 2000, (48, 32))
    sync, slog = _gpu_generate(m, "bf16", W, reqs, 6, 2000, (48, 32))
    assert log == slog and got == sync
    assert max(sum(n for _, n, _ in w) for _, w in log) <= 48


def test_static_batching_generation_same_tokens():
    """Request-level (static) batching on the same kernels: the lecture's six-request grid (18 iterations)
    and a Poisson trace; the schedule equals the oracle's static replay and the ids equal those of
    iteration-level scheduling (toy fp32: and the oracle's; bf16: bitwise), chained or not."""
    from synth import p4_grid_requests, poisson_trace
    from oracle import scheduler as OS
    m = TOY
    Wh = make_weights(m, 0, "fp32")
    W = DeviceWeights(m, "fp32", host=Wh)
    reqs = p4_grid_requests(seed=0, vocab=m.V)
    got, log = _gpu_generate(m, "fp32", W, reqs, 3, 10**4, request_level=True)
    assert len(log) == 18 and [w for _, w in log] == [w for _, w, _ in OS.replay(reqs, 3, 10**4, static=True)]
    cont, _ = _gpu_generate(m, "fp32", W, reqs, 3, 10**4)
    want, _ = OG.generate_continuous(m, Wh, reqs, max_bs=3, n_slots=10**4)
    assert got == cont == want
    mb = TINY_LLAMA
    Wb = DeviceWeights(mb, "bf16", host=make_weights(mb, 6, "bf16"))
    reqs = poisson_trace(seed=9, n=30, rate=0.6, vocab=mb.V, plo=1, phi=40, olo=1, ohi=20, reserve_out=20,
                         with_prompts=True)
    st, slog = _gpu_generate_chained(mb, "bf16", Wb, reqs, 6, 2000, request_level=True)
    co, _ = _gpu_generate(mb, "bf16", Wb, reqs, 6, 2000)
    assert st == co
    assert [w for _, w in slog] == [w for _, w, _ in OS.replay(reqs, 6, 2000, static=True)]


@pytest.mark.parametrize("chained", [False, True])
def test_figure5_generation_graph_replay_equals_oracle(chained):
    """Toy fp32 model, Figure-5 requests, iterations replayed from HIP graphs once their shape repeats
    (every decode-only iteration after the first): ids bit-exact against the oracle, schedule identical."""
    m = TOY
    Wh = make_weights(m, 0, "fp32")
    W = DeviceWeights(m, "fp32", host=Wh)
    reqs = figure5_requests(seed=0, vocab=m.V, out_len=8)
    gen = _gpu_generate_chained if chained else _gpu_generate
    got, log = gen(m, "fp32", W, reqs, 4, 64, graphs=True)
    want, olog = OG.generate_continuous(m, Wh, reqs, max_bs=4, n_slots=64)
    assert [w for _, w in log] == [w for _, w, _ in olog]
    for r in reqs:
        assert got[r.rid] == want[r.rid]


@pytest.mark.parametrize("chained", [False, True])
def test_decode_loop_graph_replay_matches_eager(chained):
    """bf16 decode loop at a steady batch (16 requests with random K/V history, 12 steps): with graph
    replay every iteration after the second runs from a captured graph, with the host's Select /
    metadata copies / Complete (and, synchronous, a wait) between replays.  Every request's ids must
    equal the eager loop's, bitwise, and the replays must actually have happened."""
    m = MINI.with_layers(2)
    W = DeviceWeights(m, "bf16", host=make_weights(m, 5, "bf16"))
    ctxs = uniform_int(5, "graph.ctx", 16, 200, 16).tolist()
    last = uniform_int(5, "graph.last", 0, m.V - 1, 16).tolist()
    steps = 12
    print_case("graph replay decode loop", chained)

    def run(graphs):
        n_slots = sum(c + steps + 1 for c in ctxs) + 8 * 16
        eng = Engine(m, "bf16", W, n_slots=n_slots, max_bs=16, max_tokens=16, max_keys_total=n_slots,
                     zero_arena=False, graphs=graphs)
        try:
            gen = torch.Generator(device="cuda")
            gen.manual_seed(9)
            for a in (eng.k_arena, eng.v_arena):
                a.view(torch.bfloat16).normal_(0.0, 1.0, generator=gen)
            for i, c in enumerate(ctxs):
                eng.add_running(i, float(i), c, steps + 1, c + steps + 1, 1, last[i])
            if chained:
                n = eng.run_chained()
            else:
                n = 0
                while eng.step() is not None:
                    n += 1
            assert n == steps
            return [list(eng.output(i)) for i in range(16)], len(eng._graph_cache)
        finally:
            eng.close()

    eager, n0 = run(False)
    replayed, n1 = run(True)
    assert n0 == 0 and n1 >= 1
    assert replayed == eager
