"""GPU parity of whole layers, the model step and generation against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import selective_batching_amd as sb
from gpu_util import TOL, assert_close_rms, dev, host, print_case
from oracle import flat as FL
from oracle import generate as OG
from oracle import model as M
from synth import (LLAMA8B, MINI, TOY, GPT175B_LAYER, ModelDims, figure5_requests, gpt175b_mixed_batch,
                   llama_mixed_batch, make_layer_weights, make_weights, mini_decode_batch, normal, random_ragged_batch,
                   synthetic_kv, uniform_int)
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
    for i, (n, c) in enumerate(batch):
        base = sb.sb_kv_reserve(eng.kv, 1000 + i, n + c)
        bases.append(base)
        cache = []
        for l in range(len(W.layers)):
            hk, hv = synthetic_kv(seed, f"L{l}.h{i}", c, m.nkv, m.d, 1.0, dtype)
            cache.append({"k": hk.astype(np.float64), "v": hv.astype(np.float64)})
            if c:
                slots = torch.arange(base, base + c, dtype=torch.int32, device="cuda")
                sb.sb_kv_write(eng.kv, l, c, slots.data_ptr(), dev(hk, dtype).data_ptr(), dev(hv, dtype).data_ptr(),
                               stream_handle())
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
        for l in range(m.n_layers):
            got = host(outs[l])
            # oracle layer on the GPU's own input of this layer: isolates one layer's error
            want = FL.layer_forward_flat(m, Wh["layers"][l], x, batch, [c[l] for c in caches])
            assert_close_rms(got, want, TOL[dtype], f"layer {l}")
            x = got
    finally:
        eng.close()


def _prefill_then_step(m, dtype, seed, prompts, max_bs):
    """Run the prompts' prefills as iteration 0, then one decode iteration; GPU and oracle."""
    Wh = make_weights(m, seed, dtype)
    W = DeviceWeights(m, dtype, host=Wh)
    reqs = [Req(i, 0.0, p, 2, len(p) + 2) for i, p in enumerate(prompts)]
    T0 = sum(len(p) for p in prompts)
    eng = Engine(m, dtype, W, n_slots=sum(r.max_tokens for r in reqs), max_bs=max_bs, max_tokens=max(T0, max_bs),
                 max_keys_total=sum(r.max_tokens for r in reqs))
    rec = []
    toks, _ = OG.generate_continuous(m, Wh, reqs, max_bs=max_bs, n_slots=10**9, record=rec)
    try:
        for r in reqs:
            eng.add(r.rid, r.arrival, r.prompt, r.out_len, r.max_tokens)
        res = [eng.step(keep=True), eng.step(keep=True)]
        assert eng.step() is None
    finally:
        eng.close()
    return rec, res, toks


def _compare_iteration(m, dtype, rec_it, res_it, what):
    for l in range(m.n_layers):
        assert_close_rms(res_it["layer_outputs"][l].numpy(), rec_it["outs"][l], TOL[dtype] * (l + 1), f"{what} layer {l}")
    assert_close_rms(res_it["logits"].numpy(), rec_it["logits"], TOL[dtype] * (m.n_layers + 1), f"{what} logits")
    want_ids = [M.greedy(r) for r in rec_it["logits"]]
    got_ids = list(res_it["tokens"])
    if dtype == "fp32":
        assert got_ids == want_ids
    else:
        # bf16: an id may differ only where the oracle's top-2 margin is within the logit tolerance
        tol = 4 * TOL[dtype] * float(np.sqrt(np.mean(rec_it["logits"] ** 2)))
        for g, w, lg in zip(got_ids, want_ids, rec_it["logits"]):
            assert g == w or lg[w] - lg[g] <= tol


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_mini_model_64_decodes(dtype):
    """The mini model (4 layers, H 256, vocab 4096) with 64 decodes, history from real prefills."""
    print_case("mini 64 decodes", dtype)
    ctx = [c for _, c in mini_decode_batch(seed=0)]
    prompts = [uniform_int(0, f"mini.prompt{i}", 0, MINI.V - 1, c).tolist() for i, c in enumerate(ctx)]
    rec, res, _ = _prefill_then_step(MINI, dtype, 0, prompts, 64)
    assert list(res[1]["n_new"]) == [1] * 64 and list(res[1]["ctx"]) == ctx
    _compare_iteration(MINI, dtype, rec[0], res[0], "prefill iteration")
    _compare_iteration(MINI, dtype, rec[1], res[1], "decode iteration")


def _gpu_generate(m, dtype, W, reqs, max_bs, n_slots):
    eng = Engine(m, dtype, W, n_slots=n_slots, max_bs=max_bs, max_tokens=sum(len(r.prompt) for r in reqs) + max_bs,
                 max_keys_total=sum(r.max_tokens for r in reqs))
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
        for i in sample:
            n, c = batch[i]
            hk, hv = synthetic_kv(seed, f"h{i}", c, m.nkv, m.d, kv_std, dtype)
            caches[i] = {"k": hk.astype(np.float64), "v": hv.astype(np.float64)}
            if c:
                slots = torch.arange(bases[i], bases[i] + c, dtype=torch.int32, device="cuda")
                sb.sb_kv_write(eng.kv, 0, c, slots.data_ptr(), dev(hk, dtype).data_ptr(), dev(hv, dtype).data_ptr(),
                               stream_handle())
        T = sum(n for n, _ in batch)
        x_in = normal(seed, "x_in", (T, m.H))
        rg = eng.build([n for n, _ in batch], [c for _, c in batch], bases, None)
        outs = []
        eng.forward(rg, layer_outputs=outs, x_in=torch.from_numpy(x_in).cuda(), head=False)
        torch.cuda.synchronize()
        cu = FL.cu_seqlens(batch)
        got_all = outs[0]
        wl = {k: v.astype(np.float64) for k, v in wl.items()}      # convert once for the oracle
        for i in sample:
            n, c = batch[i]
            got = host(got_all[cu[i]:cu[i + 1]])
            want = M.layer_forward(m, wl, x_in[cu[i]:cu[i + 1]], c, caches[i])
            assert_close_rms(got, want, TOL[dtype], f"{m.name} request {i} (n_new {n}, ctx {c})")
    finally:
        eng.close()


def test_llama8b_shape_layer_sampled():
    """Llama-3-8B-shaped layer over the 256-request mixed batch (240 decodes + 16 prefills); sampled requests."""
    batch = llama_mixed_batch(seed=0)
    dec = [0, 1, 57, 119, 200, 239]
    pre = sorted(range(240, 256), key=lambda i: batch[i][0])[:2]
    _sampled_layer_parity(LLAMA8B, "bf16", batch, dec + pre, 0, 0.02 * np.sqrt(LLAMA8B.H))


def test_llama8b_shape_lm_head_sampled():
    """Final RMSNorm + 128256-way LM head + greedy argmax at the 8B shape, 256 rows, sampled rows checked."""
    m = LLAMA8B
    B = 256
    w = {"lnf_g": normal(0, "lnf_g", (m.H,), std=0.1, mean=1.0, dtype="bf16"),
         "w_lm": normal(0, "w_lm", (m.V, m.H), std=0.02, dtype="bf16"),
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
    pre = sorted(range(96, 128), key=lambda i: batch[i][0])[:1]
    _sampled_layer_parity(GPT175B_LAYER, "bf16", batch, [0, 50, 95] + pre, 0, 0.02 * np.sqrt(GPT175B_LAYER.H))
