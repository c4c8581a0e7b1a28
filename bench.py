#!/usr/bin/env python3
"""Throughput of one selective-batched iteration on one MI355X.

Workload: the Llama-3-8B-shaped decoder (32 layers, hidden 4096, 32 query /
8 K/V heads of 128, SwiGLU 14336, vocab 128256, bf16, random init on the
device) over the mixed ragged batch of 240 decodes (cached context uniform in
[128, 2048]) and 16 prefills (prompt uniform in [32, 512]), max_bs 256 --
every request in one iteration.  Inputs are synthetic and seeded; the K/V
history of the decodes is random bf16 already resident in HBM.

A step is one pass of the whole hot path: iteration-level Select over the
request pool (host), the ragged metadata and attention work list (host) and
its copy to the GPU, embedding, 32 selective-batched layers, final norm + LM
head + greedy argmax, the copy of the 256 new token ids back, and Complete
(host).  The scheduler state is rebuilt inside the step so that every step
re-runs the same iteration (same batch, same slots).  Steps are pipelined the
way a serving loop runs them: the host side of step k (new pool, Select,
metadata into the second staging buffer, launches) runs while the GPU still
works on step k-1, which is then waited for and completed.  ``value`` is
processed tokens per second (sum of n_new over the batch / step time).

Also reported: HIP-event timing, on the launch stream during the timed steps,
of the FFN1 GEMM and attention launches (only those two classes are timed
there: every recorded event pair costs time); the roofline of the dominant
kernel (the FFN1 SwiGLU GEMM, MFMA-bound); the attention's HBM bandwidth over
the mixed batch and, launched alone, over its decodes (``decode_attention``,
the launches cycling through four layers of K/V so that none is served from
the caches); a per-class breakdown from three extra steps with every class
timed; one GPT-175B-shaped layer over its 96-decode + 32-prefill batch
(``gpt175b_layer``); the whole 2000-request serving trace on the 8B-shaped
model with its K/V pool at 60% of the free HBM, overall and steady-state
throughput and a per-iteration JSONL log (``trace``); the reservation-policy
replay, iteration- against request-level scheduling and the mini-model decode
loop; and the CPU oracle timed on one layer over the whole batch, per request
and flattened, extrapolated to the iteration.

Other modes (each prints its own JSON line instead): ``--op-gemm M,N,K,EPI``
times one GEMM shape; ``--gpt175b-layer`` times one GPT-175B-shaped layer over
its 96-decode + 32-prefill batch, per kernel class.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=40,
                    help="untimed iterations first (a fresh process on a fresh GPU runs the first few seconds slower)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-loop", action="store_true", help="skip the mini-model generation loop")
    ap.add_argument("--no-trace", action="store_true", help="skip the serving-trace window and the policy replay")
    ap.add_argument("--layers", type=int, default=32, help="decoder layers (the workload has 32)")
    ap.add_argument("--log-dir", default=os.path.join(ROOT, "gpurun_out"),
                    help="directory of the serving trace's per-iteration JSONL log ('' for none)")
    ap.add_argument("--no-gpt175b", action="store_true", help="skip the GPT-175B-shaped layer figures")
    ap.add_argument("--trace-iters", type=int, default=None,
                    help="stop the serving trace after this many iterations (for profiling; default: the whole trace)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB device-to-device copy before the steps (calibrates HBM counters)")
    ap.add_argument("--op-gemm", default=None, metavar="M,N,K,EPI",
                    help="instead of the iteration: time one bf16 GEMM of this shape (EPI: store, gelu, resid or "
                         "swiglu; N counts output columns) over --steps launches, for kernel-level profiling")
    ap.add_argument("--gpt175b-layer", action="store_true",
                    help="instead of the iteration: time one GPT-175B-shaped layer over its 96-decode + 32-prefill "
                         "batch (per kernel class), --steps layer steps after --warmup")
    return ap.parse_args()


def op_gemm(spec, steps, warmup, seed):
    """One token-wise GEMM alone, launched ``steps`` times on synthetic bf16 operands (A ~ N(0, 0.25),
    W ~ N(0, 0.02^2)); the launcher picks the tile as it does inside the iteration."""
    import torch
    from selective_batching_amd import api as A
    from selective_batching_amd.runtime import stream_handle
    import selective_batching_amd as sb
    M, N, K, epi = spec.split(",")
    M, N, K = int(M), int(N), int(K)
    code = {"store": sb.SB_EPI_STORE, "gelu": sb.SB_EPI_GELU, "resid": sb.SB_EPI_RESID, "swiglu": sb.SB_EPI_SWIGLU}[epi]
    rows = 2 * N if epi == "swiglu" else N
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    a = (torch.randn(M, K, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    w = (torch.randn(rows, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    c = torch.zeros(M, N, dtype=torch.float32 if epi == "resid" else torch.bfloat16, device="cuda")

    def run():
        A.sb_op_gemm(sb.SB_BF16, code, M, N, K, a.data_ptr(), K, w.data_ptr(), K, None, c.data_ptr(), N, 0,
                     N if epi == "swiglu" else 0, stream_handle())
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / max(steps, 1)
    print(json.dumps({"op": "gemm_bf16", "M": M, "N": N, "K": K, "epilogue": epi, "launches": steps,
                      "avg_us": round(ms * 1e3, 2), "tflops": round(2.0 * M * rows * K / ms / 1e9, 1),
                      "weight_gbs": round(rows * K * 2 / ms / 1e6, 1)}), flush=True)


def gpt175b_layer(steps, warmup, seed):
    """One GPT-175B-shaped layer (H 12288, 96 heads x 128, FFN 49152 GeLU; random init, bf16) over its ragged
    batch of 96 decodes (ctx U[512,2048]) + 32 prefills (prompt U[128,1024]) with random K/V history:
    the layer step timed with HIP events, then the same steps with every kernel class timed.  Returns the
    figures as a dict."""
    import torch
    import selective_batching_amd as sb
    from selective_batching_amd import api as A
    from selective_batching_amd.runtime import DeviceWeights, Engine, stream_handle
    from synth import GPT175B_LAYER, gpt175b_mixed_batch
    torch.cuda.set_device(0)
    m = GPT175B_LAYER
    batch = gpt175b_mixed_batch(seed=seed)
    T = sum(n for n, _ in batch)
    W = DeviceWeights(m, "bf16", host=None, seed=seed, with_head=False)
    n_slots = sum(n + c for n, c in batch) + 8 * len(batch)
    eng = Engine(m, "bf16", W, n_slots=n_slots, max_bs=len(batch), max_tokens=T, max_keys_total=n_slots,
                 zero_arena=False)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 1)
    for a in (eng.k_arena, eng.v_arena):
        a.view(torch.bfloat16).normal_(0.0, 1.0, generator=g)
    bases = [A.sb_kv_reserve(eng.kv, i, n + c) for i, (n, c) in enumerate(batch)]
    rg = eng.build([n for n, _ in batch], [c for _, c in batch], bases, None)
    xv = eng.x[:T * m.H]
    xv.copy_(torch.randn(T * m.H, device="cuda", generator=g))
    s = stream_handle()

    def run():
        A.sb_layer_step(eng.dims, W.layer_structs[0], rg, eng.kv, 0, xv.data_ptr(), eng.ws.data_ptr(), eng.ws.numel(), s)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    layer_ms = e0.elapsed_time(e1) / steps
    A.sb_timing_reset()
    A.sb_timing_enable(True)
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    A.sb_timing_enable(False)
    cls = {}
    for k, name in enumerate(sb.KERNEL_CLASSES):
        ms, n = A.sb_timing_read(k)
        if n:
            cls[name] = ms / steps
    A.sb_timing_reset()
    eng.close()
    flops = {"gemm_qkv": 2 * T * m.qkv_out * m.H, "gemm_o": 2 * T * m.H * m.nq * m.d, "gemm_ffn1": 2 * T * m.F * m.H,
             "gemm_ffn2": 2 * T * m.H * m.F}
    kv_row = 2 * m.nkv * m.d * 2
    att_bytes = sum((c + n) * kv_row for n, c in batch) + T * m.nq * m.d * 2 * 2
    att_flops = 4 * m.d * m.nq * sum(sum(c + j + 1 for j in range(n)) for n, c in batch)
    gemm_ms = sum(cls[k] for k in flops)
    del eng, W, xv
    torch.cuda.empty_cache()
    return {
        "workload": ("GPT-175B-shaped layer (hidden 12288, 96 heads x 128, FFN 49152 GeLU), random init, bf16; "
                     "96 decodes (ctx U[512,2048]) + 32 prefills (prompt U[128,1024])"),
        "tokens": T, "layer_ms": round(layer_ms, 3), "steps": steps, "warmup": warmup,
        "classes_ms": {k: round(v, 4) for k, v in cls.items()},
        "gemm_tflops": {k: round(v / (cls[k] * 1e-3) / 1e12, 1) for k, v in flops.items()},
        "gemm_all": {"tflops": round(sum(flops.values()) / (gemm_ms * 1e-3) / 1e12, 1),
                     "frac": round(sum(flops.values()) / (gemm_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        "attention": {"gbs": round(att_bytes / (cls["attention"] * 1e-3) / 1e9, 1), "bytes": att_bytes,
                      "tflops": round(att_flops / (cls["attention"] * 1e-3) / 1e12, 1), "flops": att_flops},
        "tokens_per_s": round(T / (layer_ms * 1e-3), 1)}


def algorithmic_work(m, batch, n_layers):
    """FLOPs and bytes the method must do per iteration (no padding; weights read once)."""
    T = sum(n for n, _ in batch)
    B = len(batch)
    qkv, o, f1, f2 = m.qkv_out * m.H, m.H * m.nq * m.d, 2 * m.F * m.H, m.H * m.F
    gemm = {"qkv": 2 * T * qkv, "o": 2 * T * o, "ffn1": 2 * T * f1, "ffn2": 2 * T * f2}
    kv_row = 2 * m.nkv * m.d * 2                      # K and V of one token, one layer, bf16
    dec = [(n, c) for n, c in batch if n == 1]
    pre = [(n, c) for n, c in batch if n > 1]
    attn_bytes_dec = sum((c + 1) * kv_row for _, c in dec)
    attn_bytes = sum((c + n) * kv_row for n, c in batch)                     # every K/V row read once
    attn_bytes += T * (m.nq * m.d * 2) * 2                                   # q in, o out
    attn_flops = 4 * m.d * m.nq * sum(sum(c + j + 1 for j in range(n)) for n, c in batch)
    return {"T": T, "B": B, "gemm_per_layer": gemm, "lm_flops": 2 * B * m.H * m.V,
            "attn_bytes_per_layer": attn_bytes, "attn_decode_bytes_per_layer": attn_bytes_dec,
            "attn_flops_per_layer": attn_flops, "n_dec": len(dec), "n_pre": len(pre),
            "weight_bytes": (qkv + o + f1 + f2) * 2 * n_layers + m.V * m.H * 2}


def kernel_roofline(m, work, brk):
    """Each kernel class of the iteration against its roofline: achieved rate from the per-class event
    timing, its fraction of the peak that bounds it, and of min(peak, arithmetic intensity x HBM
    bandwidth).  Algorithmic work only (each operand moved once, no padding)."""
    T, B, L, H = work["T"], work["B"], m.n_layers, m.H
    tf = MFMA_BF16_PEAK_TFLOPS * 1e12
    bw = HBM_PEAK_GBS * 1e9
    w_rows = {"gemm_qkv": (m.qkv_out, H), "gemm_o": (H, m.nq * m.d), "gemm_ffn1": (2 * m.F, H),
              "gemm_ffn2": (H, m.F)}
    out = {}
    for name, (n, k) in w_rows.items():
        if name not in brk:
            continue
        out_cols = n // 2 if name == "gemm_ffn1" else n
        c_bytes = T * out_cols * (4 * 2 if name in ("gemm_o", "gemm_ffn2") else 2)   # residual: fp32 read + write
        flops = 2.0 * T * n * k * L
        byts = (T * k * 2 + n * k * 2 + c_bytes) * L
        sec = brk[name]["ms_per_step"] * 1e-3
        out[name] = {"bound": "mfma", "tflops": round(flops / sec / 1e12, 1), "frac_of_peak": round(flops / sec / tf, 4),
                     "frac_of_attainable": round(flops / sec / min(tf, flops / byts * bw), 4)}
    if "gemm_lm" in brk:
        flops = float(work["lm_flops"])
        byts = m.V * H * 2 + B * H * 2 + B * m.V * 4
        sec = brk["gemm_lm"]["ms_per_step"] * 1e-3
        att = min(tf, flops / byts * bw)
        out["gemm_lm"] = {"bound": "mfma" if att >= tf else "hbm", "tflops": round(flops / sec / 1e12, 1),
                          "frac_of_peak": round(flops / sec / tf, 4), "frac_of_attainable": round(flops / sec / att, 4)}
    hbm_bytes = {
        "attention": work["attn_bytes_per_layer"] * L,
        "norm": (2 * L * T + B) * H * (4 + 2),                               # fp32 row in, bf16 row out
        "rope_append": L * T * (m.nq + 2 * m.nkv) * m.d * 2 * 2,            # q, k, v read; q, k, v written
        "embed": T * H * (2 + 4),
        "argmax": B * m.V * 4,
    }
    for name, byts in hbm_bytes.items():
        if name not in brk:
            continue
        gbs = byts / (brk[name]["ms_per_step"] * 1e-3) / 1e9
        out[name] = {"bound": "hbm", "gbs": round(gbs, 1), "frac_of_peak": round(gbs * 1e9 / bw, 4)}
    return out


def decode_attention(m, batch, seed, launches=20, layers=4):
    """The attention kernel alone on the iteration's decodes (240 requests, ctx U[128,2048]): algorithmic
    bytes (every cached K/V row once, q in, o out) over the average launch time, HIP events on the launch
    stream.  The launches cycle through ``layers`` layers of random-filled K/V arenas (~1.1 GB each), so
    that, as in the iteration, a launch finds none of its K/V in the caches."""
    import torch
    import selective_batching_amd as sb
    from selective_batching_amd import api as A
    from selective_batching_amd.runtime import make_dims, stream_handle
    dec = [(n, c) for n, c in batch if n == 1]
    one = m.with_layers(layers)
    dims = make_dims(one, "bf16")
    n_slots = sum(n + c for n, c in dec) + 8 * len(dec)
    arena = A.sb_kv_arena_slots(n_slots, len(dec))
    nbytes = A.sb_kv_arena_bytes(arena, layers, m.nkv, m.d, sb.SB_BF16)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 7)
    ka = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_(generator=g)
    va = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_(generator=g)
    kv = A.sb_kv_create(n_slots, arena, layers, m.nkv, m.d, sb.SB_BF16, ka.data_ptr(), va.data_ptr())
    try:
        bases = [A.sb_kv_reserve(kv, i, n + c) for i, (n, c) in enumerate(dec)]
        T = len(dec)
        mb = A.sb_ragged_bytes(dims, len(dec), T, n_slots)
        staging = torch.empty(mb, dtype=torch.uint8, pin_memory=True)
        meta = torch.empty(mb, dtype=torch.uint8, device="cuda")
        s = stream_handle()
        rg = A.sb_ragged_build(dims, [n for n, _ in dec], [c for _, c in dec], bases, None, staging.data_ptr(),
                               meta.data_ptr(), mb, s)
        qkv = (torch.randn(T, m.qkv_out, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
        o = torch.empty(T, m.nq * m.d, dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(rg.n_partials, 1) * 16 * (m.d + 2) * 4, dtype=torch.uint8, device="cuda")

        def run(i):
            A.sb_op_attention(dims, rg, kv, i % layers, qkv.data_ptr(), o.data_ptr(), ws.data_ptr(), ws.numel(), s)
        for i in range(5):
            run(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(launches):
            run(i)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / launches
    finally:
        A.sb_kv_destroy(kv)
    kv_bytes = sum((c + 1) * 2 * m.nkv * m.d * 2 for _, c in dec)
    byts = kv_bytes + T * m.nq * m.d * 2 * 2
    gbs = byts / (ms * 1e-3) / 1e9
    return {"workload": (f"attention alone over the {T} decodes of the batch (ctx U[128,2048], bf16), launches "
                         f"cycling through {layers} layers of K/V"),
            "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "avg_launch_ms": round(ms, 4), "bytes_per_launch": byts,
            "launches": launches}


def cpu_baseline(m, batch, seed, lm_sample=8):
    """The oracle (fp64 numpy, as it stands) on one decoder layer over the whole batch -- the 240 decodes
    with their synthetic K/V history and the 16 prompts, 3741 rows at seed 0 -- timed two ways: per request
    (the plain definition: each request's rows through the layer on their own) and flattened (the
    oracle's [T, H] self-check: token-wise operators on all rows at once, attention split by request).
    The iteration is then extrapolated: the layer x 32 plus the LM head (final norm, 128256-way product,
    argmax) of each request's last row, timed on ``lm_sample`` rows one at a time (per request) and on all
    rows at once (flattened).  BLAS uses every host thread."""
    import numpy as np
    from oracle import flat as FL
    from oracle import model as OM
    from synth import kv_std, make_layer_weights, normal, synthetic_kv, init_std
    cores = len(os.sched_getaffinity(0))
    wl = {k: np.asarray(v, np.float64) for k, v in make_layer_weights(m, seed, 0, "bf16").items()}
    T = sum(n for n, _ in batch)
    B = len(batch)
    caches = []
    for i, (n, c) in enumerate(batch):
        hk, hv = synthetic_kv(seed, f"cpu{i}", c, m.nkv, m.d, kv_std(m), "bf16")
        caches.append({"k": hk.astype(np.float64), "v": hv.astype(np.float64)})
    x = normal(seed, "cpu.x", (T, m.H)).astype(np.float64)
    cu = np.concatenate([[0], np.cumsum([n for n, _ in batch])])
    t0 = time.perf_counter()
    for i, (n, c) in enumerate(batch):
        OM.layer_forward(m, wl, x[cu[i]:cu[i + 1]], c, dict(caches[i]))
    t_req = time.perf_counter() - t0
    t0 = time.perf_counter()
    FL.layer_forward_flat(m, wl, x, batch, [dict(c) for c in caches])
    t_flat = time.perf_counter() - t0
    del wl, caches
    W = {"lnf_g": np.ones(m.H), "w_lm": normal(seed, "cpu.w_lm", (m.V, m.H), std=init_std(m.H),
                                               dtype="bf16").astype(np.float64)}
    last = x[cu[1:] - 1]
    t0 = time.perf_counter()
    for r in range(lm_sample):
        OM.greedy(OM.lm_logits(m, W, last[r]))
    t_lm_req = (time.perf_counter() - t0) * B / lm_sample
    t0 = time.perf_counter()
    np.argmax(OM.linear(OM.final_norm(m, W, last), W["w_lm"]), axis=1)
    t_lm_flat = time.perf_counter() - t0
    est_req = t_req * m.n_layers + t_lm_req
    est_flat = t_flat * m.n_layers + t_lm_flat
    return {"value": round(T / est_req, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"one decoder layer over the whole batch ({B} requests, {T} rows), per request: "
                       f"{t_req:.2f} s; x {m.n_layers} layers + the LM head of each request's last row "
                       f"({lm_sample} rows timed, x {B // lm_sample}: {t_lm_req:.2f} s) = {est_req:.1f} s per iteration, "
                       f"extrapolated; fp64 numpy, BLAS threads = {cores}"),
            "flattened": {"value": round(T / est_flat, 3), "unit": "tokens/s",
                          "layer_s": round(t_flat, 3), "lm_head_s": round(t_lm_flat, 3),
                          "iteration_s_extrapolated": round(est_flat, 2)},
            "per_request_layer_s": round(t_req, 3), "iteration_s_extrapolated": round(est_req, 2),
            "batched_speedup": round(est_req / est_flat, 2)}


def cpu_mini(seed):
    """The oracle on one decode iteration of the mini model (the pages' own CPU measurement: 64 decode
    requests on a small GPT, one at a time vs batched): every request through the plain per-request
    definition, then the same iteration through the flattened [T, H] self-check.  fp64 numpy, with
    all host threads and on one thread; best of three each."""
    import copy
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import flat as FL
    from oracle import model as OM
    from synth import MINI, kv_std, make_weights, mini_decode_batch, synthetic_kv, uniform_int
    m = MINI
    W = make_weights(m, seed, "bf16")
    batch = mini_decode_batch(seed=seed)
    ids = uniform_int(seed, "cpu_mini.ids", 0, m.V - 1, len(batch)).tolist()
    caches = []
    for i, (_, c) in enumerate(batch):
        per_layer = []
        for l in range(m.n_layers):
            k, v = synthetic_kv(seed, f"cpu_mini.{i}.{l}", c, m.nkv, m.d, kv_std(m), "bf16")
            per_layer.append({"k": k.astype(np.float64), "v": v.astype(np.float64)})
        caches.append(per_layer)

    def per_request():
        cs = copy.deepcopy(caches)
        return [OM.forward_request(m, W, [ids[i]], c, cs[i])[1] for i, (_, c) in enumerate(batch)]

    def flattened():
        cs = copy.deepcopy(caches)
        return FL.forward_flat(m, W, [[t] for t in ids], batch, cs)[1]

    def best(fn):
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return round(1e3 * min(ts), 2)
    cores = len(os.sched_getaffinity(0))
    out = {"workload": f"one decode iteration of the mini GPT (4 layers, hidden 256, vocab 4096), {len(batch)} "
                       "requests with cached context U[16,256]; fp64 numpy oracle",
           "cores": cores}
    out["per_request_ms"], out["flattened_ms"] = best(per_request), best(flattened)
    with threadpool_limits(1):
        out["per_request_ms_1_core"], out["flattened_ms_1_core"] = best(per_request), best(flattened)
    out["batched_speedup"] = round(out["per_request_ms"] / out["flattened_ms"], 2)
    return out


def decode_loop(seed, steps=64, reps=3, dtype="bf16"):
    """Generation loop on the mini model (4 layers, hidden 256, 8 heads, FFN 1024, vocab 4096, ``dtype``):
    64 requests in decode with cached context U[16, 256] (random K/V history), each generating ``steps``
    more tokens.  Timed three ways: the synchronous loop (each iteration waits for its ids before the
    next Select), the chained one (iteration t+1 selected and launched before t's ids reach the host),
    and the chained one with each iteration's device side replayed from a HIP graph (one launch per
    iteration instead of one per kernel).  Best of ``reps`` runs of each."""
    import torch
    from selective_batching_amd.runtime import TORCH_DT, DeviceWeights, Engine, make_dims
    from synth import MINI, mini_decode_batch, uniform_int
    m = MINI
    batch = mini_decode_batch(seed=seed)
    B = len(batch)
    W = DeviceWeights(m, dtype, host=None, seed=seed)
    n_slots = sum(c + steps + 1 for _, c in batch) + 8 * B
    eng = Engine(m, dtype, W, n_slots=n_slots, max_bs=B, max_tokens=B, max_keys_total=n_slots, zero_arena=False)
    tdt = TORCH_DT[make_dims(m, dtype).dtype]
    for a in (eng.k_arena, eng.v_arena):
        a.view(tdt).normal_(0.0, 1.0)
    last = uniform_int(seed, "decode.last", 0, m.V - 1, B).tolist()
    rid = [0]

    def fill(n_steps):
        for i, (_, c) in enumerate(batch):
            eng.add_running(rid[0], float(i), c, n_steps + 1, c + n_steps + 1, 1, last[i])
            rid[0] += 1

    def sync(n_steps):
        fill(n_steps)
        k = 0
        while eng.step() is not None:
            k += 1
        return k

    def chained(n_steps):
        fill(n_steps)
        return eng.run_chained()

    out = {}
    for name, fn, graphs in (("synchronous", sync, False), ("chained", chained, False),
                             ("chained_graphs", chained, True)):
        eng.graphs = graphs
        fn(4)                                         # warm-up (with graphs: captures the steady shape)
        best = None
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            n = fn(steps)
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            assert n == steps
            best = dt if best is None else min(best, dt)
        out[name] = {"ms_per_step": round(1e3 * best / steps, 4), "tokens_per_s": round(B * steps / best, 1)}
    eng.close()
    return {"workload": (f"mini GPT (4 layers, hidden 256, 8 heads, FFN 1024, vocab 4096) {dtype}, random init; {B} "
                         f"requests in decode, cached context U[16,256], {steps} generated tokens each"),
            **out, "chained_speedup": round(out["synchronous"]["ms_per_step"] / out["chained"]["ms_per_step"], 3),
            "chained_graphs_speedup": round(out["synchronous"]["ms_per_step"] / out["chained_graphs"]["ms_per_step"], 3)}


def reservation_policies(seed, n_slots=20000):
    """The 8B-shaped serving trace (2000 Poisson arrivals at 0.5 per iteration, prompt U[32,512], output
    U[1,512], max_bs 64) replayed through libsb's scheduler under the three reservation policies with the
    K/V pool binding at ``n_slots``: iterations to drain the trace, mean batch, generated tokens per
    iteration and the time-weighted fractions of slots reserved vs holding K/V.  Host work only."""
    import math
    import numpy as np
    from selective_batching_amd import api as A
    import selective_batching_amd as sb
    from synth import poisson_trace
    reqs = poisson_trace(seed=seed, n=2000, rate=0.5)
    out = {"workload": f"2000-request Poisson trace (rate 0.5/iteration, prompt U[32,512], output U[1,512]), "
                       f"max_bs 64, {n_slots} K/V slots (binding)"}
    for name, code in (("max", sb.SB_RESERVE_MAX), ("pow2", sb.SB_RESERVE_POW2), ("oracle", sb.SB_RESERVE_ORACLE)):
        kv = A.sb_kv_create(n_slots, A.sb_kv_arena_slots(n_slots, 64), 1, 1, 8, sb.SB_BF16)
        s = A.sb_sched_create(64, kv)
        pending = sorted(reqs, key=lambda r: (r.arrival, r.rid))
        i = t = iters = members = gen = 0
        res_sum = st_sum = 0
        while i < len(pending) or A.sb_sched_stats(s)["pool"]:
            while i < len(pending) and pending[i].arrival <= t:
                r = pending[i]
                A.sb_sched_add(s, r.rid, r.arrival, r.prompt, r.out_len,
                               A.sb_reservation_tokens(code, len(r.prompt), r.out_len, 512))
                i += 1
            if not A.sb_sched_stats(s)["pool"]:
                t = int(math.ceil(pending[i].arrival))
                continue
            ids, n_new, ctx, _ = A.sb_select_batch(s, 64)
            rv, sv = A.sb_kv_usage(s)
            res_sum += rv
            st_sum += sv
            iters += 1
            members += len(ids)
            gen += len(ids)
            A.sb_sched_complete(s, ids, np.zeros(len(ids), np.int32))
            t += 1
        A.sb_sched_destroy(s)
        A.sb_kv_destroy(kv)
        out[name] = {"iterations": iters, "mean_batch": round(members / iters, 2),
                     "generated_per_iteration": round(gen / iters, 2),
                     "reserved_frac": round(res_sum / iters / n_slots, 4), "stored_frac": round(st_sum / iters / n_slots, 4)}
    return out


SLOT_BYTES_8B = 2 * 32 * 8 * 128 * 2     # one K/V slot of the 8B-shaped model: K and V, 32 layers, 8 heads x 128, bf16


def trace_slots(frac=0.6):
    """K/V slots of the serving trace by its rule: 60% of the HBM free now, over the bytes one slot takes
    (K and V of one token in every layer)."""
    import torch
    free, _ = torch.cuda.mem_get_info()
    return int(frac * free) // SLOT_BYTES_8B, int(free)


def trace_run(W, m, seed, log_path=None, iters=None):
    """The 8B-shaped serving trace on the GPU, run to the end: 2000 requests, Poisson arrivals at 0.5 per
    iteration, prompt U[32,512], output U[1,512], max_tokens = prompt + 512, max_bs 64, K/V slots 60% of
    the free HBM (1M+ slots: the pool never binds, since at most 64 x 1024 are ever reserved), chained
    (iteration t+1 launched before t's ids reach the host).

    Throughput is reported two ways ("CS349D Lecture 2", section 5.4): overall, over the whole run, and
    steady-state, counting only up to the iteration in which the last request starts producing tokens
    (its prefill): after that only the drain remains, a few long requests in ever smaller batches, whose
    length depends on the longest output rather than on the scheduler.  Processed tokens count every
    row (prompt tokens + decodes), generated tokens one per member.  Each iteration is logged as one JSON
    line: clock t, batch ids, rows T, prefill / decode members, reserved slots after Select, device ms
    (HIP events around its work on the stream) and host ms (Select, metadata and launches)."""
    import torch
    from selective_batching_amd.runtime import Engine
    from synth import poisson_trace
    reqs = poisson_trace(seed=seed, n=2000, rate=0.5, vocab=m.V, with_prompts=True)
    n_slots, free = trace_slots()
    eng = Engine(m, "bf16", W, n_slots=n_slots, max_bs=64, max_tokens=64 * 512, max_keys_total=64 * 1024,
                 zero_arena=False)
    eng.record_events = True
    marks = []
    log = open(log_path, "w") if log_path else None

    def on_it(res):
        # settled: its ids are on the host.  No device-wide wait here -- the next iteration is already
        # queued behind it, and waiting for that one would leave the GPU idle while the host launches
        # the one after.
        n_pre = int((res["ctx"] == 0).sum())
        marks.append((time.perf_counter(), int(res["n_new"].sum()), len(res["ids"]), n_pre))
        if log is not None:
            log.write(json.dumps({"t": res["t"], "ids": [int(i) for i in res["ids"]], "T": int(res["n_new"].sum()),
                                  "n_prefill": n_pre, "n_decode": len(res["ids"]) - n_pre, "n_rsrv": res["n_rsrv"],
                                  "gpu_ms": round(res["gpu_ms"], 4), "host_ms": round(res["host_ms"], 4)}) + "\n")

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = eng.run_chained(reqs, on_iteration=on_it, max_iters=iters)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eng.close()
    del eng
    if log is not None:
        log.close()
    proc = sum(p for _, p, _, _ in marks)
    gen = sum(g for _, _, g, _ in marks)
    last_start = max(k for k, mk in enumerate(marks) if mk[3] > 0)       # the last request's prefill
    st = marks[:last_start + 1]
    st_s = st[-1][0] - t0
    return {"workload": ("8B-shaped decoder on the 2000-request Poisson trace (rate 0.5/iteration, prompt U[32,512], "
                         "output U[1,512], max_tokens = prompt + 512, max_bs 64), run to the end, chained"),
            "n_slots": n_slots, "n_slots_rule": (f"floor(0.6 x {free} free HBM bytes / {SLOT_BYTES_8B} bytes per slot "
                                                 "(K+V, 32 layers, 8 x 128, bf16)); never binding (at most 64 x 1024 "
                                                 "reserved)"),
            "iterations": n, "wall_s": round(wall, 3),
            "overall": {"processed_tokens_per_s": round(proc / wall, 1), "generated_tokens_per_s": round(gen / wall, 1),
                        "mean_batch": round(gen / len(marks), 2), "ms_per_iteration": round(1e3 * wall / len(marks), 3)},
            "steady": {"definition": "up to the iteration in which the last request produces its first token",
                       "iterations": len(st), "processed_tokens_per_s": round(sum(p for _, p, _, _ in st) / st_s, 1),
                       "generated_tokens_per_s": round(sum(g for _, _, g, _ in st) / st_s, 1),
                       "mean_batch": round(sum(g for _, _, g, _ in st) / len(st), 2),
                       "ms_per_iteration": round(1e3 * st_s / len(st), 3)},
            "iteration_log": os.path.relpath(log_path, ROOT) if log_path else None}


def scheduling_compare(W, m, seed, n=96):
    """The first ``n`` requests of the 8B-shaped serving trace (Poisson arrivals at 0.5 per iteration,
    prompt U[32,512], output U[1,512], max_bs 64) run to completion on the same kernels under
    iteration-level scheduling (Algorithm 1) and under request-level (static) batching, both chained.
    Reports iterations, wall time, generated tokens per second and the mean time to first token and to
    completion on the iteration clock."""
    import torch
    from selective_batching_amd.runtime import Engine
    from synth import poisson_trace
    reqs = poisson_trace(seed=seed, n=n, rate=0.5, vocab=m.V, with_prompts=True)
    arrive = {r.rid: r.arrival for r in reqs}
    out = {"workload": (f"first {n} requests of the 8B-shaped serving trace (Poisson 0.5/iteration, prompt "
                        "U[32,512], output U[1,512]), max_bs 64, run to completion on the same kernels")}
    for name, static in (("iteration_level", False), ("request_level", True)):
        n_slots = 64 * 1024 + 64 * 8
        eng = Engine(m, "bf16", W, n_slots=n_slots, max_bs=64, max_tokens=64 * 512, max_keys_total=n_slots,
                     zero_arena=False, request_level=static)
        first, last = {}, {}

        def on_it(res):
            for rid in res["ids"]:
                first.setdefault(int(rid), res["t"])
                last[int(rid)] = res["t"]

        torch.cuda.synchronize()
        t0 = time.perf_counter()
        iters = eng.run_chained(reqs, on_iteration=on_it)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        eng.close()
        gen = sum(r.out_len for r in reqs)
        out[name] = {"iterations": iters, "wall_s": round(wall, 3), "generated_tokens_per_s": round(gen / wall, 1),
                     "mean_ttft_iterations": round(sum(first[k] - arrive[k] + 1 for k in first) / n, 2),
                     "mean_latency_iterations": round(sum(last[k] - arrive[k] + 1 for k in last) / n, 2)}
    out["throughput_ratio"] = round(out["iteration_level"]["generated_tokens_per_s"] /
                                    out["request_level"]["generated_tokens_per_s"], 3)
    return out


def ffn1_traffic():
    """HBM bytes per FFN1 GEMM launch (FETCH_SIZE + WRITE_SIZE counter runs, scaled by a 1 GiB copy) as
    recorded in profiles/ffn1_gemm_traffic.json, or None when the GEMM sources changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "ffn1_gemm_traffic.json")
    try:
        rec = json.load(open(path))
        for src, digest in rec["sources_sha256"].items():
            if hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest() != digest:
                return None
        return rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (requests would shard by data "
              "parallelism with no exchange between GPUs).", file=sys.stderr)
        sys.exit(2)

    if args.op_gemm:
        op_gemm(args.op_gemm, args.steps, args.warmup, args.seed)
        return
    if args.gpt175b_layer:
        print(json.dumps(gpt175b_layer(args.steps, args.warmup, args.seed)), flush=True)
        return

    import numpy as np
    import torch

    import selective_batching_amd as sb
    from selective_batching_amd import api as A
    from selective_batching_amd.runtime import DeviceWeights, Engine, stream_handle
    from synth import LLAMA8B, llama_mixed_batch, uniform_int

    m = LLAMA8B.with_layers(args.layers)
    batch = llama_mixed_batch(seed=args.seed)
    work = algorithmic_work(m, batch, m.n_layers)
    T, B = work["T"], work["B"]
    torch.cuda.set_device(0)
    print(f"[bench] {torch.cuda.get_device_name(0)}; T={T} tokens, B={B} requests, {m.n_layers} layers", file=sys.stderr,
          flush=True)

    W = DeviceWeights(m, "bf16", host=None, seed=args.seed)
    n_slots = sum(n + c for n, c in batch) + 8 * B
    eng = Engine(m, "bf16", W, n_slots=n_slots, max_bs=B, max_tokens=T, max_keys_total=n_slots, zero_arena=False)
    # random bf16 K/V history already in HBM (both arenas, every slot)
    g = torch.Generator(device="cuda")
    g.manual_seed(args.seed + 1)
    for a in (eng.k_arena, eng.v_arena):
        a.view(torch.bfloat16).normal_(0.0, 1.0, generator=g)
    prompts = {i: uniform_int(args.seed, f"bench.prompt{i}", 0, m.V - 1, n).tolist()
               for i, (n, c) in enumerate(batch) if n > 1}
    last_tok = uniform_int(args.seed, "bench.last", 0, m.V - 1, B).tolist()

    def new_pool():
        """A fresh K/V manager + scheduler over the shared arenas, holding the pool of this
        iteration: decodes first (they arrived first), then the new prompts."""
        kv = A.sb_kv_create(n_slots, eng.arena_slots, m.n_layers, m.nkv, m.d, sb.SB_BF16,
                            eng.k_arena.data_ptr(), eng.v_arena.data_ptr())
        A.sb_kv_set_stream(kv, stream_handle())
        sched = A.sb_sched_create(B, kv)
        for i, (n, c) in enumerate(batch):
            if n == 1:
                # mid-generation: prompt of c tokens, 1 generated token not fed yet -> ctx = c;
                # max_tokens = ctx + n_new (the reservation this iteration needs)
                A.sb_sched_add_running(sched, i, float(i), c, 2, c + 1, 1, last_tok[i])
            else:
                A.sb_sched_add(sched, i, float(i), prompts[i], 2, n + 1)
        return kv, sched

    pools = [None, None]

    def launch(k):
        """Host side of step k (fresh pool, Select, metadata) and enqueue of its GPU work."""
        b = k % 2
        if pools[b] is not None:                 # step k-2 used this pool and has finished
            A.sb_sched_destroy(pools[b][1])
            A.sb_kv_destroy(pools[b][0])
        pools[b] = new_pool()
        p = eng.launch(sched=pools[b][1], buf=b)
        assert p is not None and len(p["ids"]) == B and int(p["n_new"].sum()) == T
        return p

    def run(n):
        """n steps, pipelined: the host side of step k runs while the GPU works on step k-1;
        step k-1 is then waited for and completed."""
        prev = None
        for k in range(n):
            p = launch(k)
            if prev is not None:
                eng.finish(prev)
            prev = p
        if prev is not None:
            eng.finish(prev)

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    run(args.warmup)
    torch.cuda.synchronize()
    # timed steps: events only around the two kernels the roofline and bandwidth figures need
    A.sb_timing_reset()
    A.sb_timing_enable(True, classes=[sb.KERNEL_CLASSES.index("gemm_ffn1"), sb.KERNEL_CLASSES.index("attention")])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    A.sb_timing_enable(False)

    def read_classes(steps):
        kern = {}
        for k, name in enumerate(sb.KERNEL_CLASSES):
            ms, n = A.sb_timing_read(k)
            if n:
                kern[name] = {"ms_per_step": ms / steps, "launches_per_step": n / steps, "avg_ms": ms / n}
        A.sb_timing_reset()
        return kern

    kern = read_classes(args.steps)
    # per-class breakdown: a few more steps with every class timed (not part of the timed region)
    n_brk = 3
    A.sb_timing_enable(True)
    run(n_brk)
    torch.cuda.synchronize()
    A.sb_timing_enable(False)
    brk = read_classes(n_brk)
    ms_step = 1000.0 * wall / args.steps
    gpu_ms = sum(v["ms_per_step"] for v in brk.values())

    # roofline of the dominant kernel: the FFN1 (SwiGLU) GEMM, one launch per layer
    f1 = kern["gemm_ffn1"]
    f1_flops = work["gemm_per_layer"]["ffn1"]
    f1_tflops = f1_flops / (f1["avg_ms"] * 1e-3) / 1e12
    kern_name = ("gemm_bf16_dma_kernel<224,384,2,4,64,2,2,true,SWIGLU> (FFN1 gate/up GEMM + SiLU*up epilogue, "
                 "224x384x64 tiles: 1275 tiles, 5 full rounds at T = 3741; copies spread over the MFMAs)")
    roofline = {"kernel": kern_name, "bound": "mfma",
                "achieved": round(f1_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(f1_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": ffn1_traffic(),
                "flops_per_launch": f1_flops, "avg_launch_ms": round(f1["avg_ms"], 4)}
    at = kern["attention"]
    attn_gbs = work["attn_bytes_per_layer"] / (at["avg_ms"] * 1e-3) / 1e9
    gemm_flops = sum(work["gemm_per_layer"].values()) * m.n_layers + work["lm_flops"]
    gemm_ms = sum(brk[k]["ms_per_step"] for k in ("gemm_qkv", "gemm_o", "gemm_ffn1", "gemm_ffn2", "gemm_lm"))
    out = {
        "metric": "tokens/s per selective-batched iteration; MFMA % + attention HBM GB/s",
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"Llama-3-8B-shaped decoder ({m.n_layers} layers, hidden 4096, GQA 32/8 x 128, "
                                "SwiGLU 14336, vocab 128256), random init; one iteration over 240 decodes "
                                "(ctx U[128,2048]) + 16 prefills (prompt U[32,512])"),
                   "tokens_per_iteration": T, "requests": B, "decodes": work["n_dec"], "prefills": work["n_pre"],
                   "max_bs": B, "seed": args.seed},
        "roofline": roofline,
        "generated_tokens_per_s": round(B / (ms_step * 1e-3), 1),
        "gpu_kernel_ms_per_step": round(gpu_ms, 3),
        "gemm_mfma": {"tflops": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 1),
                      "frac": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        "attention": {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "avg_launch_ms": round(at["avg_ms"], 4),
                      "bytes_per_launch": work["attn_bytes_per_layer"],
                      "decode_kv_bytes_per_launch": work["attn_decode_bytes_per_layer"]},
        "kernels_ms_per_step": {k: round(v["ms_per_step"], 3) for k, v in brk.items()},
        "kernel_roofline": kernel_roofline(m, work, brk),
    }
    print("[bench] decode attention alone ...", file=sys.stderr, flush=True)
    out["decode_attention"] = decode_attention(m, batch, args.seed)
    for pool in pools:
        if pool is not None:
            A.sb_sched_destroy(pool[1])
            A.sb_kv_destroy(pool[0])
    eng.close()
    del eng
    torch.cuda.empty_cache()
    if not args.no_gpt175b:
        print("[bench] GPT-175B-shaped layer ...", file=sys.stderr, flush=True)
        out["gpt175b_layer"] = gpt175b_layer(10, 3, args.seed)
    if not args.no_trace:
        print("[bench] serving trace, whole (chained) ...", file=sys.stderr, flush=True)
        log_path = None
        if args.log_dir:
            os.makedirs(args.log_dir, exist_ok=True)
            log_path = os.path.join(args.log_dir, "trace_iterations.jsonl")
        out["trace"] = trace_run(W, m, args.seed, log_path=log_path, iters=args.trace_iters)
        torch.cuda.empty_cache()
        out["reservation_policies"] = reservation_policies(args.seed)
        print("[bench] iteration-level vs request-level scheduling ...", file=sys.stderr, flush=True)
        out["scheduling"] = scheduling_compare(W, m, args.seed)
    if not args.no_decode_loop:
        print("[bench] mini-model decode loop ...", file=sys.stderr, flush=True)
        out["decode_loop"] = decode_loop(args.seed)
        out["decode_loop_fp32"] = decode_loop(args.seed, dtype="fp32")
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(m.with_layers(args.layers), batch, args.seed)
        out["cpu_mini_iteration"] = cpu_mini(args.seed)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
