"""CPU tests of libsb's host half through the C ABI: exports, K/V manager,
scheduler (bit-exact against the oracle) and the ragged metadata builder."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import selective_batching_amd as sb
from golden import load
from oracle import flat as FL
from oracle import scheduler as OS
from synth import GPT175B_LAYER, LLAMA8B, MINI, TOY, figure5_requests, gpt175b_mixed_batch, llama_mixed_batch, \
    p4_grid_requests, poisson_trace, random_ragged_batch
from selective_batching_amd.runtime import make_dims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in ("sb.h", "sb_ops.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s+\**(sb_[a-z0-9_]+)\s*\(", src, re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    from selective_batching_amd._lib import _PROTOS
    assert names == set(_PROTOS), names ^ set(_PROTOS)      # header and binding agree
    lib = ctypes.CDLL(sb.LIB_PATH)
    missing = [n for n in sorted(names) if not hasattr(lib, n)]
    assert not missing, missing


# ---------------------------------------------------------------- K/V manager
def test_kv_reserve_free_and_errors():
    kv = sb.sb_kv_create(100, sb.sb_kv_arena_slots(100, 4), 2, 2, 16, sb.SB_F32)
    b0 = sb.sb_kv_reserve(kv, 1, 30)
    b1 = sb.sb_kv_reserve(kv, 2, 70)          # exact fit: 30 + 70 == n_slots is admitted
    assert b0 % 8 == 0 and b1 % 8 == 0
    assert sb.sb_kv_stats(kv)["n_rsrv"] == 100
    with pytest.raises(sb.SBError) as e:
        sb.sb_kv_reserve(kv, 3, 1)
    assert e.value.status == sb.SB_ERR_NO_SLOTS
    with pytest.raises(sb.SBError) as e:
        sb.sb_kv_reserve(kv, 1, 1)
    assert e.value.status == sb.SB_ERR_STATE
    sb.sb_kv_free(kv, 1)
    with pytest.raises(sb.SBError) as e:
        sb.sb_kv_free(kv, 1)
    assert e.value.status == sb.SB_ERR_NOT_FOUND
    with pytest.raises(sb.SBError) as e:
        sb.sb_kv_reserve(kv, 9, 101)
    assert e.value.status == sb.SB_ERR_TOO_LARGE
    assert sb.sb_kv_stats(kv)["n_rsrv"] == 70
    sb.sb_kv_destroy(kv)


@pytest.mark.parametrize("seed", range(5))
def test_kv_placement_disjoint_aligned_and_compacts(seed):
    n_slots, max_live = 400, 12
    arena = sb.sb_kv_arena_slots(n_slots, max_live)
    kv = sb.sb_kv_create(n_slots, arena, 1, 1, 8, sb.SB_BF16)
    g = np.random.default_rng(seed)
    live = {}
    nxt = 0
    for _ in range(400):
        if live and (g.random() < 0.45 or len(live) == max_live):
            rid = list(live)[g.integers(len(live))]
            sb.sb_kv_free(kv, rid)
            del live[rid]
        else:
            mt = int(g.integers(1, 60))
            try:
                base = sb.sb_kv_reserve(kv, nxt, mt)
                live[nxt] = mt
            except sb.SBError as e:
                assert e.status == sb.SB_ERR_NO_SLOTS
                assert sum(live.values()) + mt > n_slots      # counter alone decides
            nxt += 1
        spans = sorted((sb.sb_kv_lookup(kv, r)[0], sb.sb_kv_lookup(kv, r)[1]) for r in live)
        end = 0
        for b, mt in spans:
            assert b % 8 == 0 and b >= end
            end = b + mt
        assert end <= arena
        assert sb.sb_kv_stats(kv)["n_rsrv"] == sum(live.values())
    sb.sb_kv_destroy(kv)


def test_select_reports_bases_after_compaction():
    """A reservation that compacts the arena moves the ranges of requests admitted before it: Select must
    hand out the bases the K/V manager holds after the move.  48 slots: A8 B16 C8 D16 fill the arena; A and
    C finish, leaving two 8-slot holes; E16 fits the counter (32 + 16 = 48) but no hole, so B and D are
    packed to 0 and 16 and E lands at 32."""
    kv = sb.sb_kv_create(48, 48, 1, 1, 8, sb.SB_F32)
    s = sb.sb_sched_create(4, kv)
    for rid, (mt, out) in enumerate(((8, 1), (16, 9), (8, 1), (16, 9))):
        sb.sb_sched_add(s, rid, 0.0, [1, 2, 3, 4], out, mt)
    ids, _, _, base = sb.sb_select_batch(s, 4)
    assert list(ids) == [0, 1, 2, 3] and list(base) == [0, 8, 24, 32]
    assert list(sb.sb_sched_complete(s, ids, np.zeros(4, np.int32))) == [0, 2]
    sb.sb_sched_add(s, 4, 1.0, [1, 2, 3, 4], 2, 16)
    ids, _, _, base = sb.sb_select_batch(s, 4)
    assert list(ids) == [1, 3, 4]
    assert sb.sb_kv_stats(kv)["n_compactions"] == 1
    assert list(base) == [sb.sb_kv_lookup(kv, int(r))[0] for r in ids] == [0, 16, 32]
    sb.sb_sched_destroy(s)
    sb.sb_kv_destroy(kv)


@pytest.mark.parametrize("policy", ["pow2", "oracle"])
@pytest.mark.parametrize("chunking", [None, (24, 8)])
def test_select_bases_match_manager_under_binding_reservations(policy, chunking):
    """A trace whose reservations bind (Pow2 / Oracle policies, few slots): on every iteration each member's
    base from Select equals the manager's, the members' ranges are disjoint, 8-aligned, inside the arena and
    hold the member's history plus this iteration's tokens; compaction happens many times."""
    code = {"pow2": sb.SB_RESERVE_POW2, "oracle": sb.SB_RESERVE_ORACLE}[policy]
    reqs = poisson_trace(seed=41, n=300, rate=0.9, plo=1, phi=60, olo=1, ohi=40, reserve_out=40)
    for r in reqs:
        r.max_tokens = sb.sb_reservation_tokens(code, len(r.prompt), r.out_len, 40)
    n_slots, max_bs = 400, 12
    arena = sb.sb_kv_arena_slots(n_slots, max_bs)
    kv = sb.sb_kv_create(n_slots, arena, 1, 1, 8, sb.SB_F32)
    s = sb.sb_sched_create(max_bs, kv)
    if chunking:
        sb.sb_sched_set_chunking(s, *chunking)
    pending = sorted(reqs, key=lambda r: (r.arrival, r.rid))
    mt = {r.rid: r.max_tokens for r in reqs}
    i, t, iters = 0, 0, 0
    while i < len(pending) or sb.sb_sched_stats(s)["pool"]:
        while i < len(pending) and pending[i].arrival <= t:
            r = pending[i]
            sb.sb_sched_add(s, r.rid, r.arrival, r.prompt, r.out_len, r.max_tokens)
            i += 1
        if not sb.sb_sched_stats(s)["pool"]:
            t = int(math.ceil(pending[i].arrival))
            continue
        ids, n_new, ctx, base = sb.sb_select_batch(s, max_bs)
        spans = []
        for rid, n, c, b in zip(ids, n_new, ctx, base):
            lb, lmt = sb.sb_kv_lookup(kv, int(rid))
            assert b == lb and lmt == mt[int(rid)]
            assert b % 8 == 0 and c + n <= lmt
            spans.append((int(b), int(b) + lmt))
        spans.sort()
        assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:])) and (not spans or spans[-1][1] <= arena)
        sb.sb_sched_complete(s, ids, np.zeros(len(ids), np.int32))
        t += 1
        iters += 1
    assert sb.sb_kv_stats(kv)["n_compactions"] >= 10, sb.sb_kv_stats(kv)
    sb.sb_sched_destroy(s)
    sb.sb_kv_destroy(kv)


# ---------------------------------------------------------------- scheduler vs oracle
def native_replay(reqs, max_bs, n_slots, budget=None, chunk=None, usage=None, static=False):
    """The oracle's logical-clock loop, with the scheduling decisions made by libsb."""
    kv = sb.sb_kv_create(n_slots, sb.sb_kv_arena_slots(n_slots, max_bs), 1, 1, 8, sb.SB_F32)
    s = sb.sb_sched_create(max_bs, kv)
    if static:
        sb.sb_sched_set_request_level(s, True)
    if budget is not None:
        sb.sb_sched_set_chunking(s, budget, chunk)
    pending = sorted(reqs, key=lambda r: (r.arrival, r.rid))
    i, t, log = 0, 0, []
    while i < len(pending) or sb.sb_sched_stats(s)["pool"]:
        while i < len(pending) and pending[i].arrival <= t:
            r = pending[i]
            sb.sb_sched_add(s, r.rid, r.arrival, r.prompt, r.out_len, r.max_tokens)
            i += 1
        if not sb.sb_sched_stats(s)["pool"]:
            t = int(math.ceil(pending[i].arrival))
            continue
        ids, n_new, ctx, _ = sb.sb_select_batch(s, max_bs)
        log.append((t, [(int(a), int(b), int(c)) for a, b, c in zip(ids, n_new, ctx)], sb.sb_sched_stats(s)["n_rsrv"]))
        if usage is not None:
            usage.append(sb.sb_kv_usage(s))
        sb.sb_sched_complete(s, ids, np.zeros(len(ids), np.int32))
        t += 1
    sb.sb_sched_destroy(s)
    sb.sb_kv_destroy(kv)
    return log


def test_native_scheduler_p4_timeline():
    g = load("p4_timeline.txt")
    reqs = p4_grid_requests(seed=0)
    log = native_replay(reqs, 3, 10**9)
    assert log == OS.replay(reqs, 3, 10**9)
    assert len(log) == g["iterations"][0]
    rows = OS.timeline(log, reqs)
    for r in reqs:
        assert rows[r.rid] == g[f"r{r.rid}"]


@pytest.mark.parametrize("case", range(6))
def test_native_scheduler_matches_oracle_random(case):
    reqs = poisson_trace(seed=case, n=150, rate=[0.3, 1.0, 2.0, 0.6, 5.0, 0.9][case], plo=1, phi=40, olo=1, ohi=30,
                         reserve_out=30)
    n_slots = [200, 120, 1000, 75, 300, 10**6][case]
    max_bs = [4, 8, 16, 3, 32, 1][case]
    assert native_replay(reqs, max_bs, n_slots) == OS.replay(reqs, max_bs, n_slots)


def test_native_scheduler_matches_oracle_trace_2000():
    """The Poisson trace of the 8B-shaped serving run: 2000 requests, max_bs 64, prompt U[32,512],
    out U[1,512], max_tokens = prompt + 512; slots tight enough that reservations bind."""
    reqs = poisson_trace(seed=0, n=2000, rate=0.5)
    for n_slots in (20000, 65536):
        assert native_replay(reqs, 64, n_slots) == OS.replay(reqs, 64, n_slots)


@pytest.mark.parametrize("case", range(5))
def test_native_chunked_scheduler_matches_oracle(case):
    """Chunked prefill under a token budget: libsb's decisions equal the oracle's, iteration by iteration
    (the hand-worked example, then random traces with binding reservations and budgets)."""
    if case == 0:
        from golden import load as gload
        g = gload("chunked_prefill.txt")

        class R:
            def __init__(self, rid, a, p, o):
                self.rid, self.arrival, self.prompt, self.out_len, self.max_tokens = rid, a, [0] * p, o, p + o
        reqs = [R(i, a, p, o) for i, (a, p, o) in enumerate(zip(g["arrivals"], g["prompt"], g["out_len"]))]
        assert native_replay(reqs, 4, 10**9, 6, 4) == OS.replay(reqs, 4, 10**9, budget=6, chunk=4)
        return
    budget, chunk, max_bs, n_slots = [None, (16, 8, 4, 300), (64, 16, 8, 700), (7, 3, 3, 150), (512, 128, 16, 3000)][case]
    reqs = poisson_trace(seed=200 + case, n=150, rate=[0, 0.5, 1.0, 0.3, 2.0][case], plo=1, phi=80, olo=1, ohi=25,
                         reserve_out=25)
    assert native_replay(reqs, max_bs, n_slots, budget, chunk) == \
        OS.replay(reqs, max_bs, n_slots, budget=budget, chunk=chunk)


@pytest.mark.parametrize("policy", ["max", "pow2", "oracle"])
def test_native_reservation_policies_and_kv_usage_match_oracle(policy):
    """sb_reservation_tokens == the oracle's policy; sb_kv_usage == the oracle's reserved / stored slots on
    every iteration of a trace (with and without chunked prefill)."""
    code = {"max": sb.SB_RESERVE_MAX, "pow2": sb.SB_RESERVE_POW2, "oracle": sb.SB_RESERVE_ORACLE}[policy]
    for p, n in ((1, 1), (5, 2), (10, 25), (300, 511), (40, 512)):
        assert sb.sb_reservation_tokens(code, p, n, 512) == OS.reservation(policy, p, n, 512)
    reqs = poisson_trace(seed=31, n=200, rate=0.8, plo=1, phi=80, olo=1, ohi=40, reserve_out=40)
    for r in reqs:
        r.max_tokens = sb.sb_reservation_tokens(code, len(r.prompt), r.out_len, 40)
    for budget, chunk in ((None, None), (24, 8)):
        usage = []
        log = native_replay(reqs, 12, 900, budget, chunk, usage)
        olog = OS.replay(reqs, 12, 900, budget=budget, chunk=chunk)
        assert log == olog
        _, _, stored = OS.kv_usage(olog, reqs, 900)
        assert [u[0] for u in usage] == [n for _, _, n in olog] and [u[1] for u in usage] == stored


def test_reservation_policy_errors():
    for args in ((3, 1, 2, 4), (0, 1, 0, 4), (0, 0, 2, 4), (0, 1, 5, 4)):
        with pytest.raises(sb.SBError) as e:
            sb.sb_reservation_tokens(*args)
        assert e.value.status == sb.SB_ERR_INVALID


def test_native_request_level_matches_oracle():
    """Static batching in libsb: the lecture's static grid (18 iterations) and random traces with
    reservations that bind, decision for decision against the oracle."""
    reqs = p4_grid_requests(seed=0)
    log = native_replay(reqs, 3, 10**9, static=True)
    assert log == OS.replay(reqs, 3, 10**9, static=True) and len(log) == 18
    for seed, (max_bs, n_slots) in enumerate(((4, 200), (8, 300), (16, 10**6))):
        reqs = poisson_trace(seed=60 + seed, n=120, rate=1.0, plo=1, phi=40, olo=1, ohi=30, reserve_out=30)
        assert native_replay(reqs, max_bs, n_slots, static=True) == OS.replay(reqs, max_bs, n_slots, static=True)
    kv = sb.sb_kv_create(10, sb.sb_kv_arena_slots(10, 2), 1, 1, 8, sb.SB_F32)
    s = sb.sb_sched_create(2, kv)
    sb.sb_sched_set_chunking(s, 8, 4)
    with pytest.raises(sb.SBError) as e:
        sb.sb_sched_set_request_level(s, True)              # chunks and whole-batch scheduling exclude
    assert e.value.status == sb.SB_ERR_INVALID
    sb.sb_sched_destroy(s)
    sb.sb_kv_destroy(kv)


def test_chunking_argument_errors():
    kv = sb.sb_kv_create(10, sb.sb_kv_arena_slots(10, 2), 1, 1, 8, sb.SB_F32)
    s = sb.sb_sched_create(2, kv)
    for bad in ((0, 4), (8, 0), (-1, -1)):
        with pytest.raises(sb.SBError) as e:
            sb.sb_sched_set_chunking(s, *bad)
        assert e.value.status == sb.SB_ERR_INVALID
    sb.sb_sched_set_chunking(s, 8, 4)
    sb.sb_sched_set_chunking(s, 0, 0)
    sb.sb_sched_destroy(s)
    sb.sb_kv_destroy(kv)


def test_native_scheduler_tokens_and_outputs():
    kv = sb.sb_kv_create(64, sb.sb_kv_arena_slots(64, 4), 1, 1, 8, sb.SB_F32)
    s = sb.sb_sched_create(4, kv)
    reqs = figure5_requests(seed=0)
    for r in reqs[:2]:
        sb.sb_sched_add(s, r.rid, r.arrival, r.prompt, 8, r.max_tokens)
    ids, n_new, ctx, base = sb.sb_select_batch(s, 4)
    assert list(ids) == [0, 1] and list(n_new) == [3, 1] and list(ctx) == [0, 0]
    assert list(sb.sb_batch_tokens(s, ids, 16)) == reqs[0].prompt + reqs[1].prompt
    sb.sb_sched_complete(s, ids, [11, 12])
    for r in reqs[2:]:
        sb.sb_sched_add(s, r.rid, r.arrival, r.prompt, 8, r.max_tokens)
    ids, n_new, ctx, base = sb.sb_select_batch(s, 4)
    g = load("figure5.txt")
    assert list(n_new) == g["n_new"] and list(ctx) == g["ctx"]
    assert list(sb.sb_batch_tokens(s, ids, 16)) == [11, 12] + reqs[2].prompt + reqs[3].prompt
    sb.sb_sched_complete(s, ids, [21, 22, 23, 24])
    assert list(sb.sb_sched_output(s, 0)) == [11, 21]
    with pytest.raises(sb.SBError) as e:
        sb.sb_sched_complete(s, ids, [0, 0, 0, 0])         # they are not running any more
    assert e.value.status == sb.SB_ERR_STATE


def test_native_scheduler_errors():
    kv = sb.sb_kv_create(10, sb.sb_kv_arena_slots(10, 2), 1, 1, 8, sb.SB_F32)
    with pytest.raises(sb.SBError) as e:
        sb.sb_sched_create(0, kv)
    assert e.value.status == sb.SB_ERR_INVALID
    s = sb.sb_sched_create(2, kv)
    with pytest.raises(sb.SBError) as e:
        sb.sb_sched_add(s, 0, 0.0, [1, 2, 3], 9, 11)
    assert e.value.status == sb.SB_ERR_TOO_LARGE
    ids, *_ = sb.sb_select_batch(s, 2)
    assert len(ids) == 0                                    # empty pool -> empty batch
    sb.sb_sched_add(s, 1, 0.0, [1], 1, 1)
    with pytest.raises(sb.SBError) as e:
        sb.sb_sched_add(s, 1, 0.0, [1], 1, 1)
    assert e.value.status == sb.SB_ERR_STATE
    ids, *_ = sb.sb_select_batch(s, 2)
    fin = sb.sb_sched_complete(s, ids, [5])
    assert list(fin) == [1] and sb.sb_kv_stats(kv)["n_rsrv"] == 0


def _fake_token(rid, k, V=1000):
    """Stand-in for the model: the k-th generated token of request rid."""
    return (rid * 7919 + k * 104729 + 13) % V


def _deferred_vs_sync(reqs, max_bs, n_slots, chunking=None):
    """Drive two schedulers with the same arrivals: one completes with the token values, the other one
    iteration ahead (deferred completion; the decodes' tokens resolved from the previous iteration's
    'device' ids through their references).  Batches, fed tokens and outputs must agree."""
    kvs = [sb.sb_kv_create(n_slots, sb.sb_kv_arena_slots(n_slots, max_bs), 1, 1, 8, sb.SB_F32) for _ in range(2)]
    sy, de = sb.sb_sched_create(max_bs, kvs[0]), sb.sb_sched_create(max_bs, kvs[1])
    if chunking is not None:
        for s_ in (sy, de):
            sb.sb_sched_set_chunking(s_, *chunking)
    plen = {r.rid: len(r.prompt) for r in reqs}
    pending = sorted(reqs, key=lambda r: (r.arrival, r.rid))
    made = {r.rid: 0 for r in reqs}            # tokens generated so far (the fake model's clock per request)
    i, t, n_iter, prev = 0, 0, 0, None          # prev: (ids, device ids, ticket) of the deferred side
    while True:
        if prev is not None:
            _, ticket = sb.sb_sched_complete_deferred(de, prev[0])
            prev = (prev[0], prev[1], ticket)
        while i < len(pending) and pending[i].arrival <= t:
            r = pending[i]
            for s_ in (sy, de):
                sb.sb_sched_add(s_, r.rid, r.arrival, r.prompt, r.out_len, r.max_tokens)
            i += 1
        ids, n_new, ctx, _ = sb.sb_select_batch(sy, max_bs)
        ids_d, n_new_d, ctx_d, _ = sb.sb_select_batch(de, max_bs)
        assert list(ids) == list(ids_d) and list(n_new) == list(n_new_d) and list(ctx) == list(ctx_d)
        if len(ids):
            want = sb.sb_batch_tokens(sy, ids, 4096)
            refs, ticket = sb.sb_batch_token_refs(de, ids, 4096)
            if prev is None:
                assert ticket == -1
            if ticket >= 0:
                assert ticket == prev[2]
                if (refs < 0).any():
                    with pytest.raises(sb.SBError) as e:            # values unknown: plain tokens refuse
                        sb.sb_batch_tokens(de, ids, 4096)
                    assert e.value.status == sb.SB_ERR_STATE
            got = np.array([prev[1][-1 - v] if v < 0 else v for v in refs], np.int32)
            assert list(got) == list(want)
            # members that yield a token: decodes and the chunk that ends a prompt (others: ignored value)
            emits = [int(c) + int(n) >= plen[int(r)] for r, n, c in zip(ids, n_new, ctx)]
            out = np.array([_fake_token(int(r), made[int(r)]) if e else -7 for r, e in zip(ids, emits)], np.int32)
            for r, e in zip(ids, emits):
                made[int(r)] += e
            sb.sb_sched_complete(sy, ids, out)
        if prev is not None:
            sb.sb_sched_set_tokens(de, prev[2], prev[1])
            with pytest.raises(sb.SBError) as e:
                sb.sb_sched_set_tokens(de, prev[2], prev[1])       # settled once only
            assert e.value.status == sb.SB_ERR_NOT_FOUND
        if not len(ids):
            prev = None
            if i >= len(pending):
                break
            t = int(math.ceil(pending[i].arrival))
            continue
        prev, n_iter, t = (ids, out, None), n_iter + 1, t + 1
    for r in reqs:
        assert list(sb.sb_sched_output(de, r.rid)) == list(sb.sb_sched_output(sy, r.rid)) == \
            [_fake_token(r.rid, k) for k in range(r.out_len)]
    for s_ in (sy, de):
        sb.sb_sched_destroy(s_)
    for kv in kvs:
        assert sb.sb_kv_stats(kv)["n_rsrv"] == 0
        sb.sb_kv_destroy(kv)
    return n_iter


def test_deferred_completion_p4_timeline_and_figure5():
    """Completion one iteration behind (NEXT-1 of the plan: select and launch t+1 before t's ids reach
    the host) schedules exactly as the synchronous loop: the lecture's 10-iteration grid, Figure 5 with
    the reservation binding (x4 blocked at 30 slots)."""
    assert _deferred_vs_sync(p4_grid_requests(seed=0), 3, 10**9) == 10
    for n_slots in (64, 30):
        _deferred_vs_sync(figure5_requests(seed=0, vocab=1000, out_len=8), 4, n_slots)


@pytest.mark.parametrize("chunking", [(16, 8), (5, 2)])
def test_deferred_completion_with_chunked_prefill(chunking):
    """Deferred completion with prompt chunks that yield no token: references still point at the rows
    that did yield one."""
    reqs = poisson_trace(seed=21, n=60, rate=0.7, plo=1, phi=40, olo=1, ohi=15, reserve_out=15, vocab=1000,
                         with_prompts=True)
    _deferred_vs_sync(reqs, 6, 400, chunking)


@pytest.mark.parametrize("case", range(3))
def test_deferred_completion_random_traces(case):
    reqs = poisson_trace(seed=10 + case, n=120, rate=[0.5, 2.0, 0.2][case], plo=1, phi=30, olo=1, ohi=20,
                         reserve_out=20, vocab=1000, with_prompts=True)
    _deferred_vs_sync(reqs, [4, 16, 2][case], [150, 400, 60][case])


def test_deferred_completion_errors():
    kv = sb.sb_kv_create(64, sb.sb_kv_arena_slots(64, 4), 1, 1, 8, sb.SB_F32)
    s = sb.sb_sched_create(4, kv)
    sb.sb_sched_add(s, 0, 0.0, [5, 6], 3, 8)
    ids, *_ = sb.sb_select_batch(s, 4)
    _, t0 = sb.sb_sched_complete_deferred(s, ids)
    with pytest.raises(sb.SBError) as e:
        sb.sb_sched_set_tokens(s, t0, [1, 2])                      # one request in that batch
    assert e.value.status == sb.SB_ERR_INVALID
    with pytest.raises(sb.SBError) as e:
        sb.sb_sched_set_tokens(s, t0 + 5, [1])
    assert e.value.status == sb.SB_ERR_NOT_FOUND
    ids, *_ = sb.sb_select_batch(s, 4)
    refs, tk = sb.sb_batch_token_refs(s, ids, 16)
    assert list(refs) == [-1] and tk == t0
    _, t1 = sb.sb_sched_complete_deferred(s, ids)                   # second pending token, newer ticket
    ids, *_ = sb.sb_select_batch(s, 4)
    refs, tk = sb.sb_batch_token_refs(s, ids, 16)
    assert list(refs) == [-1] and tk == t1
    sb.sb_sched_set_tokens(s, t1, [42])
    sb.sb_sched_set_tokens(s, t0, [41])
    assert list(sb.sb_sched_output(s, 0)) == [41, 42]
    assert list(sb.sb_batch_tokens(s, ids, 16)) == [42]
    sb.sb_sched_destroy(s)
    sb.sb_kv_destroy(kv)


def test_ragged_rejects_token_ids_out_of_range():
    dims = make_dims(TOY, "fp32")
    buf = np.zeros(1 << 16, np.int32)
    sb.sb_ragged_build(dims, [2], [0], [0], [-1, TOY.V - 1], buf.ctypes.data, None, buf.nbytes)   # ref + literal
    for bad in ([TOY.V, 0], [0, -(1 << 20) - 1]):
        with pytest.raises(sb.SBError) as e:
            sb.sb_ragged_build(dims, [2], [0], [0], bad, buf.ctypes.data, None, buf.nbytes)
        assert e.value.status == sb.SB_ERR_INVALID


# ---------------------------------------------------------------- ragged metadata
def host_ragged(m, dtype, batch, slot_base=None, tokens=None):
    dims = make_dims(m, dtype)
    n_new = [b[0] for b in batch]
    ctx = [b[1] for b in batch]
    if slot_base is None:
        slot_base, acc = [], 0
        for n, c in batch:
            slot_base.append(acc)
            acc += (n + c + 7) // 8 * 8
    keys = sum(n + c for n, c in batch)
    nbytes = sb.sb_ragged_bytes(dims, len(batch), sum(n_new), keys)
    buf = np.zeros(nbytes // 4 + 1, np.int32)
    rg = sb.sb_ragged_build(dims, n_new, ctx, slot_base, tokens, buf.ctypes.data, None, nbytes)
    return rg, buf, slot_base


def _arr(ptr, n):
    return np.ctypeslib.as_array((ctypes.c_int32 * n).from_address(ptr)).copy() if n else np.zeros(0, np.int32)


@pytest.mark.parametrize("name", ["figure5", "exercise4"])
def test_ragged_metadata_pinned_batches(name):
    g = load(f"{name}.txt")
    batch = list(zip(g["n_new"], g["ctx"]))
    rg, _, base = host_ragged(TOY, "fp32", batch)
    B, T = len(batch), rg.n_tokens
    assert T == g["tokens"][0]
    assert list(_arr(rg.cu_seqlens, B + 1)) == FL.cu_seqlens(batch)
    assert list(_arr(rg.ctx_lens, B)) == g["ctx"]
    assert list(_arr(rg.tok_pos, T)) == FL.positions(batch)
    assert list(_arr(rg.last_row, B)) == FL.last_rows(batch)
    want_slots = [base[i] + c + j for i, (n, c) in enumerate(batch) for j in range(n)]
    assert list(_arr(rg.tok_slot, T)) == want_slots


UNIT = 512   # keys per independently reduced unit (the library's kUnitKeys)
ITEM_INTS = 12   # ints per attention work item (the library's kItemInts)


def _coverage(m, batch, rg, rg_dtype="bf16"):
    """Every (request, kv head, row) must see every visible key exactly once across the work items: row tiles
    (mode 0) and runs of whole key units (mode 1); a request split over several runs leaves one partial per
    unit, named in order by one combine group."""
    G = m.nq // m.nkv
    items = _arr(rg.items, rg.n_items * ITEM_INTS).reshape(-1, ITEM_INTS)
    cu = FL.cu_seqlens(batch)
    slots = _arr(rg.tok_slot, rg.n_tokens)
    spans = {}          # (request, kv head, row) -> key intervals seen by that row
    empty = items[:, 4] == 0                         # padding of the dispatch order: no rows, no keys
    assert np.all(items[empty][:, [2, 3, 5, 6]] == 0) and np.all(items[empty][:, 7] == -1)
    assert empty.sum() <= (len(items) - empty.sum()) // 4 + 8
    items = items[~empty]
    rbs = set()
    for req, kvh, mode, row0, nrows, kb, ke, part, tok0, ctx_i, slot0, rb in items:
        n_new, ctx = batch[req]
        # the request's first row, cached tokens and slot base, carried by the item
        assert tok0 == cu[req] and ctx_i == ctx and slot0 == slots[cu[req]] - ctx
        assert 0 <= kb < ke <= n_new + ctx
        if mode == 0:
            # row tiles of rb 16-row blocks per wave (two only in bf16), one choice for the whole batch
            assert rb in ((1, 2) if rg_dtype == "bf16" else (1,))
            rbs.add(int(rb))
            assert nrows <= 64 * rb and row0 % (64 * rb) == 0 and kb == 0 and part == -1
        else:
            assert mode == 1 and row0 == 0 and nrows == n_new * G <= 16
            assert kb % UNIT == 0 and ((ke - kb) % UNIT == 0 or ke == n_new + ctx)
        for r in range(row0, row0 + nrows):
            tok = r // G
            assert tok < n_new
            hi = min(ke, ctx + tok + 1)
            if hi > kb:
                spans.setdefault((req, kvh, r), []).append((kb, hi))
    # each row's intervals tile [0, ctx + tok + 1) exactly: no key missed, none seen twice
    for req, (n_new, ctx) in enumerate(batch):
        for kvh in range(m.nkv):
            for r in range(n_new * G):
                iv = sorted(spans.pop((req, kvh, r)))
                assert iv[0][0] == 0 and iv[-1][1] == ctx + r // G + 1
                assert all(a[1] == b[0] for a, b in zip(iv, iv[1:]))
    assert not spans
    assert len(rbs) <= 1
    groups = _arr(rg.groups, rg.n_groups * 8).reshape(-1, 8)
    p0 = {}
    for req, kvh, row0, nrows, gp0, np_, tok0, _ in groups:
        n_new, ctx = batch[req]
        assert tok0 == cu[req]
        assert np_ == -(-(n_new + ctx) // UNIT) > 1 and row0 == 0 and nrows == n_new * G
        p0[(req, kvh)] = gp0
    assert sorted(int(g[4]) + u for g in groups for u in range(g[5])) == list(range(rg.n_partials))
    runs = items[items[:, 2] == 1]
    for req, kvh, _, _, _, kb, ke, part in runs[:, :8]:
        if part >= 0:       # one of several runs of the request: partials of its units, in unit order
            assert part == p0[(req, kvh)] + kb // UNIT
        else:               # the run covers all of the request's units
            assert (req, kvh) not in p0 and kb == 0 and ke == sum(batch[req])


@pytest.mark.parametrize("m,dtype", [(TOY, "fp32"), (MINI, "bf16"), (LLAMA8B, "bf16")])
@pytest.mark.parametrize("seed", range(4))
def test_attention_work_list_covers_each_pair_once(m, dtype, seed):
    batch = random_ragged_batch(seed, 6, 1100, 40)
    rg, buf, _ = host_ragged(m, dtype, batch)
    _coverage(m, batch, rg, dtype)


def test_attention_work_list_llama_mixed_batch_counts():
    batch = llama_mixed_batch(seed=0)
    rg, buf, _ = host_ragged(LLAMA8B, "bf16", batch)
    assert rg.n_req == 256 and rg.n_tokens == sum(n for n, _ in batch)
    _coverage(LLAMA8B, batch, rg)
    items = _arr(rg.items, rg.n_items * ITEM_INTS).reshape(-1, ITEM_INTS)
    # 1816 tiles of 64 rows: the row tiles take two 16-row blocks per wave (128 rows)
    assert set(items[items[:, 2] == 0][:, 11]) == {2}
    # decode runs carry most of this batch's work: heaviest first (row tiles weighted 4 x their keys),
    # no padding
    assert np.all(items[:, 4] > 0)
    cost = np.where(items[:, 2] == 0, 4 * items[:, 6], items[:, 6] - items[:, 5])
    assert np.all(np.diff(cost) <= 0)
    # at this size every decode's units fit one run: no partials, no combine
    assert rg.n_partials == 0 and rg.n_groups == 0
    assert FL.useful_pairs(batch) > 0


@pytest.mark.parametrize("m,batch", [(LLAMA8B, "llama prefills"), (GPT175B_LAYER, "gpt175b prefills")])
def test_attention_work_list_prefill_heavy_xcd_lanes(m, batch):
    """Prefill tiles carry most of the work: the row tiles of one request and K/V head sit at indices of one
    residue mod 8 (one XCD: workgroups are dealt to the 8 XCDs round-robin), consecutive within that XCD's
    lane; empty padding items stay within a quarter of the others; every (request, head, row, key) is
    still covered exactly once."""
    src = llama_mixed_batch(seed=0) if m is LLAMA8B else gpt175b_mixed_batch(seed=0)
    b = [x for x in src if x[0] > 1][:8]
    rg, buf, _ = host_ragged(m, "bf16", b)
    _coverage(m, b, rg)
    items = _arr(rg.items, rg.n_items * ITEM_INTS).reshape(-1, ITEM_INTS)
    assert len(items) % 8 == 0
    pos = {}
    for k, (req, kvh, mode, row0, nrows) in enumerate(items[:, :5]):
        if nrows and mode == 0:
            pos.setdefault((req, kvh), []).append(k)
    assert len(pos) == len(b) * m.nkv
    for ks in pos.values():
        assert len({k % 8 for k in ks}) == 1
        assert np.all(np.diff(ks) == 8)


def test_attention_work_list_small_batch_one_unit_per_run():
    """Few keys in all: one unit per run, so even a single long request spreads over many workgroups, and
    the partials stay within the bound the workspace is sized by."""
    batch = [(1, 2047)]
    rg, buf, _ = host_ragged(LLAMA8B, "bf16", batch)
    _coverage(LLAMA8B, batch, rg)
    assert rg.n_items == 8 * 4 and rg.n_partials == 8 * 4 and rg.n_groups == 8
    assert rg.n_partials <= sb.sb_attn_max_partials(make_dims(LLAMA8B, "bf16"), 1, 2048)


def test_ragged_rejects_bad_input():
    dims = make_dims(TOY, "fp32")
    buf = np.zeros(4096, np.int32)
    with pytest.raises(sb.SBError) as e:
        sb.sb_ragged_build(dims, [1], [0], [3], None, buf.ctypes.data, None, buf.nbytes)   # unaligned slot base
    assert e.value.status == sb.SB_ERR_INVALID
    with pytest.raises(sb.SBError) as e:
        sb.sb_ragged_build(dims, [0], [0], [0], None, buf.ctypes.data, None, buf.nbytes)
    assert e.value.status == sb.SB_ERR_INVALID
    with pytest.raises(sb.SBError) as e:
        sb.sb_ragged_build(dims, [5] * 300, [0] * 300, [0] * 300, None, buf.ctypes.data, None, 64)
    assert e.value.status in (sb.SB_ERR_WORKSPACE, sb.SB_ERR_INVALID)


@pytest.mark.parametrize("dtype,head_dim", [("bf16", 96), ("bf16", 16), ("fp32", 48), ("fp32", 80), ("fp32", 96),
                                            ("fp32", 112)])
def test_ragged_rejects_head_dims_attention_lacks(dtype, head_dim):
    """Only the head dims the attention kernel is built for pass validation (bf16 32/64/128, fp32
    16/32/64/128): any other is refused at the first call that takes the shape, before any launch."""
    from synth import ModelDims
    nq = 4 if head_dim != 112 else 8
    m = ModelDims("hd", "llama", n_layers=1, H=nq * head_dim, nq=nq, nkv=nq, d=head_dim, F=256, V=64, max_pos=0)
    dims = make_dims(m, dtype)
    buf = np.zeros(4096, np.int32)
    with pytest.raises(sb.SBError) as e:
        sb.sb_ragged_build(dims, [1], [0], [0], None, buf.ctypes.data, None, buf.nbytes)
    assert e.value.status == sb.SB_ERR_INVALID and "head_dim" in str(e.value)
    assert sb.sb_ragged_bytes(dims, 4, 16, 64) == 0
    for ok in ((("bf16", d) for d in (32, 64, 128)), (("fp32", d) for d in (16, 32, 64, 128))):
        for dt, d in ok:
            mm = ModelDims("hd", "llama", n_layers=1, H=4 * d, nq=4, nkv=4, d=d, F=256, V=64, max_pos=0)
            sb.sb_ragged_build(make_dims(mm, dt), [1], [0], [0], None, buf.ctypes.data, None, buf.nbytes)


@pytest.mark.parametrize("epi", ["store", "resid", "swiglu"])
def test_gemm_rejects_operands_past_32bit_offsets(epi):
    """The GEMM kernels index operands with 32-bit element offsets: an operand of 2^31 elements or more is
    refused on the host, before any launch (the pointers here are never touched).  A GPT-175B-shaped FFN2
    at 43,691 rows has an A operand of 43,691 x 49152 > 2^31 elements."""
    code = {"store": sb.SB_EPI_STORE, "resid": sb.SB_EPI_RESID, "swiglu": sb.SB_EPI_SWIGLU}[epi]
    fake = 1 << 20
    K, F = 49152, 12288
    cases = [(43691, 12288, K, K, K, 12288, F)]                 # M * lda >= 2^31
    cases.append((16, 12288, 4096, 4096, 1 << 18, 12288, F))     # weight rows * ldw >= 2^31
    cases.append((1 << 17, 64, 64, 64, 64, 1 << 14, 64))         # M * ldc >= 2^31
    if epi == "swiglu":
        cases.append((16, 64, 4096, 4096, 4096, 64, 1 << 18))   # 2F weight rows * ldw >= 2^31
    for M, N, Kk, lda, ldw, ldc, FF in cases:
        with pytest.raises(sb.SBError) as e:
            sb.sb_op_gemm(sb.SB_BF16, code, M, N, Kk, fake, lda, fake, ldw, None, fake, ldc, 0, FF)
        assert e.value.status == sb.SB_ERR_INVALID and "2^31" in str(e.value)
