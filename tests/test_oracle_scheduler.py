"""Pins of the oracle scheduler against the pages' worked examples and invariants."""
import itertools

import numpy as np
import pytest

from golden import load
from oracle import scheduler as S
from synth import figure5_requests, p4_grid_requests, poisson_trace, rng_for


def test_p4_continuous_timeline_exact():
    g = load("p4_timeline.txt")
    reqs = p4_grid_requests(seed=0)
    assert [int(r.arrival) for r in reqs] == g["arrivals"]
    assert [r.out_len for r in reqs] == g["out_len"]
    log = S.replay(reqs, max_bs=g["max_bs"][0], n_slots=10**9)
    assert len(log) == g["iterations"][0]
    rows = S.timeline(log, reqs)
    for r in reqs:
        assert rows[r.rid] == g[f"r{r.rid}"], (r.rid, rows[r.rid])


def test_figure3_iterations():
    g = load("figure3.txt")

    class R:
        pass

    reqs = []
    for i, (pl, n) in enumerate(zip(g["prompt_len"], g["iterations_needed"])):
        r = R()
        r.rid, r.arrival, r.prompt, r.out_len, r.max_tokens = i, 0.0, [0] * pl, n, pl + n
        reqs.append(r)
    log = S.replay(reqs, max_bs=8, n_slots=100)
    last = {}
    for t, work, _ in log:
        for rid, _, _ in work:
            last[rid] = t
    # x2 leaves after its 2nd iteration, x1 after its 4th; nobody waits for anybody.
    assert last == {0: 3, 1: 1}
    assert len(log) == 4


def _brute_select(pool, n_rsrv, max_bs, n_slots):
    """Largest k such that the first k arrival-ordered candidates respect both limits."""
    cand = sorted((r for r in pool if r.state != S.RUNNING), key=lambda r: (r.arrival, r.order))
    best = 0
    for k in range(len(cand) + 1):
        need = sum(r.max_tokens for r in cand[:k] if r.state == S.INITIATION)
        if k <= max_bs and n_rsrv + need <= n_slots:
            best = k
        else:
            break
    need = sum(r.max_tokens for r in cand[:best] if r.state == S.INITIATION)
    return [r.rid for r in cand[:best]], n_rsrv + need


@pytest.mark.parametrize("seed", range(40))
def test_select_is_longest_feasible_prefix(seed):
    g = rng_for(seed, "select-brute")
    n = int(g.integers(0, 9))
    pool = []
    for i in range(n):
        r = S.SReq(i, float(g.integers(0, 4)), int(g.integers(0, 100)), 1, 1, int(g.integers(1, 20)))
        r.state = [S.INITIATION, S.INCREMENT][int(g.integers(0, 2))]
        pool.append(r)
    n_slots = int(g.integers(1, 60))
    n_rsrv = int(g.integers(0, n_slots + 1))
    max_bs = int(g.integers(1, 6))
    batch, nr = S.select(pool, n_rsrv, max_bs, n_slots)
    want_ids, want_nr = _brute_select(pool, n_rsrv, max_bs, n_slots)
    assert [r.rid for r in batch] == want_ids
    assert nr == want_nr


def _check_invariants(reqs, log, max_bs, n_slots):
    arrival = {r.rid: r.arrival for r in reqs}
    order = {r.rid: i for i, r in enumerate(sorted(reqs, key=lambda r: (r.arrival, r.rid)))}
    max_tok = {r.rid: r.max_tokens for r in reqs}
    out_len = {r.rid: r.out_len for r in reqs}
    runs = {r.rid: 0 for r in reqs}
    live = set()
    for t, work, n_rsrv in log:
        ids = [w[0] for w in work]
        assert 1 <= len(ids) <= max_bs
        # batch is in arrival order
        assert ids == sorted(ids, key=lambda i: order[i])
        # every admitted, unfinished request runs every iteration (no skipping)
        assert live <= set(ids)
        for i in ids:
            assert arrival[i] <= t
            live.add(i)
        assert n_rsrv == sum(max_tok[i] for i in live) <= n_slots
        for i in ids:
            runs[i] += 1
        # iteration-level FCFS: an earlier arrival has run at least as many iterations
        arrived = [r.rid for r in reqs if r.arrival <= t]
        for a, b in itertools.combinations(sorted(arrived, key=lambda i: order[i]), 2):
            assert runs[a] >= runs[b] or runs[a] == out_len[a]
        # waiting requests were not skipped: a waiting arrival never precedes an admitted newcomer
        waiting = [i for i in arrived if runs[i] == 0]
        if waiting:
            first_wait = min(order[i] for i in waiting)
            assert all(order[i] < first_wait for i in live)
        for i in ids:
            if runs[i] == out_len[i]:
                live.discard(i)
    assert all(runs[r.rid] == r.out_len for r in reqs)


@pytest.mark.parametrize("seed", range(6))
def test_replay_invariants_random_trace(seed):
    reqs = poisson_trace(seed=seed, n=60, rate=0.8, plo=1, phi=20, olo=1, ohi=15, reserve_out=15)
    n_slots = [40, 80, 200, 10**6, 36, 60][seed]
    max_bs = [2, 3, 8, 4, 16, 1][seed]
    log = S.replay(reqs, max_bs=max_bs, n_slots=n_slots)
    _check_invariants(reqs, log, max_bs, n_slots)


def test_max_bs_one_is_sequential():
    reqs = poisson_trace(seed=3, n=12, rate=2.0, plo=1, phi=5, olo=1, ohi=4, reserve_out=4)
    log = S.replay(reqs, max_bs=1, n_slots=10**6)
    seq = [w[0][0] for _, w, _ in log]
    want = []
    for r in sorted(reqs, key=lambda r: (r.arrival, r.rid)):
        want += [r.rid] * r.out_len
    assert seq == want


def test_reservation_exact_fit_admitted_and_blocking():
    # figure-5 requests: max_tokens 11, 9, 10, 11.  n_slots = 30: x3 fits exactly, x4 must wait.
    reqs = figure5_requests(seed=0)
    log = S.replay(reqs, max_bs=4, n_slots=30)
    t1 = [w for t, w, _ in log if t == 1][0]
    assert [w[0] for w in t1] == [0, 1, 2]
    first_x4 = min(t for t, w, _ in log if any(x[0] == 3 for x in w))
    # x4 starts only once the requests freed enough slots (after the first finisher, x1 at 8 tokens)
    assert first_x4 == 8
    _check_invariants(reqs, log, 4, 30)


def test_too_large_rejected():
    s = S.Scheduler(max_bs=4, n_slots=10)
    with pytest.raises(S.TooLarge):
        s.add(0, 0.0, 5, 6, 11)
    s.add(1, 0.0, 5, 5, 10)
    assert [r.rid for r in s.select()] == [1]


def test_head_of_line_blocking_no_skip():
    s = S.Scheduler(max_bs=8, n_slots=20)
    s.add(0, 0.0, 5, 3, 12)
    s.add(1, 1.0, 5, 3, 12)   # does not fit next to request 0
    s.add(2, 2.0, 1, 1, 2)    # would fit, but must not jump the queue
    assert [r.rid for r in s.select()] == [0]
    assert s.n_rsrv == 12


def test_empty_pool_clock_jumps():
    reqs = poisson_trace(seed=1, n=3, rate=0.01, plo=1, phi=2, olo=1, ohi=2, reserve_out=2)
    log = S.replay(reqs, max_bs=4, n_slots=100)
    starts = [t for t, _, _ in log]
    assert starts[0] == int(np.ceil(reqs[0].arrival))


# ---------------------------------------------------------------- chunked prefill
class _CReq:
    def __init__(self, rid, arrival, prompt_len, out_len, max_tokens):
        self.rid, self.arrival, self.prompt_len, self.out_len, self.max_tokens = rid, arrival, prompt_len, out_len, \
            max_tokens


def test_chunked_prefill_hand_worked_example():
    g = load("chunked_prefill.txt")
    names = "ABC"
    reqs = [_CReq(i, a, p, o, p + o) for i, (a, p, o) in enumerate(zip(g["arrivals"], g["prompt"], g["out_len"]))]
    log = S.replay(reqs, g["max_bs"][0], 10**9, budget=g["budget"][0], chunk=g["chunk"][0])
    got = {f"t{t}": [f"{names[rid]}:{n}:{c}" for rid, n, c in work] for t, work, _ in log}
    want = {k: v for k, v in g.items() if k.startswith("t") and k[1:].isdigit()}
    assert got == want


@pytest.mark.parametrize("seed", range(4))
def test_chunked_prefill_unbounded_is_algorithm1(seed):
    """An unlimited budget and chunk reduce the chunked Select to Algorithm 1 exactly (the p4 grid, and
    random traces with reservations that bind)."""
    reqs = p4_grid_requests(seed=0)
    assert S.replay(reqs, 3, 10**9, budget=10**9, chunk=10**9) == S.replay(reqs, 3, 10**9)
    reqs = poisson_trace(seed=seed, n=200, rate=[0.5, 2.0, 1.0, 0.3][seed], plo=1, phi=40, olo=1, ohi=30,
                         reserve_out=30)
    for max_bs, n_slots in ((4, 200), (16, 500), (2, 10**6)):
        assert S.replay(reqs, max_bs, n_slots, budget=10**9, chunk=10**9) == S.replay(reqs, max_bs, n_slots)


@pytest.mark.parametrize("seed", range(6))
def test_chunked_prefill_invariants(seed):
    """Budget respected, each prompt fed once in order in chunks <= chunk, decodes before prompt chunks
    (and every decoding request served while budget and max_bs allow), out_len tokens per request,
    reservations within the slots, FCFS admission."""
    budget, chunk, max_bs, n_slots = [(16, 8, 4, 300), (64, 16, 8, 800), (7, 3, 3, 120), (128, 128, 16, 2000),
                                      (5, 5, 2, 100), (33, 10, 6, 400)][seed]
    reqs = poisson_trace(seed=100 + seed, n=150, rate=[0.5, 1.0, 0.3, 2.0, 0.2, 0.8][seed], plo=1, phi=60, olo=1,
                         ohi=25, reserve_out=25)
    log = S.replay(reqs, max_bs, n_slots, budget=budget, chunk=chunk)
    by = {r.rid: r for r in reqs}
    fed = {r.rid: 0 for r in reqs}            # prompt tokens fed so far
    made = {r.rid: 0 for r in reqs}           # tokens yielded
    admitted = []
    live = set()
    for t, work, n_rsrv in log:
        assert sum(n for _, n, _ in work) <= budget and len(work) <= max_bs and n_rsrv <= n_slots
        seen_prefill = False
        for rid, n, c in work:
            plen = len(by[rid].prompt)
            if c < plen:                                          # a prompt chunk
                seen_prefill = True
                assert c == fed[rid] and 1 <= n <= chunk and c + n <= plen
                if c == 0:
                    admitted.append(rid)
                fed[rid] += n
                if fed[rid] == plen:
                    made[rid] += 1
            else:                                                 # a decode
                assert not seen_prefill and n == 1 and fed[rid] == plen
                assert c == plen + made[rid] - 1
                made[rid] += 1
            live.add(rid)
        decoding = {rid for rid in live if fed[rid] == len(by[rid].prompt) and made[rid] < by[rid].out_len}
        in_batch = {rid for rid, _, _ in work}
        if seen_prefill:                      # prompt chunks only after every eligible decode
            assert (decoding - in_batch) == set() or len(work) == max_bs
        live = {rid for rid in live if made[rid] < by[rid].out_len}
    assert all(made[r.rid] == r.out_len and fed[r.rid] == len(r.prompt) for r in reqs)
    order = sorted(reqs, key=lambda r: (r.arrival, r.rid))
    assert admitted == [r.rid for r in order]


# ---------------------------------------------------------------- reservation policies / K/V usage
def test_reservation_policy_closed_forms():
    """Lecture section 6.1: Max reserves the longest output, Pow2 rounds the output up to a power of two
    (an output of 25 reserves 32 positions), Oracle exactly the tokens that get K/V."""
    assert S.reservation("max", 10, 25, 512) == 10 + 512
    assert S.reservation("pow2", 10, 25, 512) == 10 + 32
    assert [S.reservation("pow2", 0, n, 512) for n in (1, 2, 3, 32, 33, 512)] == [1, 2, 4, 32, 64, 512]
    assert S.reservation("oracle", 10, 25, 512) == 10 + 25 - 1
    for p, n in ((1, 1), (7, 300), (512, 512)):
        assert S.reservation("oracle", p, n, 512) <= S.reservation("pow2", p, n, 512) <= S.reservation("max", p, n, 512)
        assert S.reservation("pow2", p, n, 512) - p < 2 * n


def test_kv_usage_hand_worked():
    """One request, prompt 3, out 2, Oracle reservation 4 of 10 slots: iteration 0 prefills (3 tokens
    stored), iteration 1 decodes (4 stored) and finishes: reserved 0.4, stored (3 + 4) / 2 / 10 = 0.35."""
    class R:
        rid, arrival, prompt, out_len, max_tokens = 0, 0.0, [1, 2, 3], 2, 4
    log = S.replay([R()], 1, 10)
    res, st, per = S.kv_usage(log, [R()], 10)
    assert per == [3, 4] and res == pytest.approx(0.4) and st == pytest.approx(0.35)


@pytest.mark.parametrize("policy", S.POLICIES)
def test_kv_usage_invariants(policy):
    """Stored never exceeds reserved; under Oracle a request's stored K/V reaches its reservation exactly
    on its last iteration; tighter policies finish the same work in no more iterations here."""
    reqs = poisson_trace(seed=5, n=300, rate=1.0, plo=1, phi=60, olo=1, ohi=60, reserve_out=60)
    for r in reqs:
        r.max_tokens = S.reservation(policy, len(r.prompt), r.out_len, 60)
    log = S.replay(reqs, 16, 800)
    res, st, per = S.kv_usage(log, reqs, 800)
    assert all(s_ <= n_rsrv for s_, (_, _, n_rsrv) in zip(per, log)) and st <= res <= 1.0
    if policy == "oracle":
        last = {}
        for t, work, _ in log:
            for rid, n, c in work:
                last[rid] = c + n
        assert all(last[r.rid] == r.max_tokens for r in reqs)


# ---------------------------------------------------------------- request-level (static) batching
def test_static_batching_timeline_exact():
    """The lecture's static grid: same six requests, max_bs 3, whole batches: 18 iterations, every row."""
    g = load("p4_static_timeline.txt")
    reqs = p4_grid_requests(seed=0)
    log = S.replay(reqs, max_bs=3, n_slots=10**9, static=True)
    assert len(log) == g["iterations"][0] == load("p4_timeline.txt")["static_iterations"][0]
    rows = S.timeline_static(log, reqs)
    for r in reqs:
        assert rows[r.rid] == g[f"r{r.rid}"], (r.rid, rows[r.rid])


@pytest.mark.parametrize("seed", range(4))
def test_static_batching_invariants(seed):
    """Batches are disjoint, start only when the previous one is done, take waiting requests in arrival
    order, never admit a request mid-batch; every request still gets out_len tokens; max_bs = 1 is the
    same as iteration-level scheduling."""
    reqs = poisson_trace(seed=40 + seed, n=120, rate=[0.3, 1.0, 3.0, 0.5][seed], plo=1, phi=30, olo=1, ohi=20,
                         reserve_out=20)
    log = S.replay(reqs, 8, 400, static=True)
    seen = set()
    current = set()
    for t, work, _ in log:
        ids = {rid for rid, _, _ in work}
        if all(c == 0 for _, _, c in work):            # a new batch: the previous one has finished
            assert not (ids & seen)
            current = set(ids)
            seen |= ids
        else:
            assert ids <= current and all(c > 0 for _, _, c in work)
    n_tok = {}
    for _, work, _ in log:
        for rid, _, _ in work:
            n_tok[rid] = n_tok.get(rid, 0) + 1
    assert all(n_tok[r.rid] == r.out_len for r in reqs)
    assert S.replay(reqs, 1, 400, static=True) == S.replay(reqs, 1, 400)
