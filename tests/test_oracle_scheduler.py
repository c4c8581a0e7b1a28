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
