"""Iteration-level scheduling: Algorithm 1 ``Select`` and the loop around it.

Sources: "连续批处理完全拆解" (Algorithm 1 and the notes after it, sections
迭代级 FCFS / 两个约束), "CS349D Lecture 2 · 批处理与调度" (section 4.1 timeline,
section 4.3 scheduling algorithm, exercise 1), and the ``select_batch`` of
"Orca: The beginning of Morden LLM serving" (section Scheduling Algorithm).

Readings taken where the pages are garbled or silent:
  * every non-RUNNING request that passes the checks joins the batch, in both
    phases; only a request in the INITIATION phase reserves slots;
  * the reservation check breaks when ``n_rsrv + max_tokens > n_slots``, so an
    exact fit is admitted; a failed check stops the scan (never skips);
  * equal arrival times are ordered by submission order;
  * a request is finished once it has generated ``out_len`` tokens; its
    ``max_tokens`` slots return to the pool after that iteration;
  * a request whose ``max_tokens`` exceeds ``n_slots`` can never be admitted
    and is rejected when it is submitted;
  * one worker (one batch in flight), so no request is RUNNING when Select runs.

Chunked prefill ("从静态批处理到连续批处理", section Chunked Prefill; "CS349D
Lecture 2", exercise 9): with a per-iteration token budget, long prompts are fed
in chunks, SeqWork(n_new = chunk, n_past = prompt tokens already processed).
The pages fix the idea but not every rule; the reading taken here:
  * decodes first: every request past its prompt takes one token, in arrival
    order, while the budget and max_bs allow;
  * then requests still in their prompt, in arrival order, each take
    min(chunk, prompt tokens left, budget left) tokens; the first scheduling
    reserves max_tokens as in Algorithm 1 and a failed reservation stops the
    scan; an exhausted budget or max_bs stops it too;
  * only the chunk that completes a prompt yields a token (the first one).
With an unlimited budget and chunk this is Algorithm 1 itself (with one worker
every decoding request arrived before every waiting one).

Request-level (static) batching, the baseline the pages compare against ("CS349D
Lecture 2", section 4.1, the static grid; "从静态批处理到连续批处理", 静态批处理的
困境): a batch starts only when the previous one has entirely finished, takes up
to max_bs waiting requests in arrival order (reserving as above), and runs until
its longest member is done; nobody joins mid-batch.  On ragged kernels a finished
member needs no padding work: it leaves the computed batch but its seat stays
empty until the batch ends (reading taken here: its compute is not charged).
"""
import math

INITIATION = "INITIATION"
RUNNING = "RUNNING"
INCREMENT = "INCREMENT"


class TooLarge(ValueError):
    """max_tokens exceeds the K/V slot pool: the request could never be admitted."""


class SReq:
    """Scheduler view of a request."""

    __slots__ = ("rid", "arrival", "order", "prompt_len", "out_len", "max_tokens", "state", "generated", "prefilled",
                 "cur_new")

    def __init__(self, rid, arrival, order, prompt_len, out_len, max_tokens):
        self.rid = rid
        self.arrival = arrival
        self.order = order
        self.prompt_len = prompt_len
        self.out_len = out_len
        self.max_tokens = max_tokens
        self.state = INITIATION
        self.generated = 0
        self.prefilled = 0      # prompt tokens already processed (their K/V cached)
        self.cur_new = 0        # tokens fed in the current iteration


def select(pool, n_rsrv, max_bs, n_slots):
    """Algorithm 1 ``Select``: returns (batch, n_rsrv).

    Scan the requests that are not RUNNING in arrival order; stop at ``max_bs``;
    a request that has never been scheduled must first fit its ``max_tokens``
    into the remaining slots, otherwise the scan stops there.
    """
    batch = []
    candidates = sorted((r for r in pool if r.state != RUNNING), key=lambda r: (r.arrival, r.order))
    for r in candidates:
        if len(batch) == max_bs:
            break
        if r.state == INITIATION:
            wanted = n_rsrv + r.max_tokens
            if wanted > n_slots:
                break
            n_rsrv = wanted
        batch.append(r)
    return batch, n_rsrv


def select_chunked(pool, n_rsrv, max_bs, n_slots, budget, chunk):
    """``Select`` with a token budget and prompts fed in chunks: returns (batch of (request, n_new), n_rsrv)."""
    cand = sorted((r for r in pool if r.state != RUNNING), key=lambda r: (r.arrival, r.order))
    batch, left = [], budget
    for r in cand:                                   # decodes first, one token each
        if r.prefilled < r.prompt_len:
            continue
        if len(batch) == max_bs or left == 0:
            break
        batch.append((r, 1))
        left -= 1
    for r in cand:                                   # then prompt chunks, arrival order
        if r.prefilled == r.prompt_len:
            continue
        if len(batch) == max_bs or left == 0:
            break
        if r.state == INITIATION:
            if n_rsrv + r.max_tokens > n_slots:
                break
            n_rsrv += r.max_tokens
        n = min(chunk, r.prompt_len - r.prefilled, left)
        batch.append((r, n))
        left -= n
    return batch, n_rsrv


def work_of(r):
    """(n_new, ctx) a batch member processes this iteration.

    A request that has not run yet feeds its whole prompt with nothing cached;
    afterwards it feeds its last generated token, with the prompt and all but
    that token already cached.
    """
    if r.generated == 0:
        return r.prompt_len, 0
    return 1, r.prompt_len + r.generated - 1


class Scheduler:
    """Pool, counters and the per-iteration state transitions (one worker)."""

    def __init__(self, max_bs, n_slots, budget=None, chunk=None, static=False):
        if max_bs <= 0:
            raise ValueError("max_bs must be positive")
        if (budget is None) != (chunk is None) or (budget is not None and (budget < 1 or chunk < 1)):
            raise ValueError("budget and chunk: both positive, or both None")
        self.max_bs = max_bs
        self.n_slots = n_slots
        self.budget, self.chunk = budget, chunk
        if static and budget is not None:
            raise ValueError("request-level batching feeds whole prompts")
        self.static = static
        self.seated = []                 # request-level batching: the running batch's unfinished members
        self.n_rsrv = 0
        self.pool = []
        self._order = 0

    def add(self, rid, arrival, prompt_len, out_len, max_tokens):
        if max_tokens > self.n_slots:
            raise TooLarge(f"request {rid}: max_tokens {max_tokens} > n_slots {self.n_slots}")
        if prompt_len < 1 or out_len < 1 or prompt_len + out_len - 1 > max_tokens:
            raise ValueError(f"request {rid}: inconsistent lengths")
        r = SReq(rid, arrival, self._order, prompt_len, out_len, max_tokens)
        self._order += 1
        self.pool.append(r)
        return r

    def select(self):
        if self.static:
            if not self.seated:          # the previous batch has entirely finished: form a new one
                self.seated, self.n_rsrv = select(self.pool, self.n_rsrv, self.max_bs, self.n_slots)
            batch = list(self.seated)
            for r in batch:
                r.cur_new = work_of(r)[0]
        elif self.budget is None:
            batch, self.n_rsrv = select(self.pool, self.n_rsrv, self.max_bs, self.n_slots)
            for r in batch:
                r.cur_new = work_of(r)[0]
        else:
            chosen, self.n_rsrv = select_chunked(self.pool, self.n_rsrv, self.max_bs, self.n_slots, self.budget,
                                                 self.chunk)
            batch = []
            for r, n in chosen:
                r.cur_new = n
                batch.append(r)
        for r in batch:
            r.state = RUNNING
        return batch

    def work(self, r):
        """(n_new, ctx) of a member this iteration."""
        if self.budget is None:
            return work_of(r)
        if r.prefilled < r.prompt_len:
            return r.cur_new, r.prefilled
        return 1, r.prompt_len + r.generated - 1

    def complete(self, batch):
        """Every member that finished its prompt or decoded yields one token: move to INCREMENT, retire
        finished ones."""
        finished = []
        for r in batch:
            r.state = INCREMENT
            if r.prefilled < r.prompt_len:
                r.prefilled = r.prompt_len if self.budget is None else r.prefilled + r.cur_new
                if r.prefilled < r.prompt_len:
                    continue                       # a prompt chunk that does not end the prompt: no token
            r.generated += 1
            if r.generated == r.out_len:
                self.n_rsrv -= r.max_tokens
                finished.append(r)
        if finished:
            gone = {id(r) for r in finished}
            self.pool = [r for r in self.pool if id(r) not in gone]
            self.seated = [r for r in self.seated if id(r) not in gone]
        return finished


def replay(reqs, max_bs, n_slots, engine=None, budget=None, chunk=None, static=False):
    """Run the iteration loop on a logical clock t = 0, 1, 2, ...

    ``reqs``: objects with ``rid, arrival, prompt (or prompt_len), out_len,
    max_tokens``.  A request may join from iteration t on when its arrival is
    ``<= t``; when the pool is empty the clock jumps to the next arrival.
    ``engine(t, batch_work)`` -- if given -- is called with the list of
    ``(rid, n_new, ctx)`` of the iteration, in batch order.

    ``budget``/``chunk``: chunked prefill (module docstring); a member yields a token iff
    ``ctx + n_new >= prompt length``.

    Returns the per-iteration log ``[(t, [(rid, n_new, ctx), ...], n_rsrv_after_select)]``.
    """
    s = Scheduler(max_bs, n_slots, budget, chunk, static)
    pending = sorted(reqs, key=lambda r: (r.arrival, r.rid))
    i = 0
    t = 0
    log = []
    while i < len(pending) or s.pool:
        while i < len(pending) and pending[i].arrival <= t:
            r = pending[i]
            plen = len(r.prompt) if hasattr(r, "prompt") else r.prompt_len
            s.add(r.rid, r.arrival, plen, r.out_len, r.max_tokens)
            i += 1
        if not s.pool:
            t = int(math.ceil(pending[i].arrival))
            continue
        batch = s.select()
        if not batch:
            raise RuntimeError("non-empty pool produced an empty batch")
        work = [(r.rid, *s.work(r)) for r in batch]
        log.append((t, work, s.n_rsrv))
        if engine is not None:
            engine(t, work)
        s.complete(batch)
        t += 1
    return log


# ---------------------------------------------------------------- reservation policies
# "CS349D Lecture 2", section 6.1 (KV 预留：被占着 ≠ 被用着): Orca reserves a request's K/V slots when it is
# first scheduled; how many is a policy.  Readings: Max = the prompt plus the longest output allowed;
# Pow2 = the prompt plus the output length rounded up to a power of two (a length prediction that
# over-reserves by at most 2x); Oracle = exactly the tokens that ever get K/V: prompt + out_len - 1
# (the last generated token is never fed back).
POLICIES = ("max", "pow2", "oracle")


def reservation(policy, prompt_len, out_len, max_out):
    """max_tokens a request reserves under ``policy``."""
    if policy == "max":
        return prompt_len + max_out
    if policy == "pow2":
        p = 1
        while p < out_len:
            p *= 2
        return prompt_len + p
    if policy == "oracle":
        return prompt_len + out_len - 1
    raise ValueError(policy)


def kv_usage(log, reqs, n_slots):
    """Time-weighted K/V occupancy of a replay on the iteration clock (lecture section 6.1's two columns):
    'reserved' = slots reserved while the iteration runs (n_rsrv after Select), 'stored' = slots holding
    K/V at the end of the iteration (every token fed so far by a request that holds its reservation during
    that iteration).  Each iteration weighs one time unit.  Returns (reserved, stored) as fractions of
    ``n_slots`` and the per-iteration stored counts."""
    plen = {r.rid: (len(r.prompt) if hasattr(r, "prompt") else r.prompt_len) for r in reqs}
    out_len = {r.rid: r.out_len for r in reqs}
    fed, made, stored_t = {}, {}, []
    res_sum = st_sum = 0
    for t, work, n_rsrv in log:
        for rid, n_new, ctx in work:
            fed[rid] = ctx + n_new                      # K/V of every token fed so far
        stored = sum(fed.values())
        stored_t.append(stored)
        res_sum += n_rsrv
        st_sum += stored
        for rid, n_new, ctx in work:                    # a member yields a token iff its work passes its prompt
            if ctx + n_new >= plen[rid]:
                made[rid] = made.get(rid, 0) + 1
                if made[rid] == out_len[rid]:
                    del fed[rid]                        # finished: its slots are freed after this iteration
    n = max(len(log), 1)
    return res_sum / n / n_slots, st_sum / n / n_slots, stored_t


def timeline_static(log, reqs):
    """As ``timeline`` for a request-level replay, with '-' for a seat its finished request still holds
    until the rest of its batch is done."""
    rows = timeline(log, reqs)
    n_it = log[-1][0] + 1 if log else 0
    grid = {rid: list(row.ljust(n_it)) for rid, row in rows.items()}
    # batches: maximal runs of iterations whose members are a subset of the first iteration's (all prefill)
    starts = [i for i, (_, work, _) in enumerate(log) if all(ctx == 0 for _, _, ctx in work)]
    for b, i0 in enumerate(starts):
        i1 = starts[b + 1] if b + 1 < len(starts) else len(log)
        t_end = log[i1 - 1][0]
        for rid, _, _ in log[i0][1]:
            last = max(t for t, work, _ in log[i0:i1] if any(w[0] == rid for w in work))
            for t in range(last + 1, t_end + 1):
                grid[rid][t] = "-"
    return {rid: "".join(v).rstrip() for rid, v in grid.items()}


def timeline(log, reqs):
    """Render a replay log as one row of P/D/wait marks per request (lecture section 4.1 style).

    'P' = prefill this iteration, 'D' = decode, '·' = arrived and waiting,
    ' ' = not arrived yet or already finished.
    """
    n_it = log[-1][0] + 1 if log else 0
    rows = {r.rid: [" "] * n_it for r in reqs}
    last = {}
    for t, work, _ in log:
        for rid, n_new, ctx in work:
            rows[rid][t] = "P" if ctx == 0 and _is_first(rid, t, log) else "D"
            last[rid] = t
    for r in reqs:
        for t in range(n_it):
            if rows[r.rid][t] == " " and r.arrival <= t and t < last.get(r.rid, n_it):
                rows[r.rid][t] = "·"
    return {rid: "".join(v).rstrip() for rid, v in rows.items()}


def _is_first(rid, t, log):
    for tt, work, _ in log:
        for w in work:
            if w[0] == rid:
                return tt == t
    return False
