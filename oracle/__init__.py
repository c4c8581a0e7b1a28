"""Plain, slow CPU oracle of one selective-batched iteration and its scheduler.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the package
``selective_batching_amd``) may import, call, link or execute this package.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP path; both draw their
inputs from the data-only ``synth`` package.

What it computes (fp64 numpy unless stated):

* ``scheduler`` -- iteration-level FCFS ``Select`` with K/V-slot reservation
  and the iteration loop around it, written from Algorithm 1 of the
  "连续批处理完全拆解" walk-through (sections 迭代级 FCFS and 两个约束) and the
  scheduling section (4.3) of "CS349D Lecture 2 · 批处理与调度".
* ``model`` -- the plain per-request Transformer: each request alone, with the
  K/V history its earlier iterations produced.  Selective batching must reach
  exactly this result (up to rounding order): batching only changes when a
  token is computed, not what is computed ("CS349D Lecture 2", section 4.1 and
  common pitfall 3).
* ``flat`` -- the method itself in numpy: token-wise operators on the
  flattened ``[sum L_i, H]`` tensor, Split by request offsets before attention
  and Merge after it ("连续批处理完全拆解", Figure 5 walk-through).  Used as a
  self-check against ``model``.
* ``brute`` -- attention by explicit Python loops with ``math.exp`` for tiny
  inputs (textbook scaled-dot-product attention with a causal mask).
* ``generate`` -- greedy generation one request at a time and under the
  continuous-batching loop.
* ``precision`` -- optional storage-precision mode: the tensors handed from
  one operator to the next are rounded to the model dtype (the pages fix no
  precision; this is the reading the bf16 configurations are checked under,
  next to the exact fp64 oracle).

Pins (tests marked ``not gpu``) tie each part to facts the pages fix: the
lecture's continuous-batching timeline, the Figure-3 and Figure-5 counts, the
exercise-4 token and (query, key)-pair counts, closed forms of the scalar
functions, brute-force attention, and the continuous == one-at-a-time
invariant.  Every function here has such a pin.  The pages also print two
measurements of the lecture's own program (a largest logit difference of
1.1e-6 between batched and one-at-a-time computation, and 4.88x fewer weight
bytes read); no function here computes either figure -- they depend on that
program's model and byte accounting, which the pages do not give.  The
property behind the first (batched equals one-at-a-time up to rounding) is
pinned by the flat == per-request and continuous == one-at-a-time tests.
"""
from . import scheduler, model, flat, brute, generate, precision  # noqa: F401
