"""CPU oracle for the triggered (gated) chunked all-gather.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or runs
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP path (``triggered_copy_amd``) and imports nothing from it.

It is a plain, slow, sequential restatement of what the method computes, in
the notation of the pages it follows:

* "Triggered Plans" (Iris documentation): sections *Model*, *The kernel
  author's contract*, *Memory ordering*, *Gates and rounds*, *Requirements and
  limits*.
* "Triggered SDMA Plans" (Iris pull request): sections *API* and
  *Design notes* (the schedule-per-rank constructor, the poll -> copy -> atomic
  chain on one in-order queue per peer).
* "Barrier: Signals Only" (pypto documentation): sections *The idea*,
  *Walkthrough*, *Edge cases* (the dedicated-row notify/wait barrier).

Modules
-------
``values``    seeded value hash the synthetic producers write (SplitMix64 mix).
``cvalues``   the same hash in plain C (``values.c``), for full-size checks.
``schedule``  views -> regions -> chunks; ``whole``/``chunks``/``tile_chunks``;
              grouped step->tile order; plan-creation validation.
``plan``      the step-by-step simulation of gates, in-order queues and rounds.
``barrier``   the notify/wait dedicated-row barrier, sequentially.
``gemm``      the fp32-accumulated reference for the GEMM producer.
``consumer``  which chunks a consumer of the gathered rows waits for.

Every function's pin (the independent fact that checks it) lives in
``tests/test_oracle_pins.py``.  Parts with no such pin say "parity unpinned".
"""

from . import values, schedule, plan, barrier, gemm, consumer  # noqa: F401
