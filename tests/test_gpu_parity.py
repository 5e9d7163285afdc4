"""GPU parity: the HIP path against the CPU oracle, element by element.

Bit-exact replicas, gate tables and queue cursors after every round, on the
small workloads (several tiles, ragged tails, unaligned pitches) and on the
two-rank bf16 workload at its full size; the barrier against its closed form
and reveal; the misuse paths (extra mark, withheld mark, round limit, state
order).  Every call goes through the C boundary.
"""

import numpy as np
import pytest
import torch

import triggered_copy_amd as tc
from oracle import barrier as obarrier
from oracle import plan as oplan
from synth import BASE_SEED, workloads
from tests.gpu_common import Pair, log, require_gpu, wait_until

pytestmark = pytest.mark.gpu


def _run_all_rounds(name, w):
    pair = Pair(w)
    try:
        for r in range(1, w["rounds"] + 1):
            log(f"{name} round {r}")
            if w.get("shuffled"):
                orders, dev = pair.orders_device(r)
                pair.gpu_round_fill(serial=True, order=dev, order_stride=orders.shape[1])
                mark_order = [(p, int(c)) for p in range(pair.P) for c in orders[p]
                              for _ in range(pair.sim.writers(p, int(c)))]
                pair.oracle_round(mark_order=mark_order)
            else:
                pair.gpu_round_fill()
                pair.oracle_round()
            pair.compare(f"{name} round {r}")
            assert pair.plan.state == "DONE"
            pair.plan.next_round()
            pair.sim.next_round()
    finally:
        pair.close()


@pytest.mark.parametrize("name", sorted(workloads.SMALL))
def test_small_workload_rounds(name):
    _run_all_rounds(name, workloads.SMALL[name])


def test_bf16_chunks_p2_full():
    _run_all_rounds("bf16_chunks_p2", workloads.FULL["bf16_chunks_p2"])


def test_deferred_marks_and_ctas_sweep():
    w = dict(workloads.SMALL["u32_chunks_ragged_p3"])
    for ctas, piece in ((1, 256), (3, 512), (64, 0)):
        pair = Pair(w, engine_ctas=ctas, piece_bytes=piece)
        try:
            for r in (1, 2):
                log(f"deferred ctas={ctas} piece={piece} round {r}")
                pair.gpu_round_fill(mark=False)
                pair.oracle_round()
                pair.compare(f"deferred ctas={ctas} round {r}")
                pair.plan.next_round()
                pair.sim.next_round()
        finally:
            pair.close()


def test_waves_fill():
    # A persistent producer grid completing every rank's chunk 0, then every
    # rank's chunk 1, ...: grids smaller and larger than the slot count.
    w = dict(workloads.SMALL["u32_chunks_ragged_p3"])
    for ctas in (1, 4, 0):
        pair = Pair(w)
        try:
            for r in (1, 2):
                log(f"waves fill ctas={ctas} round {r}")
                pair.gpu_round_fill(waves=True, ctas=ctas)
                pair.oracle_round()
                pair.compare(f"waves ctas={ctas} round {r}")
                pair.plan.next_round()
                pair.sim.next_round()
        finally:
            pair.close()


ONESHOT_CASES = {
    # blocks per share from one to several, ragged tails
    "u32_chunks_ragged_p3": dict(workloads.SMALL["u32_chunks_ragged_p3"]),
    "u32_chunks_multi_block_p4": dict(P=4, rows=300, cols=1000, elem="u32", builder="chunks", n=3,
                                      writers=5),
    "u32_whole_p5": dict(workloads.SMALL["u32_whole_p5"]),
    # shares that start and end off 16-byte boundaries: the byte path
    "u8_chunks_unaligned_p3": dict(P=3, rows=301, cols=101, elem="u8", builder="chunks", n=4,
                                   writers=3),
    "bf16_whole_odd_p2": dict(P=2, rows=7, cols=4097, elem="bf16", builder="whole", writers=7),
    # more writers than pieces: empty shares still mark
    "u32_whole_many_writers_p2": dict(P=2, rows=1, cols=3000, elem="u32", builder="whole",
                                      writers=9),
}


@pytest.mark.parametrize("fill", ["oneshot", "writer_ctas"])
@pytest.mark.parametrize("name", sorted(ONESHOT_CASES))
def test_range_share_fills(name, fill):
    # Every chunk one byte range in a contiguous view.  oneshot: one CTA per
    # 16 KiB block of each writer's share, the share's last block to finish
    # marks.  writer_ctas: one CTA per writer, which then writes its share
    # through to memory and marks without an L2 write-back.  Shares that
    # start and end off 16-byte boundaries take the byte path.  Rounds
    # alternate in-kernel and deferred marks, so a deferred round must leave
    # the block counters as it found them.
    w = ONESHOT_CASES[name]
    pair = Pair(w, piece_bytes=4096)
    try:
        for r, mark in ((1, True), (2, False), (3, True), (4, True)):
            log(f"{fill} {name} round {r} mark={mark}")
            pair.gpu_round_fill(mark=mark, oneshot=fill == "oneshot")
            pair.oracle_round()
            pair.compare(f"{fill} {name} round {r}")
            pair.plan.next_round()
            pair.sim.next_round()
    finally:
        pair.close()


def test_oneshot_fill_rejects_tiles_and_strided_views():
    for name in ("bf16_tiles_ragged_p4", "u8_tiles_odd_p2"):
        pair = Pair(dict(workloads.SMALL[name]))
        try:
            h = pair.plan.start(pair.stream)
            with pytest.raises(tc.InvalidArgument, match="one byte range"):
                pair.plan.fill(h, pair.tv, pair.seed, kind=pair.w["elem"], oneshot=True,
                               stream=pair.stream)
            pair.plan.fill(h, pair.tv, pair.seed, kind=pair.w["elem"], stream=pair.stream)
            pair.plan.wait(10.0)
        finally:
            pair.close()
    # Byte-range chunks over a view read with a row stride the plan was not
    # cut for: the fill's contiguity check refuses it before any launch.
    w = dict(workloads.SMALL["u32_chunks_ragged_p3"])
    pair = Pair(w)
    try:
        h = pair.plan.start(pair.stream)
        strided = [tc.View(v.byte_offset, v.rows // 2, v.cols // 2, v.cols, v.elem_bytes, 0)
                   for v in pair.tv]
        with pytest.raises(tc.InvalidArgument, match="contiguous views"):
            pair.plan.fill(h, strided, pair.seed, kind=w["elem"], oneshot=True, stream=pair.stream)
        pair.plan.fill(h, pair.tv, pair.seed, kind=w["elem"], oneshot=True, stream=pair.stream)
        pair.plan.wait(10.0)
        pair.oracle_round()
        pair.compare("oneshot after a refused call")
    finally:
        pair.close()


def _expected_replicas(pair, r):
    """Every replica after round r delivered in full (oracle)."""
    pair.oracle_round()
    return [rep.copy() for rep in pair.sim.rep]


def test_close_mid_round_sends_chunks_as_they_stand():
    w = dict(workloads.SMALL["u32_chunks_ragged_p3"])
    pair = Pair(w)
    try:
        h = pair.plan.start(pair.stream)
        # data written, only rank 0's chunks marked: the others' gates stay shut
        pair.plan.fill(h, pair.tv, pair.seed, kind="u32", mark=False, stream=pair.stream)
        for c in range(5):
            pair.plan.mark(h, 0, c, 2, stream=pair.stream)
        pair.stream.synchronize()
        assert pair.plan.close() == "CLOSED"
        want = _expected_replicas(pair, 1)
        host = pair.rep.cpu().numpy()
        for q in range(pair.P):
            assert np.array_equal(host[q], want[q]), f"replica {q} after close"
    finally:
        pair.close()


def test_close_after_timeout_sends_chunks_as_they_stand():
    w = dict(workloads.SMALL["u32_whole_p5"])
    pair = Pair(w)
    try:
        h = pair.plan.start(pair.stream)
        pair.plan.fill(h, pair.tv, pair.seed, kind="u32", mark=False, stream=pair.stream)
        with pytest.raises(tc.PlanTimeout):
            pair.plan.wait(0.2)            # the engine is stopped
        pair.stream.synchronize()
        assert pair.plan.close() == "CLOSED"
        want = _expected_replicas(pair, 1)
        host = pair.rep.cpu().numpy()
        for q in range(pair.P):
            assert np.array_equal(host[q], want[q]), f"replica {q} after close"
    finally:
        pair.close()


def test_plan_queued_behind_another_is_closing():
    # Two plans over the same buffers (row blocks, and the whole block) share
    # the engine stream: B's round is queued behind A's, whose gates stay
    # shut.  B's close() returns CLOSING; closing A sends A's chunks as they
    # stand and lets B's engine run; B's second close() frees it.
    w = dict(P=3, rows=24, cols=40, elem="u32", builder="chunks", n=3, writers=1, rounds=1)
    pair = Pair(w)
    b = tc.TriggeredPlan(pair.rep, [tc.whole(v, 1) for v in pair.tv], backstop_s=20.0)
    try:
        ha = pair.plan.start(pair.stream)
        hb = b.start(pair.stream)
        pair.plan.fill(ha, pair.tv, pair.seed, kind="u32", mark=False, stream=pair.stream)
        pair.stream.synchronize()
        assert b.close() == "CLOSING"
        assert b.state == "CLOSING"
        assert pair.plan.close() == "CLOSED"
        # B's engine starts once A's has left the stream
        assert wait_until(lambda: b.close() == "CLOSED", 5.0)
        want = _expected_replicas(pair, 1)
        host = pair.rep.cpu().numpy()
        for q in range(pair.P):
            assert np.array_equal(host[q], want[q]), f"replica {q} after closing both"
        del hb
    finally:
        b.close()
        pair.close()


@pytest.mark.parametrize("rounds_before", [0, 1])
def test_close_before_start_sends_chunks_as_they_stand(rounds_before):
    # [TP] The kernel author's contract: closing a plan before its round
    # starts still sends each rank's chunks as they stand.  The producer
    # writes the round's data into a READY plan (no start, no marks); close()
    # must deliver it everywhere, as a full round of the oracle does.
    w = dict(workloads.SMALL["u32_chunks_ragged_p3"])
    pair = Pair(w)
    try:
        for r in range(1, rounds_before + 1):
            pair.gpu_round_fill()
            pair.oracle_round()
            pair.compare(f"close-before-start warm-up round {r}")
            pair.plan.next_round()
            pair.sim.next_round()
        h = pair.plan.current_handle()
        pair.plan.fill(h, pair.tv, pair.seed, kind="u32", mark=False, stream=pair.stream)
        pair.stream.synchronize()
        assert pair.plan.state == "READY"
        log(f"close before start, round {rounds_before + 1}")
        assert pair.plan.close() == "CLOSED"
        want = _expected_replicas(pair, rounds_before + 1)
        host = pair.rep.cpu().numpy()
        for q in range(pair.P):
            assert np.array_equal(host[q], want[q]), f"replica {q} after close before start"
    finally:
        pair.close()


def test_plan_behind_a_slow_unblocked_plan_closes_closed():
    # A's gates are all open but its engine is slow (one CTA, 256-byte
    # pieces); B's round is queued behind it on the shared engine stream.
    # B is not behind *waiting* copies, so close() must wait for A's engine
    # and then free B (CLOSED, not CLOSING), with B's round delivered.
    wa = dict(P=2, rows=2048, cols=16384, elem="u32", builder="whole", writers=4, rounds=1)
    wb = dict(P=3, rows=24, cols=40, elem="u32", builder="chunks", n=3, writers=1, rounds=1)
    a = Pair(wa, oracle_bytes=False, engine_ctas=1, piece_bytes=256)
    b = Pair(wb, seed=BASE_SEED + 5)
    try:
        ha = a.plan.start(a.stream)
        a.plan.fill(ha, a.tv, a.seed, kind="u32", mark=True, stream=a.stream)
        hb = b.plan.start(a.stream)
        b.plan.fill(hb, b.tv, b.seed, kind="u32", mark=True, stream=a.stream)
        a.stream.synchronize()
        import time
        t0 = time.perf_counter()
        assert b.plan.close() == "CLOSED"
        log(f"close() behind a slow unblocked plan returned after {time.perf_counter() - t0:.3f} s")
        a.plan.wait(30.0)
        log(f"the slow plan's engine took {a.plan.stats()['engine_ms']:.1f} ms")
        a.oracle_round()
        a.compare("slow plan")
        want = _expected_replicas(b, 1)
        host = b.rep.cpu().numpy()
        for q in range(b.P):
            assert np.array_equal(host[q], want[q]), f"replica {q} of the closed plan"
    finally:
        b.close()
        a.close()


def test_wait_deadline_while_producer_runs_still_counts_its_marks():
    # wait() waits on the host for the producer's stream until its deadline;
    # past it, the completion check is queued behind the producer on the
    # device.  A deadline far shorter than a slow producer (one CTA writing
    # every rank's block), followed by an extra mark queued on the same
    # stream, must still report that mark (EEXTRA, plan FAILED): the check
    # runs only after the producer's work.  The engine is stopped from the
    # host at the deadline, so every kernel exits normally.
    w = dict(P=4, rows=1024, cols=16384, elem="u32", builder="chunks", n=4, writers=2, rounds=1)
    pair = Pair(w, oracle_bytes=False)
    try:
        h = pair.plan.start(pair.stream)
        pair.plan.fill(h, pair.tv, pair.seed, kind="u32", waves=True, ctas=1, stream=pair.stream)
        pair.plan.mark(h, 2, 1, 1, stream=pair.stream)
        with pytest.raises(tc.ExtraMarksError) as ei:
            pair.plan.wait(0.001)
        assert ei.value.chunks == [(2, 1)]
        assert pair.plan.state == "FAILED"
        pair.stream.synchronize()
        with pytest.raises(oplan.PlanError) as eo:
            pair.oracle_round(extra=[(2, 1)])
        assert eo.value.chunks == [(2, 1)]
    finally:
        pair.close()


def test_nested_plans_in_with_blocks():
    # Two plans as nested context managers over separate buffers ([TP]
    # Model: a plan is a context manager; leaving the block closes it).  A
    # round of each runs inside the inner block, the outer plan runs a second
    # round after the inner one has closed, and both match their oracles.
    wa = dict(P=3, rows=24, cols=40, elem="u32", builder="chunks", n=3, writers=2, rounds=2)
    wb = dict(P=2, rows=16, cols=64, elem="bf16", builder="whole", writers=3, rounds=1)
    a, b = Pair(wa), Pair(wb, seed=BASE_SEED + 1)
    a.plan.close()
    b.plan.close()
    with tc.TriggeredPlan(a.rep, a.ts, backstop_s=20.0) as pa:
        a.plan = pa
        with tc.TriggeredPlan(b.rep, b.ts, backstop_s=20.0) as pb:
            b.plan = pb
            for pair, name in ((a, "outer"), (b, "inner")):
                log(f"nested {name} round 1")
                pair.gpu_round_fill()
                pair.oracle_round()
                pair.compare(f"nested {name} round 1")
                pair.plan.next_round()
                pair.sim.next_round()
        assert pb.close() == "CLOSED"           # already closed by its block
        log("nested outer round 2")
        a.gpu_round_fill()
        a.oracle_round()
        a.compare("nested outer round 2")
    assert pa.close() == "CLOSED"


def _swap_in(pair, tsched, osched_list, **plan_kw):
    """Replace the Pair's plan and oracle with other schedules on the same buffers."""
    pair.plan.close()
    pair.plan = tc.TriggeredPlan(pair.rep, tsched, backstop_s=20.0, **plan_kw)
    pair.ts, pair.os = tsched, osched_list
    pair.sim = oplan.PlanSim(pair.sim.rep, osched_list)


def _rounds(pair, n, what, deferred=(), **fill_kw):
    """n rounds of fill, wait and oracle comparison; rounds listed in
    ``deferred`` fill without marks, then issue them with the mark kernel."""
    for r in range(1, n + 1):
        log(f"{what} round {r}")
        h = pair.plan.start(pair.stream)
        pair.plan.fill(h, pair.tv, pair.seed, kind=pair.w["elem"], mark=r not in deferred,
                       stream=pair.stream, **fill_kw)
        if r in deferred:
            pair.plan.mark_all(h, stream=pair.stream)
        pair.plan.wait(10.0)

        def produce(p, rr):
            if pair.os[p] is not None:
                from tests.gpu_common import oracle_produce_regions
                oracle_produce_regions(pair.sim.rep[p], pair.ov[p], pair.os[p], pair.w["elem"],
                                       pair.seed, p, rr)
        oplan.run_round(pair.sim, produce)
        pair.compare(f"{what} round {r}")
        pair.plan.next_round()
        pair.sim.next_round()


def test_broadcast_from_one_rank():
    # Only rank 0 sends (the others pass empty schedules): a broadcast.
    w = dict(P=4, rows=33, cols=50, elem="u32", builder="chunks", n=3, writers=2, rounds=2)
    pair = Pair(w)
    try:
        _swap_in(pair, [pair.ts[0], None, None, None], [pair.os[0], None, None, None])
        _rounds(pair, 2, "broadcast")
    finally:
        pair.close()


def test_hand_built_schedules():
    # Regions that cut tiles and regions that span several: part of a tile,
    # three tiles side by side as one 2-D window, a linear range across row
    # ends, all in one chunk table with 1-3 writers per chunk.
    from oracle import schedule as osched
    w = dict(P=3, rows=24, cols=40, elem="u8", builder="whole", writers=1, rounds=2)
    pair = Pair(w)
    try:
        rows, cols = w["rows"], w["cols"]
        ts, os_ = [], []
        for p in range(3):
            base = p * rows * cols
            regions = [
                (base + 2 * cols + 3, 5, 7, cols),          # 5 x 7 piece of a tile
                (base + 8 * cols, 4, 36, cols),             # 3 tiles of 12 columns side by side
                (base + 13 * cols + 30, 1, 25, 25),         # linear across a row end
                (base + 20 * cols, 4, cols, cols),          # whole rows: linear after normalising
            ]
            chunks = [(0, 1, 1), (1, 2, 3), (3, 1, 2)]
            ts.append(tc.from_arrays(chunks, regions))
            os_.append(osched.from_tables(chunks, regions))
        _swap_in(pair, ts, os_)
        _rounds(pair, 2, "hand-built")
    finally:
        pair.close()


def _random_tables(rng, base, rows, cols):
    """A random hand-built table over one rank's rows [base, base + rows*cols)
    of a u8 view: the rows cut into bands, each band one region (a 2-D window
    of some columns, or a linear range that may cross row ends), the regions
    shuffled and grouped into chunks of 1-3 regions with 1-3 writers."""
    cuts = sorted(rng.choice(np.arange(1, rows), size=min(rows - 1, int(rng.integers(1, 6))),
                             replace=False).tolist())
    regions = []
    for r0, r1 in zip([0] + cuts, cuts + [rows]):
        if rng.random() < 0.5:
            c0 = int(rng.integers(0, cols))
            width = int(rng.integers(1, cols - c0 + 1))
            if rng.random() < 0.5 and cols % 16 == 0:       # the engine's 16-byte vector path
                c0 = c0 // 16 * 16
                width = max(16, width // 16 * 16) if c0 + 16 <= cols else cols - c0
            regions.append((base + r0 * cols + c0, r1 - r0, width, cols))
        else:
            band = (r1 - r0) * cols
            a = int(rng.integers(0, band))
            regions.append((base + r0 * cols + a, 1, int(rng.integers(1, band - a + 1)), 0))
    regions = [regions[i] for i in rng.permutation(len(regions))]
    chunks, at = [], 0
    while at < len(regions):
        n = min(int(rng.integers(1, 4)), len(regions) - at)
        chunks.append((at, n, int(rng.integers(1, 4))))
        at += n
    return chunks, regions


@pytest.mark.parametrize("case", range(32))
def test_random_hand_built_tables(case):
    # Random region tables (unaligned 2-D windows, 16-byte aligned ones,
    # linear ranges across row ends), random chunking and writers, random
    # piece sizes and engine sizes: bit-exact with the oracle over 2 rounds.
    from oracle import schedule as osched
    rng = np.random.default_rng(1000 + case)
    P = int(rng.integers(2, 6))
    cols = int(rng.choice([16, 48, 64, int(rng.integers(5, 90))]))
    rows = int(rng.integers(3, 40))
    w = dict(P=P, rows=rows, cols=cols, elem="u8", builder="whole", writers=1, rounds=2)
    pair = Pair(w, seed=BASE_SEED + case)
    try:
        ts, os_ = [], []
        for p in range(P):
            if P > 2 and rng.random() < 0.15:           # a rank that sends nothing
                ts.append(None)
                os_.append(None)
                continue
            chunks, regions = _random_tables(rng, p * rows * cols, rows, cols)
            ts.append(tc.from_arrays(chunks, regions))
            os_.append(osched.from_tables(chunks, regions))
        kw = dict(piece_bytes=int(rng.choice([256, 512, 1024, 8192])),
                  engine_ctas=int(rng.integers(1, 9)))
        log(f"random tables case {case}: P={P} rows={rows} cols={cols} {kw}")
        _swap_in(pair, ts, os_, **kw)
        _rounds(pair, 2, f"random tables case {case}")
    finally:
        pair.close()


@pytest.mark.parametrize("case", range(16))
def test_random_byte_range_tables_range_fills(case):
    # Every rank's bytes cut at random points into linear regions, grouped
    # into chunks of 1-3 adjacent regions with 1-6 writers (more writers
    # than pieces leaves empty shares), random piece sizes: the one-shot
    # fill's share and block tables (even cases) or the write-through writer
    # CTAs (odd cases) against the oracle over 3 rounds, the second with
    # deferred marks.
    from oracle import schedule as osched
    rng = np.random.default_rng(3000 + case)
    P = int(rng.integers(2, 6))
    cols = int(rng.integers(700, 5000))
    rows = int(rng.integers(1, 60))
    w = dict(P=P, rows=rows, cols=cols, elem="u8", builder="whole", writers=1, rounds=3)
    pair = Pair(w, seed=BASE_SEED + 11 * case)
    try:
        ts, os_ = [], []
        n = rows * cols
        for p in range(P):
            cuts = sorted(set(rng.integers(1, n, size=int(rng.integers(0, 9))).tolist()))
            edges = [0] + cuts + [n]
            regions = [(p * n + a, 1, b - a, 0) for a, b in zip(edges[:-1], edges[1:])]
            chunks, at = [], 0
            while at < len(regions):
                k = min(int(rng.integers(1, 4)), len(regions) - at)
                chunks.append((at, k, int(rng.integers(1, 7))))
                at += k
            ts.append(tc.from_arrays(chunks, regions))
            os_.append(osched.from_tables(chunks, regions))
        kw = dict(piece_bytes=int(rng.choice([256, 4096, 8192, 65536])),
                  engine_ctas=int(rng.integers(1, 9)))
        log(f"random byte-range tables case {case}: P={P} bytes/rank={n} {kw}")
        _swap_in(pair, ts, os_, **kw)
        _rounds(pair, 3, f"random byte ranges case {case}", deferred=(2,), oneshot=case % 2 == 0)
    finally:
        pair.close()


def test_prepare_all_gather_default_whole():
    w = dict(P=3, rows=16, cols=64, elem="u32", builder="whole", writers=4, rounds=2)
    pair = Pair(w)
    try:
        pair.plan.close()
        pair.plan, views = tc.prepare_all_gather(pair.rep, w["rows"], w["cols"], 4, writers=4,
                                                 backstop_s=20.0)
        assert [v.byte_offset for v in views] == [t.byte_offset for t in pair.tv]
        _rounds(pair, 2, "prepare_all_gather")
        # a schedule reaching into the next rank's rows is refused
        bad = [tc.whole(tc.View(0, 17, 64, 64, 4, 0), 1), None, None]
        with pytest.raises(tc.BoundsError):
            tc.prepare_all_gather(pair.rep, w["rows"], w["cols"], 4, schedules=bad)
    finally:
        pair.close()


def test_many_chunks():
    # 275 one-tile chunks per rank, 1100 in all: more chunks than the
    # completion check has threads, each chunk marked by its own CTA.
    w = dict(P=4, rows=1100, cols=64, elem="u32", builder="tile_chunks", bm=4, bn=64,
             tiles_per_chunk=1, rounds=2)
    _run_all_rounds("many chunks", w)


def test_large_pieces():
    # Pieces of 1 MiB: a 1 MiB region per chunk goes to one wave whole.
    w = dict(P=3, rows=512, cols=1024, elem="u32", builder="chunks", n=2, writers=4, rounds=2)
    pair = Pair(w, piece_bytes=1 << 20)
    try:
        assert pair.plan.stats()["pieces"] == 6
        for r in (1, 2):
            log(f"large pieces round {r}")
            pair.gpu_round_fill()
            pair.oracle_round()
            pair.compare(f"large pieces round {r}")
            pair.plan.next_round()
            pair.sim.next_round()
    finally:
        pair.close()


def test_rank_that_sends_nothing_and_single_rank():
    w = dict(P=3, rows=20, cols=24, elem="u32", builder="chunks", n=2, writers=1, rounds=2)
    pair = Pair(w)
    try:
        pair.plan.close()
        sched = list(pair.ts)
        sched[1] = None                                   # broadcast-style: rank 1 silent
        pair.plan = tc.TriggeredPlan(pair.rep, sched, backstop_s=20.0)
        pair.sim = oplan.PlanSim(pair.sim.rep, [pair.os[0], None, pair.os[2]])
        h = pair.plan.start(pair.stream)
        pair.plan.fill(h, pair.tv, pair.seed, kind="u32", stream=pair.stream)
        pair.plan.wait(10.0)

        def produce(p, r):
            if p != 1:
                from tests.gpu_common import oracle_produce
                oracle_produce(pair.sim.rep[p], pair.ov[p], "u32", pair.seed, p, r)
        oplan.run_round(pair.sim, produce)
        # the GPU fill writes only scheduled bytes, so rank 1's rows keep the sentinel
        pair.compare("silent rank")
    finally:
        pair.close()
    w1 = dict(P=1, rows=8, cols=64, elem="u32", builder="whole", writers=2, rounds=2)
    _run_all_rounds("single rank", w1)


def test_plan_where_no_rank_sends():
    # Every schedule empty: rounds still start, complete and advance, and the
    # replicas keep their sentinel.
    w = dict(P=3, rows=8, cols=32, elem="u32", builder="whole", writers=1, rounds=3)
    pair = Pair(w)
    try:
        _swap_in(pair, [None] * 3, [None] * 3)
        for r in range(1, 4):
            log(f"no sender round {r}")
            h = pair.plan.start(pair.stream)
            pair.plan.fill(h, pair.tv, pair.seed, kind="u32", stream=pair.stream)
            pair.plan.wait(10.0)
            assert pair.plan.state == "DONE"
            oplan.run_round(pair.sim, lambda p, rr: None)
            pair.compare(f"no sender round {r}")
            pair.plan.next_round()
            pair.sim.next_round()
    finally:
        pair.close()


def test_withheld_mark_times_out_then_resumes():
    w = dict(workloads.SMALL["u32_chunks_ragged_p3"])
    pair = Pair(w)
    try:
        h = pair.plan.start(pair.stream)
        pair.plan.fill(h, pair.tv, pair.seed, kind="u32", mark=False, stream=pair.stream)
        # every mark except one of rank 1's chunk 2
        for p in range(3):
            for c in range(5):
                n = 2 - (1 if (p, c) == (1, 2) else 0)
                pair.plan.mark(h, p, c, n, stream=pair.stream)
        with pytest.raises(tc.PlanTimeout) as ei:
            pair.plan.wait(0.5)
        assert (1, 2) in ei.value.chunks and (1, 3) in ei.value.chunks
        assert pair.plan.state == "STARTED"
        # the oracle names the same chunks
        pair.sim.start()
        from tests.gpu_common import oracle_produce
        for p in range(3):
            oracle_produce(pair.sim.rep[p], pair.ov[p], "u32", pair.seed, p, 1)
        for p in range(3):
            for c in range(5):
                for _ in range(2 - (1 if (p, c) == (1, 2) else 0)):
                    pair.sim.mark(p, c)
        with pytest.raises(oplan.PlanError) as eo:
            pair.sim.wait()
        assert sorted(ei.value.chunks) == sorted(eo.value.chunks)
        pair.compare("after timeout", partial=True)
        pair.plan.mark(h, 1, 2, 1, stream=pair.stream)
        pair.sim.mark(1, 2)
        pair.plan.wait(10.0)
        pair.sim.wait()
        pair.compare("after resume")
        assert pair.plan.stats()["launches"] == 2
    finally:
        pair.close()


def test_extra_mark_fails_the_plan():
    w = dict(workloads.SMALL["u32_whole_p5"])
    pair = Pair(w)
    try:
        for r in (1, 2):
            h = pair.plan.start(pair.stream)
            pair.plan.fill(h, pair.tv, pair.seed, kind="u32", stream=pair.stream)
            extra = [(3, 0)] if r == 2 else []
            for p, c in extra:
                pair.plan.mark(h, p, c, 1, stream=pair.stream)
            if r == 2:
                with pytest.raises(tc.ExtraMarksError) as ei:
                    pair.plan.wait(10.0)
                assert ei.value.chunks == [(3, 0)]
                with pytest.raises(oplan.PlanError) as eo:
                    pair.oracle_round(extra=extra)
                assert eo.value.code == "EEXTRA" and eo.value.chunks == [(3, 0)]
                assert pair.plan.state == "FAILED"
                torch.cuda.synchronize()
                g = pair.plan.gates()
                assert np.array_equal(g, pair.sim.gate_bytes())
                with pytest.raises(tc.StateError):
                    pair.plan.next_round()
            else:
                pair.plan.wait(10.0)
                pair.oracle_round()
                pair.compare("extra-mark run round 1")
                pair.plan.next_round()
                pair.sim.next_round()
    finally:
        pair.close()


# (P, chunks per rank): by gate rows over several passes and two batches of
# 64 (2, 40), over three passes (8, 3); one lane per chunk over two batches
# (3, 30) and (16, 5).
@pytest.mark.parametrize("P,n", [(2, 40), (8, 3), (3, 30), (16, 5)])
def test_in_engine_check_names_the_chunks_the_oracle_names(P, n):
    # The copy engine's own completion check covers the chunks either one
    # gate row per lane or one chunk per lane, batch by batch of up to 64,
    # and must name exactly the chunks the oracle names in any of them.  The
    # engine runs the check only if wait()'s request reaches it within its
    # polling window (else the check kernel runs it, with the same result),
    # so a fresh plan is tried again, a few times at most, until the engine
    # did.
    w = dict(P=P, rows=4 * n, cols=64, elem="u32", builder="chunks", n=n, writers=1, rounds=2)
    extra = [(0, 1), (P // 2, n - 2), (P - 1, n - 1)]
    paths = []
    for attempt in range(4):
        pair = Pair(w)
        try:
            assert pair.plan.G == P * n
            log(f"in-engine check P={P} n={n} attempt {attempt} round 1")
            h = pair.plan.start(pair.stream)
            pair.plan.fill(h, pair.tv, pair.seed, kind="u32", stream=pair.stream)
            pair.plan.wait(10.0)
            paths.append(pair.plan.stats()["engine_checked"])
            pair.oracle_round()
            pair.compare(f"in-engine check P={P} round 1")
            pair.plan.next_round()
            pair.sim.next_round()
            log(f"in-engine check P={P} n={n} attempt {attempt} round 2")
            h = pair.plan.start(pair.stream)
            pair.plan.fill(h, pair.tv, pair.seed, kind="u32", stream=pair.stream)
            for p, c in extra:
                pair.plan.mark(h, p, c, 1, stream=pair.stream)
            with pytest.raises(tc.ExtraMarksError) as ei:
                pair.plan.wait(10.0)
            in_engine = pair.plan.stats()["engine_checked"]
            paths.append(in_engine)
            with pytest.raises(oplan.PlanError) as eo:
                pair.oracle_round(extra=extra)
            assert eo.value.code == "EEXTRA"
            assert sorted(ei.value.chunks) == sorted(eo.value.chunks) == sorted(extra)
        finally:
            pair.close()
        if in_engine:
            break
    log(f"check paths (1 = in the engine): {paths}")
    assert paths[-1] == 1


def test_state_order_and_round_limit():
    w = dict(P=2, rows=4, cols=64, elem="u32", builder="whole", writers=1, rounds=1)
    pair = Pair(w)
    try:
        with pytest.raises(tc.InvalidArgument):          # the legacy default stream
            pair.plan.start(torch.cuda.default_stream())
        with pytest.raises(tc.StateError):
            pair.plan.wait(1.0)
        with pytest.raises(tc.StateError):
            pair.plan.next_round()
        h = pair.plan.start(pair.stream)
        with pytest.raises(tc.StateError):
            pair.plan.start(pair.stream)
        pair.plan.fill(h, pair.tv, pair.seed, kind="u32", stream=pair.stream)
        pair.plan.wait(10.0)
        pair.plan.debug_set_round(0xFFFFFFFF)
        with pytest.raises(tc.RoundLimitError):
            pair.plan.next_round()
    finally:
        pair.close()


def test_create_rejects_overlap_and_small_workspace():
    require_gpu()
    rep = torch.zeros((2, 4096), dtype=torch.uint8, device="cuda")
    whole_out = tc.whole(tc.View(0, 2, 2048, 2048, 1, 0))
    with pytest.raises(tc.OverlapError):
        tc.TriggeredPlan(rep, [whole_out, whole_out])
    mine = [tc.whole(tc.View(p * 2048, 1, 2048, 2048, 1, 0)) for p in range(2)]
    with pytest.raises(tc.WorkspaceTooSmall):
        tc.TriggeredPlan(rep, mine, workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    with pytest.raises(tc.BoundsError):
        tc.TriggeredPlan(rep, [mine[1], mine[0]], own_rows_bytes=2048)


def test_create_checks_replica_and_workspace_memory():
    # Through the C-ABI: a replica in host memory, a replica size past the end
    # of its allocation, and a workspace size past the end of its allocation
    # are refused at create time; the same call with good memory succeeds.
    import ctypes as C
    from triggered_copy_amd import _lib
    require_gpu()
    B = 4096
    rep = torch.zeros((2, B), dtype=torch.uint8, device="cuda")
    scheds = [tc.whole(tc.View(p * 2048, 1, 2048, 2048, 1, 0)) for p in range(2)]
    need = C.c_uint64()
    sp = (C.c_void_p * 2)(*[s_.ptr.value for s_ in scheds])
    assert tc.lib().tc_plan_workspace_bytes(2, sp, 0, C.byref(need)) == _lib.OK
    ws = torch.zeros(need.value, dtype=torch.uint8, device="cuda")
    host = torch.zeros(B, dtype=torch.uint8).pin_memory()

    def create(reps, buffer_bytes=B, ws_bytes=need.value):
        rp = (C.c_void_p * 2)(*reps)
        d = _lib.PlanDesc()
        d.nranks, d.flags = 2, 0
        d.replicas = C.cast(rp, C.POINTER(C.c_void_p))
        d.buffer_bytes = buffer_bytes
        d.schedules = C.cast(sp, C.POINTER(C.c_void_p))
        d.workspace, d.workspace_bytes = ws.data_ptr(), ws_bytes
        d.engine_backstop_us = 20_000_000
        out = C.c_void_p()
        rc = tc.lib().tc_plan_create(C.byref(d), C.byref(out))
        return rc, out

    good = [rep[0].data_ptr(), rep[1].data_ptr()]
    rc, _ = create([good[0], host.data_ptr()])
    assert rc == _lib.EINVAL, tc.lib().tc_last_error()
    rc, _ = create(good, buffer_bytes=1 << 40)
    assert rc == _lib.EBOUNDS, tc.lib().tc_last_error()
    rc, _ = create(good, ws_bytes=1 << 40)
    assert rc == _lib.EBOUNDS, tc.lib().tc_last_error()
    rc, out = create(good)
    assert rc == _lib.OK, tc.lib().tc_last_error()
    closing = C.c_int(0)
    assert tc.lib().tc_plan_close(out, C.byref(closing)) == _lib.OK


def test_barrier_p8_thousand_generations():
    require_gpu()
    w = workloads.FULL["barrier_p8"]
    P, G = w["P"], w["gens"]
    W = torch.zeros((P, P), dtype=torch.int32, device="cuda")
    x = torch.zeros((2, P), dtype=torch.int32, device="cuda")
    y = torch.zeros((G, P), dtype=torch.int32, device="cuda")
    snap = torch.zeros((G, P, P), dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    log("barrier P=8 x 1000")
    tc.barrier(W, P, 1, G, status, x=x, y=y, snap=snap)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(W.cpu().numpy(), obarrier.run(P, G))
    assert np.array_equal(y.cpu().numpy(), obarrier.reveal(P, 1, G))
    s = snap.cpu().numpy().astype(np.int64)
    for i in range(G):
        g = i + 1
        off = ~np.eye(P, dtype=bool)
        rows = s[i]
        assert (np.diagonal(rows) == 0).all()
        assert np.isin(rows[off], [g, g + 1]).all()
    # one more generation on the same window: first_gen continues the count
    tc.barrier(W, P, G + 1, 1, status)
    torch.cuda.synchronize()
    assert np.array_equal(W.cpu().numpy(), obarrier.closed_form(P, G + 1))


def test_barrier_one_generation_rows_p2():
    require_gpu()
    W = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    tc.barrier(W, 2, 1, 1, status)
    torch.cuda.synchronize()
    assert W.cpu().numpy().tolist() == obarrier.run(2, 1).tolist() == [[0, 1], [1, 0]]


def test_barrier_missing_peer_ends_with_status():
    require_gpu()
    # Generation 2 on a zero window whose peers never ran generation 1: every
    # wait must run out of polls and the kernel must still end.
    W = torch.zeros((3, 3), dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    tc.barrier(W, 3, 2, 1, status, max_polls=2000)
    torch.cuda.synchronize()
    assert int(status.item()) != 0


def test_consumer_wait_runs_out_of_polls():
    # A chunk whose last mark is withheld never arrives: the consumer's wait
    # for it ends after its poll budget with status 2 (the kernel exits), the
    # other chunks are consumed with status 1; closing the plan then sends the
    # withheld chunk as it stands.
    w = dict(workloads.SMALL["u32_tiles_shuffled_p3"])
    pair = Pair(w)
    try:
        G = pair.plan.G
        out = torch.full_like(pair.rep[0], 0x5A)
        status = torch.zeros(G, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        h = pair.plan.start(pair.stream)
        pair.plan.fill(h, pair.tv, pair.seed, kind="u32", mark=False, stream=pair.stream)
        last = pair.sim.n[0] - 1
        for p in range(pair.P):
            for c in range(pair.sim.n[p]):
                wr = pair.sim.writers(p, c)
                n = wr - 1 if (p, c) == (0, last) else wr
                if n:
                    pair.plan.mark(h, p, c, n, stream=pair.stream)
        log("consumer with a withheld chunk, 2000 polls per wait")
        pair.plan.consume_copy(h, 2, out, status, max_polls=2000, stream=pair.stream)
        # Read on the producers' stream: a copy on the legacy default stream
        # would wait for the engine, which waits for the withheld gate.
        with torch.cuda.stream(pair.stream):
            st = status.cpu().numpy()
        g_withheld = last                      # rank 0's chunks come first
        assert st[g_withheld] == 2, st.tolist()
        assert (np.delete(st, g_withheld) == 1).all(), st.tolist()
        with pytest.raises(tc.PlanTimeout):
            pair.plan.wait(0.2)
        assert pair.plan.close() == "CLOSED"
    finally:
        pair.close()


def test_device_view_consumer_sees_fresh_data():
    w = dict(workloads.SMALL["u32_tiles_shuffled_p3"])
    pair = Pair(w)
    try:
        G = pair.plan.G
        out = torch.full_like(pair.rep[0], 0x5A)
        status = torch.zeros(G, dtype=torch.int32, device="cuda")
        side = torch.cuda.Stream()
        for r in (1, 2):
            log(f"consumer round {r}")
            status.zero_()
            orders, dev = pair.orders_device(r)
            torch.cuda.synchronize()         # nothing may wait for the device after start()
            h = pair.plan.start(pair.stream)
            # The consumer spins on arrivals, so it is queued after the work it
            # depends on: streams may share a hardware queue.
            pair.plan.fill(h, pair.tv, pair.seed, kind="u32", serial=True, order=dev,
                           order_stride=orders.shape[1], stream=pair.stream)
            with torch.cuda.stream(side):
                pair.plan.consume_copy(h, 2, out, status, max_polls=1 << 22, stream=side)
            pair.plan.wait(10.0)
            side.synchronize()
            pair.oracle_round()
            pair.compare(f"consumer round {r}")
            assert (status.cpu().numpy() == 1).all()
            # what the consumer copied out of replica 2 is this round's data
            got = out.cpu().numpy()
            want = pair.sim.rep[2]
            for s in pair.os:
                for ch in s.chunks:
                    for off, rows, rb, pitch in ch.regions:
                        for i in range(rows):
                            a = off + i * pitch
                            assert np.array_equal(got[a:a + rb], want[a:a + rb])
            pair.plan.next_round()
            pair.sim.next_round()
    finally:
        pair.close()
