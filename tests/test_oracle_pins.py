"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test checks one oracle part against a published value, a closed form, a
library routine it must reduce to, a brute-force enumeration, or a value the
pages print (fixtures under tests/golden/, each with its citation).
"""

import itertools
import os
import random
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import barrier, cvalues, gemm, plan, schedule, values
from oracle.schedule import GIB, View

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line)
    return rows


# ------------------------------------------------------------------ values

def test_splitmix64_published_vector():
    # Published output of the reference splitmix64.c generator seeded with
    # 1234567 (first five outputs).
    assert values.splitmix64_stream(1234567, 5) == [
        6457827717110365317, 3203168211198807973, 9817491932198370423,
        4593380528125082431, 16408922859458223821]


def test_c_twin_reproduces_the_published_vector():
    # The oracle's C twin of the value hash (oracle/values.c), used to check
    # every element of the largest workloads, pinned to the same published
    # splitmix64.c output for seed 1234567.
    assert cvalues.splitmix64_stream(1234567, 5) == [
        6457827717110365317, 3203168211198807973, 9817491932198370423,
        4593380528125082431, 16408922859458223821]


@pytest.mark.parametrize("rank,rnd,first,n,nthreads", [(0, 1, 0, 4099, 1), (3, 2, (1 << 32) - 5000, 5000, 7),
                                                        (15, 65535, 123456789, 100003, 16)])
def test_c_twin_pattern_equals_the_numpy_oracle(rank, rnd, first, n, nthreads):
    # Element by element, across thread splits and at the top of the index
    # range; a wrong key layout (rank or round in the wrong bits) or a
    # dropped salt fails here.
    out = np.zeros(n, dtype=np.uint32)
    cvalues.u32_pattern_into(out, 0x7C0FFEE, rank, rnd, first, nthreads=nthreads)
    want = values.u32_pattern(0x7C0FFEE, rank, rnd, np.arange(first, first + n, dtype=np.uint64))
    assert np.array_equal(out, want)
    with pytest.raises(ValueError):
        cvalues.u32_pattern_into(np.zeros(2, dtype=np.uint32), 1, 1 << 16, 0, 0)


def test_mix64_vectorised_matches_scalar():
    xs = [0, 1, 2, 0xFFFFFFFFFFFFFFFF, 0x123456789ABCDEF0] + [random.getrandbits(64) for _ in range(100)]
    got = values.mix64_np(np.array(xs, dtype=np.uint64))
    assert [int(v) for v in got] == [values.mix64_int(x) for x in xs]


def test_bf16_uniform_by_exact_arithmetic():
    idx = np.arange(0, 4096, dtype=np.uint64)
    bits = values.bf16_uniform_bits(7, 1, 2, idx)
    h = values.element_hash(7, 1, 2, idx)
    for i in range(0, 4096, 97):
        u = int(h[i]) >> 41
        f = Fraction(u - (1 << 22), 1 << 22)            # exact value in [-1, 1)
        f32 = struct.unpack("<I", struct.pack("<f", float(f)))[0]
        assert float(f) == f                             # exact in binary32
        assert int(bits[i]) == f32 >> 16                 # truncated to bf16
    as_f = (bits.astype(np.uint32) << 16).view(np.float32)
    assert as_f.min() >= -1.0 and as_f.max() < 1.0
    assert abs(float(as_f.mean())) < 0.05


def test_value_keys_are_distinct_per_rank_round_index():
    idx = np.arange(1000, dtype=np.uint64)
    a = values.element_hash(3, 0, 1, idx)
    b = values.element_hash(3, 1, 1, idx)
    c = values.element_hash(3, 0, 2, idx)
    assert len(set(a.tolist()) | set(b.tolist()) | set(c.tolist())) == 3000


# --------------------------------------------------------------- regions

def _element_bytes(v: View, r0, r1, c0, c1):
    out = set()
    for i in range(r0, r1):
        for j in range(c0, c1):
            base = v.byte_offset + (i * v.row_stride + j) * v.elem_bytes
            out.update(range(base, base + v.elem_bytes))
    return out


def _region_bytes(regs):
    out = []
    for off, rows, row_bytes, pitch in regs:
        for i in range(rows):
            out.extend(range(off + i * pitch, off + i * pitch + row_bytes))
    return out


def test_window_regions_bruteforce():
    rnd = random.Random(1)
    for _ in range(400):
        e = rnd.choice([1, 2, 4])
        cols = rnd.randint(1, 9)
        v = View(rnd.randint(0, 40), rnd.randint(1, 9), cols, cols + rnd.choice([0, 0, 1, 3]), e)
        r0 = rnd.randrange(v.rows)
        r1 = rnd.randint(r0 + 1, v.rows)
        c0 = rnd.randrange(v.cols)
        c1 = rnd.randint(c0 + 1, v.cols)
        regs = schedule.window_regions(v, r0, r1, c0, c1)
        got = _region_bytes(regs)
        assert len(got) == len(set(got))
        assert set(got) == _element_bytes(v, r0, r1, c0, c1)
        for off, rows, row_bytes, pitch in regs:       # normal form
            assert rows >= 1 and row_bytes >= 1
            if rows == 1:
                assert pitch == row_bytes


def test_linear_split_closed_forms():
    assert schedule.split_region((0, 1, GIB, GIB)) == [(0, 1, GIB, GIB)]
    assert schedule.split_region((16, 1, GIB + 1, GIB + 1)) == [(16, 1, GIB, GIB), (16 + GIB, 1, 1, 1)]
    n = 5 * GIB + 12345
    parts = schedule.split_region((64, 1, n, n))
    assert sum(p[2] for p in parts) == n and all(p[2] <= GIB for p in parts)
    assert [p[0] for p in parts] == [64 + k * GIB for k in range(6)]


def test_split_golden_whole_1p5gib():
    want = [tuple(int(x) for x in r.split()) for r in _golden("split_1gib.txt")]
    v = View(0, 786432, 512, 512, 4)
    s = schedule.whole(v, 192)
    assert [(r[0], r[2]) for r in s.chunks[0].regions] == want


def test_2d_split_by_whole_rows():
    # 3000 rows of 1 MiB at a 2 MiB pitch: 1024 rows per piece.
    reg = (0, 3000, 1 << 20, 2 << 20)
    parts = schedule.split_region(reg)
    assert [p[1] for p in parts] == [1024, 1024, 952]
    assert sum(p[1] * p[2] for p in parts) == 3000 << 20
    assert sorted(_region_bytes([(0, 3, 5, 9)])) == sorted(_region_bytes(schedule.split_region((0, 3, 5, 9))))


# ------------------------------------------------------------- builders

def test_chunks_follow_array_split():
    for rows in range(1, 40):
        for n in range(1, rows + 1):
            blocks = schedule.row_blocks(rows, n)
            ref = np.array_split(np.arange(rows), n)
            assert [(int(b[0]), int(b[-1]) + 1) for b in ref] == blocks
    with pytest.raises(schedule.ScheduleError):
        schedule.row_blocks(3, 4)


def test_tile_chunks_partition_the_view():
    rnd = random.Random(2)
    for _ in range(60):
        e = rnd.choice([1, 2, 4])
        cols = rnd.randint(1, 9)
        v = View(rnd.randint(0, 16), rnd.randint(1, 9), cols, cols + rnd.choice([0, 2]), e)
        bm, bn = rnd.randint(1, 4), rnd.randint(1, 4)
        tm, tn = -(-v.rows // bm), -(-v.cols // bn)
        order = list(range(tm * tn))
        rnd.shuffle(order)
        T = rnd.randint(1, 5)
        s = schedule.tile_chunks(v, bm, bn, T, order)
        allb = []
        for ch in s.chunks:
            allb.extend(_region_bytes(ch.regions))
        assert sorted(allb) == sorted(_element_bytes(v, 0, v.rows, 0, v.cols))
        assert sum(ch.writers for ch in s.chunks) == tm * tn
        assert all(ch.writers <= T for ch in s.chunks)


def test_tile_chunks_gemm_tile_census():
    v = View(0, 2000, 2000, 2000, 2)
    order = [schedule.tile_of(s, 16, 16, 8) for s in range(256)]
    s = schedule.tile_chunks(v, 128, 128, 256, order)
    assert len(s.chunks) == 1 and s.chunks[0].writers == 256
    regs = s.chunks[0].regions
    shapes = sorted((r[1], r[2]) for r in regs)
    census = {k: shapes.count(k) for k in set(shapes)}
    assert census == {(128, 256): 225, (128, 160): 15, (80, 256): 15, (80, 160): 1}
    assert sum(r[1] * r[2] for r in regs) == 8_000_000
    assert all(r[3] == 4000 for r in regs)


def test_grouped_order_reductions():
    for tm in range(1, 21):
        for tn in range(1, 21):
            nt = tm * tn
            for g in range(1, 10):
                order = [schedule.tile_of(s, tm, tn, g) for s in range(nt)]
                assert sorted(order) == list(range(nt))
            assert [schedule.tile_of(s, tm, tn, 1) for s in range(nt)] == list(range(nt))
            for g in range(tm, tm + 3):          # one band: column-major
                assert [schedule.tile_of(s, tm, tn, g) for s in range(nt)] == \
                    [(s % tm) * tn + s // tm for s in range(nt)]


def test_tile_chunks_rejects_non_permutation():
    v = View(0, 4, 4, 4, 4)
    with pytest.raises(schedule.ScheduleError):
        schedule.tile_chunks(v, 2, 2, 2, [0, 1, 1, 3])


# ------------------------------------------------------------ validation

def _bytes_of_schedule(s):
    out = set()
    for ch in s.chunks:
        out.update(_region_bytes(ch.regions))
    return out


def test_overlap_check_bruteforce():
    rnd = random.Random(3)
    for _ in range(300):
        P = rnd.randint(2, 3)
        B = 64
        scheds = []
        for p in range(P):
            regs = []
            for _ in range(rnd.randint(1, 3)):
                rows = rnd.randint(1, 3)
                rb = rnd.randint(1, 6)
                pitch = rb + rnd.randint(0, 4) if rows > 1 else rb
                off = rnd.randint(0, B - ((rows - 1) * pitch + rb))
                regs.append((off, rows, rb, pitch))
            scheds.append(schedule.from_tables([(0, len(regs), 1)], regs))
        sets = [_bytes_of_schedule(s) for s in scheds]
        clash = any(sets[a] & sets[b] for a in range(P) for b in range(a + 1, P))
        if clash:
            with pytest.raises(schedule.ScheduleError) as ei:
                schedule.validate(B, scheds)
            assert ei.value.code == schedule.EOVERLAP
        else:
            schedule.validate(B, scheds)


def test_whole_buffer_on_every_rank_rejected():
    P, rows, cols = 4, 8, 16
    out = View(0, P * rows, cols, cols, 4)
    with pytest.raises(schedule.ScheduleError) as ei:
        schedule.validate(P * rows * cols * 4, [schedule.whole(out) for _ in range(P)])
    assert ei.value.code == schedule.EOVERLAP
    mine = [schedule.whole(View(p * rows * cols * 4, rows, cols, cols, 4)) for p in range(P)]
    schedule.validate(P * rows * cols * 4, mine, own_rows_bytes=rows * cols * 4)


def test_bounds_and_own_rows():
    v = View(0, 4, 4, 4, 4)
    with pytest.raises(schedule.ScheduleError) as ei:
        schedule.validate(63, [schedule.whole(v)])
    assert ei.value.code == schedule.EBOUNDS
    other = View(64, 4, 4, 4, 4)
    with pytest.raises(schedule.ScheduleError) as ei:
        schedule.validate(128, [schedule.whole(other), None], own_rows_bytes=64)
    assert ei.value.code == schedule.EBOUNDS


# ----------------------------------------------------------- simulation

def _sim(P, rows, cols, builder, **kw):
    nbytes = P * rows * cols * 4
    reps = [np.full(nbytes, 0xA5, dtype=np.uint8) for _ in range(P)]
    views = [View(p * rows * cols * 4, rows, cols, cols, 4) for p in range(P)]
    scheds = [builder(v, **kw) for v in views]
    return plan.PlanSim(reps, scheds), views


def _produce(sim, views, seed=11):
    def f(p, rnd):
        v = views[p]
        n = v.rows * v.cols
        sim.rep[p][v.byte_offset:v.byte_offset + 4 * n] = values.block_bytes("u32", seed, p, rnd, n)
    return f


def test_writer_counter_closed_form_and_no_stale_data():
    sim, views = _sim(3, 6, 8, schedule.chunks, n=3, writers=2)
    for r in range(1, 5):
        plan.run_round(sim, _produce(sim, views))
        for p in range(3):
            for c in range(3):
                row = sim.gates[p, sim.g(p, c)]
                assert int(row[plan.WRITERS]) == r * 2 and int(row[plan.READY]) == r
                assert int(row[plan.ARRIVAL]) == 0
                for q in range(3):
                    if q != p:
                        peer = sim.gates[q, sim.g(p, c)]
                        assert int(peer[plan.ARRIVAL]) == r
                        assert int(peer[plan.READY]) == 0 and int(peer[plan.WRITERS]) == 0
        want = np.concatenate([values.block_bytes("u32", 11, p, r, 48) for p in range(3)])
        for q in range(3):
            assert np.array_equal(sim.rep[q], want)      # this round's data everywhere
        assert (sim.cur[~np.eye(3, dtype=bool)] == 3).all()
        sim.next_round()


def test_u32_whole_p8_counters_after_ten_rounds():
    # Counters do not depend on the block size, so a small block stands in.
    sim, views = _sim(8, 1, 64, schedule.whole, writers=8)
    for r in range(1, 11):
        plan.run_round(sim, _produce(sim, views))
        if r < 10:
            sim.next_round()
    for p in range(8):
        own = sim.gates[p, p]
        assert (int(own[plan.WRITERS]), int(own[plan.READY])) == (80, 10)
        assert all(int(sim.gates[q, p, plan.ARRIVAL]) == 10 for q in range(8) if q != p)


def test_extra_mark_is_named_and_fails_the_plan():
    sim, views = _sim(8, 1, 64, schedule.whole, writers=8)
    for r in range(1, 7):
        plan.run_round(sim, _produce(sim, views))
        sim.next_round()
    with pytest.raises(plan.PlanError) as ei:
        plan.run_round(sim, _produce(sim, views), extra_marks=[(3, 0)])
    assert ei.value.code == "EEXTRA" and ei.value.chunks == [(3, 0)]
    assert sim.state == plan.FAILED
    assert int(sim.gates[3, 3, plan.WRITERS]) == 8 * 7 + 1
    with pytest.raises(plan.PlanError):
        sim.next_round()


def test_withheld_mark_times_out_naming_the_chunk_then_recovers():
    sim, views = _sim(3, 6, 8, schedule.chunks, n=3, writers=2)
    with pytest.raises(plan.PlanError) as ei:
        plan.run_round(sim, _produce(sim, views), withheld=[(1, 1)])
    assert ei.value.code == "ETIMEOUT"
    # chunk (1,1) is short; (1,2) is marked but queued behind it
    assert ei.value.chunks == [(1, 1), (1, 2)]
    assert sim.state == plan.STARTED
    sim.mark(1, 1)
    sim.wait()
    assert sim.state == plan.DONE


def _prefix_len(marked, n):
    k = 0
    while k < n and k in marked:
        k += 1
    return k


def test_head_of_line_prefix_invariant_all_orders():
    # Every order of single-writer marks: after each mark the cursor is the
    # longest marked prefix, and each queue's log is 0, 1, ..., n-1.
    for n in range(1, 5):
        for perm in itertools.permutations(range(n)):
            sim, views = _sim(3, n, 4, schedule.chunks, n=n)
            sim.start()
            for p in range(3):
                _produce(sim, views)(p, 1)
            marked = set()
            for c in perm:
                for p in range(3):
                    sim.mark(p, c)
                marked.add(c)
                for p in range(3):
                    for q in range(3):
                        if p != q:
                            assert int(sim.cur[p, q]) == _prefix_len(marked, n)
            sim.wait()
            assert all(log == list(range(n)) for log in sim.log.values())


def test_interleavings_are_confluent():
    # Random interleavings of marks (2 writers) and single queue steps reach
    # the same final replicas, gates and cursors.
    rnd = random.Random(4)
    ref = None
    for trial in range(300):
        sim, views = _sim(3, 4, 4, schedule.chunks, n=4, writers=2)
        sim.start()
        for p in range(3):
            _produce(sim, views)(p, 1)
        events = [("m", p, c) for p in range(3) for c in range(4) for _ in range(2)]
        events += [("s", p, q) for p in range(3) for q in range(3) if p != q for _ in range(6)]
        rnd.shuffle(events)
        for ev in events:
            if ev[0] == "m":
                sim.mark(ev[1], ev[2], advance=False)
            else:
                sim.step_queue(ev[1], ev[2])
        sim.wait()
        state = (tuple(r.tobytes() for r in sim.rep), sim.gates.tobytes(), sim.cur.tobytes())
        if ref is None:
            ref = state
        assert state == ref


def test_counters_only_mode_follows_the_full_simulation():
    # The counters-only mode (no replica bytes; used for the 1.5 GiB GPU
    # runs) is tied to the pinned full simulation: on random schedules and
    # mark orders, over several rounds, its gate rows, cursors and delivery
    # logs equal the full mode's after every single mark.
    rnd = random.Random(11)
    for trial in range(40):
        P = rnd.randint(2, 4)
        rows, cols = rnd.randint(4, 12), rnd.randint(3, 9)
        nbytes = P * rows * cols * 4
        views = [schedule.View(p * rows * cols * 4, rows, cols, cols, 4) for p in range(P)]
        sched = [schedule.chunks(v, rnd.randint(1, min(rows, 4)), rnd.randint(1, 3)) for v in views]
        full = plan.PlanSim([np.zeros(nbytes, np.uint8) for _ in range(P)], sched)
        bare = plan.PlanSim(None, sched, buffer_bytes=nbytes)
        for r in range(1, 4):
            full.start()
            bare.start()
            marks = [(p, c) for p in range(P) for c in range(full.n[p]) for _ in range(full.writers(p, c))]
            rnd.shuffle(marks)
            for p, c in marks:
                full.mark(p, c)
                bare.mark(p, c)
                assert np.array_equal(full.gates, bare.gates) and np.array_equal(full.cur, bare.cur)
            full.wait()
            bare.wait()
            assert full.log == bare.log
            full.next_round()
            bare.next_round()


def test_simulation_equals_plain_definition():
    rnd = random.Random(5)
    for P in (2, 3, 4):
        rows, cols = 9, 7
        nbytes = P * rows * cols * 4
        reps = [np.full(nbytes, 0xA5, dtype=np.uint8) for _ in range(P)]
        views = [View(p * rows * cols * 4, rows, cols, cols, 4) for p in range(P)]
        scheds = [schedule.tile_chunks(v, 4, 3, 2) if p % 2 else schedule.chunks(v, 3) for p, v in enumerate(views)]
        scheds[rnd.randrange(P)] = None                  # one rank sends nothing
        sim = plan.PlanSim(reps, scheds)
        blocks = []
        sim.start()
        for p in range(P):
            v = views[p]
            sim.rep[p][v.byte_offset:v.byte_offset + 4 * rows * cols] = values.block_bytes("u32", 9, p, 1, rows * cols)
            blocks.append(sim.rep[p].copy())
        before = [r.copy() for r in sim.rep]            # after the producers ran
        for p in range(P):
            for c in range(sim.n[p]):
                for _ in range(sim.writers(p, c)):
                    sim.mark(p, c)
        sim.wait()
        want = plan.expected_after_round(scheds, blocks, before)
        for q in range(P):
            assert np.array_equal(sim.rep[q], want[q])


def test_round_limit():
    sim, views = _sim(2, 2, 4, schedule.whole)
    plan.run_round(sim, _produce(sim, views))
    sim.round = plan.ROUND_LIMIT                      # as after 2**32 - 2 rounds
    with pytest.raises(plan.PlanError) as ei:
        sim.next_round()
    assert ei.value.code == "EROUNDS"


def test_state_machine_misuse():
    sim, views = _sim(2, 2, 4, schedule.whole)
    with pytest.raises(plan.PlanError):
        sim.wait()
    with pytest.raises(plan.PlanError):
        sim.next_round()
    sim.start()
    with pytest.raises(plan.PlanError):
        sim.start()


# --------------------------------------------------------------- barrier

def test_barrier_golden_rows_p2():
    want = {int(k): [int(x) for x in v.split()] for k, v in (r.split(":") for r in _golden("barrier_rows_p2.txt"))}
    W = barrier.run(2, 1)
    for r, row in want.items():
        assert list(W[r]) == row


def test_barrier_own_row_pattern_and_closed_form():
    for P in range(2, 9):
        W = barrier.run(P, 1)
        for r in range(P):
            assert list(W[r]) == [0 if s == r else 1 for s in range(P)]
        assert np.array_equal(barrier.run(P, 17), barrier.closed_form(P, 17))
        assert np.array_equal(barrier.run(P, 5, first_gen=13, W=barrier.closed_form(P, 12)),
                              barrier.closed_form(P, 17))


def test_barrier_reveal_golden_p2():
    want = {int(k): int(v) for k, v in (r.split(":") for r in _golden("reveal_p2.txt"))}
    y = barrier.reveal(2, 1, 3)
    for i, g in enumerate(range(1, 4)):
        for r, src in want.items():
            assert y[i, r] == barrier.stage_value(g, src)


# ------------------------------------------------------------------ gemm

def test_gemm_reference_against_float64():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal((64, 96)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bt = (rng.standard_normal((48, 96)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    r32 = gemm.gemm_ref(a, bt)
    r64 = gemm.gemm_ref_f64(a, bt)
    assert np.linalg.norm(r32 - r64) / np.linalg.norm(r64) < 1e-5
    ok, _, _ = gemm.within_tolerance(r32, r64)
    assert ok
    bad = r64.copy()
    bad[3, 4] += 0.5 * np.sqrt(np.mean(r64 ** 2))
    assert not gemm.within_tolerance(bad, r64)[0]


# ------------------------------------------------------------- consumer deps

def _deps_brute(schedules, v, tile_rows):
    """Every region byte enumerated: its view row and column decide its block."""
    pitch, e = v.row_stride * v.elem_bytes, v.elem_bytes
    nb = -(-v.rows // tile_rows)
    deps = [set() for _ in range(nb)]
    for p, s in enumerate(schedules):
        if s is None:
            continue
        for c, ch in enumerate(s.chunks):
            for off, rows, row_bytes, rpitch in ch.regions:
                for i in range(rows):
                    for byte in range(off + i * rpitch, off + i * rpitch + row_bytes):
                        rel = byte - v.byte_offset
                        if rel < 0 or rel >= v.rows * pitch or rel % pitch >= v.cols * e:
                            continue
                        deps[(rel // pitch) // tile_rows].add((p, c))
    return [sorted(d) for d in deps]


def test_consumer_row_deps_bruteforce():
    from oracle import consumer as ocons
    rng = np.random.default_rng(11)
    for _ in range(40):
        P = int(rng.integers(1, 4))
        rows, cols = int(rng.integers(1, 10)), int(rng.integers(1, 9))
        e = int(rng.choice([1, 2, 4]))
        stride = cols + int(rng.integers(0, 3))
        scheds = []
        for p in range(P):
            v = schedule.View(p * rows * stride * e, rows, cols, stride, e)
            kind = int(rng.integers(0, 3))
            if kind == 0:
                scheds.append(schedule.whole(v, 1))
            elif kind == 1:
                scheds.append(schedule.chunks(v, int(rng.integers(1, rows + 1)), 1))
            else:
                scheds.append(schedule.tile_chunks(v, int(rng.integers(1, 4)), int(rng.integers(1, 4)),
                                                 int(rng.integers(1, 4)), None))
        gathered = schedule.View(0, P * rows, cols, stride, e)
        tr = int(rng.integers(1, 7))
        assert ocons.row_deps(scheds, gathered, tr) == _deps_brute(scheds, gathered, tr)


def test_consumer_row_deps_rank_blocks():
    # 128-row blocks over 4 ranks of 2000 rows each, one chunk per rank:
    # block b depends on the ranks whose rows [2000 p, 2000 (p+1)) meet
    # [128 b, 128 (b+1)) -- one rank, or two at a boundary.
    from oracle import consumer as ocons
    views = [schedule.View(p * 2000 * 64 * 2, 2000, 64, 64, 2) for p in range(4)]
    scheds = [schedule.whole(v, 1) for v in views]
    deps = ocons.row_deps(scheds, schedule.View(0, 8000, 64, 64, 2), 128)
    assert len(deps) == 63
    for b, d in enumerate(deps):
        r0, r1 = 128 * b, min(8000, 128 * (b + 1)) - 1
        assert d == [(p, 0) for p in range(r0 // 2000, r1 // 2000 + 1)]
