#!/usr/bin/env python
"""Benchmark of the triggered chunked all-gather on one MI355X.

A step is one round of the whole path on the 4-rank x 1.5 GiB workload
(per-rank u32 [786432, 512], three 0.5 GiB row-block chunks, 64 writers
each): the producer (a persistent grid taking the writer slots) writes
every rank's block, the round starts, the writers' marks open the gates, the copy engine delivers every chunk to the
three other replicas and signals its arrivals, wait() checks completion,
next_round() re-arms.  Marks are deferred (issued by a mark kernel after the
fill), so the copy engine's window holds no producer traffic.

Printed: one JSON line.  `value` = delivered bytes per step (P(P-1)S) / step
time.  `roofline` = the copy-engine kernel: algorithmic HBM bytes per launch
(P^2 S: every source byte read once, written P-1 times) / its mean launch
time from HIP events on the engine's stream.  Extras: the GEMM producer's
slowdown when the engine overlaps it, barrier and small-round latencies,
and the CPU oracle on a bounded sample.
"""

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "delivered all-gather GB/s and % of HBM peak; producer overlap slowdown %"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


# The code that decides the copy engine's traffic for a given schedule: the
# shared headers, plan.hip's device code and launch (everything before its
# host API, which starts at `using namespace tc;`), and the piece builder of
# schedule.cpp.  (file, first line containing, line after the end containing)
ENGINE_SOURCES = (("include/tc_device.h", None, None),
                  ("triggered_copy_amd/csrc/internal.h", None, None),
                  ("triggered_copy_amd/csrc/plan_internal.h", None, None),
                  ("triggered_copy_amd/csrc/plan.hip", None, "using namespace tc;"),
                  ("triggered_copy_amd/csrc/schedule.cpp", "void tc::build_pieces(", None))
TRAFFIC_PROFILE = "profiles/engine_kernel_u32_chunks_1p5g_p4_hbm_bytes.md"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def code_only(src):
    """C/C++ source without comments and with whitespace collapsed, so that
    editing a comment does not count as changing the kernel."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def engine_source_hash():
    """sha256 over the code (comments and whitespace removed) of the parts of
    ENGINE_SOURCES, in order."""
    import hashlib
    h = hashlib.sha256()
    for f, start, end in ENGINE_SOURCES:
        with open(os.path.join(ROOT, f)) as fh:
            text = fh.read()
        if start is not None:
            text = text[text.index(start):]
        if end is not None:
            text = text[:text.index(end)]
        h.update(code_only(text).encode())
    return h.hexdigest()


def counted_traffic(workload, engine_ctas, piece_bytes):
    """HBM bytes per engine launch from the committed FETCH_SIZE/WRITE_SIZE
    summary, or None when the engine sources or the launch differ from the
    ones the counters were taken on."""
    import re
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if workload != "u32_chunks_1p5g_p4" or engine_ctas != 1024 or piece_bytes != 8192:
        return None
    try:
        text = open(path).read()
        digest = engine_source_hash()
    except (OSError, ValueError):
        return None
    want = re.search(r"engine_source_sha256: ([0-9a-f]{64})", text)
    val = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    if not want or not val or want.group(1) != digest:
        return None
    return int(val.group(1))


def rank_setup(w, torch, tc):
    e = {"u32": 4, "bf16": 2, "u8": 1}[w["elem"]]
    P, rows, cols = w["P"], w["rows"], w["cols"]
    B = P * rows * cols * e
    views = [tc.View(p * rows * cols * e, rows, cols, cols, e, 0) for p in range(P)]
    rep = torch.full((P, B), 0xA5, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()       # producers run on other streams
    return views, rep, B


def build_sched(w, views, tc):
    if w["builder"] == "whole":
        return [tc.whole(v, w["writers"]) for v in views]
    if w["builder"] == "chunks":
        return [tc.chunks(v, w["n"], w["writers"]) for v in views]
    tm, tn = -(-w["rows"] // w["bm"]), -(-w["cols"] // w["bn"])
    order = tc.order_grouped(tm, tn, w["group_m"]) if w.get("group_m") else None
    return [tc.tile_chunks(v, (w["bm"], w["bn"]), w["tiles_per_chunk"], order=order) for v in views]


def run_headline(args, torch, tc, workloads, seed):
    w = workloads.FULL[args.workload]
    P = w["P"]
    views, rep, B = rank_setup(w, torch, tc)
    S = B // P
    scheds = build_sched(w, views, tc)
    plan = tc.TriggeredPlan(rep, scheds, engine_ctas=args.engine_ctas, piece_bytes=args.piece_bytes)
    prod = torch.cuda.Stream()
    engine_ms, window_ticks = [], []
    fill_kw = {args.fill: True}

    def step(record):
        h = plan.current_handle()
        plan.fill(h, views, seed, kind=w["elem"], mark=False, stream=prod, **fill_kw)
        if args.premark:
            # Profiling order: the marks precede start(), so no kernel ever
            # waits on a kernel queued after it (a profiler that runs kernels
            # one at a time cannot stall the engine).
            plan.mark_all(h, stream=prod)
            plan.start(prod)
        else:
            plan.start(prod)
            plan.mark_all(h, stream=prod)
        plan.wait(60.0)
        if record:
            st = plan.stats()
            engine_ms.append(st["engine_ms"])
            window_ticks.append(st["window_ticks"])
        plan.next_round()

    log(f"headline {args.workload}: P={P}, {S / 2**30:.2f} GiB per rank, warmup {args.warmup}")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    st = plan.stats()
    delivered = P * (P - 1) * S
    algo_bytes = P * P * S
    eng = statistics.mean(engine_ms)
    achieved = algo_bytes / (eng * 1e-3) / 1e9
    out = dict(ms_per_step=ms_per_step, value=delivered / (ms_per_step * 1e-3) / 1e9,
               engine_ms_mean=eng, engine_ms_median=statistics.median(engine_ms),
               engine_ms_min=min(engine_ms), achieved=achieved,
               engine_ms_p10=sorted(engine_ms)[len(engine_ms) // 10],
               engine_ms_p90=sorted(engine_ms)[(9 * len(engine_ms)) // 10],
               window_ms_median=statistics.median(window_ticks) / 1e5,
               engine_ctas=st["engine_ctas"], pieces=st["pieces"],
               piece_bytes=args.piece_bytes or 8192,
               delivered=delivered, algo_bytes=algo_bytes, S=S, P=P, w=w)

    # Full triggered rounds: the fill marks each chunk as its writers finish,
    # so copies overlap the production of later chunks.  The producer is the
    # persistent writer grid (every rank's chunk 0 first, then chunk 1, ...):
    # with the engine running beside it, it beats the one-shot grid.  Beside
    # the engine, 3 CTAs per CU (5.77-5.80 ms rounds) beat the fill's own
    # default of 2 (5.83-5.86), which is best for the fill alone.
    if not args.no_extras:
        times = []
        wave_ctas = 3 * torch.cuda.get_device_properties(0).multi_processor_count
        for i in range(max(3, args.steps // 4)):
            torch.cuda.synchronize()
            a = time.perf_counter()
            h = plan.start(prod)
            plan.fill(h, views, seed, kind=w["elem"], mark=True, waves=True, ctas=wave_ctas, stream=prod)
            plan.wait(60.0)
            plan.next_round()
            times.append(time.perf_counter() - a)
        out["overlapped_round_ms"] = statistics.median(times) * 1e3
        out["overlapped_delivered_gbs"] = delivered / statistics.median(times) / 1e9
    plan.close()
    del rep
    torch.cuda.empty_cache()
    return out


def overlap_mask(torch, ncus):
    """CU mask words selecting the first `ncus` CUs for the engine (None: all)."""
    if not ncus:
        return None
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    mask = [0] * ((ncu + 31) // 32)
    for i in range(min(ncus, ncu)):
        mask[i // 32] |= 1 << (i % 32)
    return mask


def queue_behind_sleep(torch, stream):
    """Occupies `stream` for about 80 us so that the launches the host makes
    next are all queued before the first of them runs: the events around
    them then time the device's back-to-back work, not the host's first
    launch (about 5 us of binding and runtime calls per kernel).  The GEMM
    overlap measurement does not use it: its round is timed on the host, and
    its three variants are timed alike."""
    with torch.cuda.stream(stream):
        torch.cuda._sleep(200_000)


def run_overlap(torch, tc, workloads, seed, reps=40, cu_mask=None, engine_ctas=0):
    """GEMM producer time for P ranks back to back, without any plan and with
    the copy engine delivering each rank's tiles while the next GEMM runs."""
    from synth import gemm_operands
    import numpy as np
    w = workloads.FULL["gemm_tiles_p4"]
    P, M, N, K = w["P"], w["rows"], w["cols"], w["K"]
    views, rep, B = rank_setup(w, torch, tc)
    ops = []
    for p in range(P):
        a, bt = gemm_operands(seed, p, 1, M, N, K)
        ops.append((torch.from_numpy(a.view(np.int16)).cuda(), torch.from_numpy(bt.view(np.int16)).cuda()))
    prod = torch.cuda.Stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def gemms(h):
        for p in range(P):
            tc.gemm_bf16(ops[p][0], ops[p][1], rep[p][p * M * N * 2:], ldc=N, M=M, N=N,
                         programs=w["programs"], group_m=w["group_m"], handle=h, rank=p,
                         first_chunk=0, tiles_per_chunk=w["tiles_per_chunk"], stream=prod)

    # Three variants, interleaved rep by rep so that clock or placement drift
    # hits all of them alike: the GEMMs with no plan; the same GEMMs marking
    # the gates of a throwaway plan whose round is never started (the cost of
    # the mark protocol alone); and full rounds with the copy engine running.
    scratch = tc.TriggeredPlan(rep, build_sched(w, views, tc), engine_ctas=1)
    h0 = scratch.current_handle()
    plan = tc.TriggeredPlan(rep, build_sched(w, views, tc), cu_mask=cu_mask, engine_ctas=engine_ctas)

    def timed(h):
        torch.cuda.synchronize()
        e0.record(prod)
        gemms(h)
        e1.record(prod)
        e1.synchronize()
        return e0.elapsed_time(e1)

    alone, marks_only, over, rounds = [], [], [], []
    for i in range(reps + 3):
        a_ms = timed(None)
        m_ms = timed(h0)
        torch.cuda.synchronize()
        a = time.perf_counter()
        h = plan.start(prod)
        e0.record(prod)
        gemms(h)
        e1.record(prod)
        plan.wait(30.0)
        plan.next_round()
        b = time.perf_counter()
        if i >= 3:
            alone.append(a_ms)
            marks_only.append(m_ms)
            over.append(e0.elapsed_time(e1))
            rounds.append((b - a) * 1e3)
    scratch.close()
    ectas = plan.stats()["engine_ctas"]
    plan.close()
    flops = 2.0 * M * N * K * P
    ma, mo = statistics.median(alone), statistics.median(over)
    mm = statistics.median(marks_only)
    return dict(gemm_ms_alone=ma, gemm_ms_marks_only=mm, gemm_ms_overlapped=mo,
                slowdown_pct=(mo / ma - 1) * 100,
                slowdown_vs_marks_only_pct=(mo / mm - 1) * 100,
                mark_protocol_cost_pct=(mm / ma - 1) * 100, engine_ctas=ectas,
                gemm_tflops_alone=flops / (ma * 1e-3) / 1e12,
                mfma_frac_alone=flops / (ma * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                round_ms=statistics.median(rounds),
                delivered_gbs=P * (P - 1) * (B // P) / (statistics.median(rounds) * 1e-3) / 1e9)


def run_consumer_overlap(torch, tc, workloads, seed, reps=20, N2=256):
    """The 4 GEMM producers' round followed by each rank's in-kernel consumer
    (Y_q = gathered rows of replica q [8000, 2000] x W [2000, 256]), two ways:
    consumers launched after wait() returns ("sequential"), and queued right
    behind the producers, waiting on the device for the chunks still being
    copied ("chained").  Chained consumers go on a stream of their own that
    waits for an event recorded after the producers: wait() learns that the
    producers' stream has drained as soon as the producers are done, so the
    engine runs the completion check while the consumers wait or compute."""
    from synth import gemm_operands
    import numpy as np
    w = workloads.FULL["gemm_tiles_p4"]
    P, M, N, K = w["P"], w["rows"], w["cols"], w["K"]
    views, rep, B = rank_setup(w, torch, tc)
    ops = []
    for p in range(P):
        a, bt = gemm_operands(seed, p, 1, M, N, K)
        ops.append((torch.from_numpy(a.view(np.int16)).cuda(), torch.from_numpy(bt.view(np.int16)).cuda()))
    R = P * M
    rng = np.random.default_rng(9)
    wt = torch.from_numpy((rng.standard_normal((N2, N)).astype(np.float32).view(np.uint32) >> 16)
                          .astype(np.uint16).view(np.int16)).cuda()
    plan = tc.TriggeredPlan(rep, build_sched(w, views, tc))
    start, pairs = plan.row_deps(tc.View(0, R, N, N, 2, 0), 128)
    ds = torch.from_numpy(start.astype(np.int32)).cuda()
    dp = torch.from_numpy(np.ascontiguousarray(pairs).astype(np.int32).reshape(-1)).cuda()
    Y = [torch.zeros(R * N2, dtype=torch.int16, device="cuda") for _ in range(P)]
    status = torch.zeros((P, len(start) - 1), dtype=torch.int32, device="cuda")
    prod = torch.cuda.Stream()
    cons = torch.cuda.Stream()
    produced = torch.cuda.Event()

    def producers(h):
        for p in range(P):
            tc.gemm_bf16(ops[p][0], ops[p][1], rep[p][p * M * N * 2:], ldc=N, M=M, N=N,
                         programs=w["programs"], group_m=w["group_m"], handle=h, rank=p,
                         first_chunk=0, tiles_per_chunk=w["tiles_per_chunk"], stream=prod)

    def consumers(h, stream, programs):
        for q in range(P):
            tc.gemm_consume_bf16(h, q, ds, dp, rep[q], wt, Y[q], M=R, N=N2, K=N, status=status[q],
                                 programs=programs, stream=stream)

    times = {"sequential": [], "chained": []}
    for i in range(reps + 2):
        for mode in times:
            torch.cuda.synchronize()
            a = time.perf_counter()
            h = plan.start(prod)
            producers(h)
            if mode == "chained":
                produced.record(prod)
                cons.wait_event(produced)
                consumers(h, cons, 256)
            plan.wait(30.0)
            if mode == "sequential":
                consumers(h, prod, 256)
            torch.cuda.synchronize()
            plan.next_round()
            b = time.perf_counter()
            if i >= 2:
                times[mode].append((b - a) * 1e3)
    bad = int((status != 0).sum().item())
    plan.close()
    flops = 2.0 * R * N2 * N * P
    med = {k: statistics.median(v) for k, v in times.items()}
    return dict(sequential_ms=med["sequential"], chained_ms=med["chained"],
                chained_saved_pct=(1 - med["chained"] / med["sequential"]) * 100,
                consumer_gflop=flops / 1e9, failed_waits=bad)


def run_placement_trials(torch, tc, workloads, seed, trials, rounds=6):
    """Copy-engine bandwidth on the headline workload for `trials` fresh
    allocations of the replicas (each freed before the next): where the
    driver places the replicas' pages in HBM changes the engine's rate."""
    w = workloads.FULL["u32_chunks_1p5g_p4"]
    P = w["P"]
    out = []
    for _ in range(trials):
        views, rep, B = rank_setup(w, torch, tc)
        plan = tc.TriggeredPlan(rep, build_sched(w, views, tc))
        prod = torch.cuda.Stream()
        ms = []
        for r in range(rounds):
            h = plan.current_handle()
            plan.fill(h, views, seed, kind=w["elem"], mark=False, stream=prod)
            plan.start(prod)
            plan.mark_all(h, stream=prod)
            plan.wait(60.0)
            if r >= 2:
                ms.append(plan.stats()["engine_ms"])
            plan.next_round()
        plan.close()
        del rep
        torch.cuda.empty_cache()
        out.append(round(P * B / (statistics.mean(ms) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
    return out


def run_gemm_only(torch, tc, workloads, seed, reps):
    """The P GEMM producers back to back with no plan, `reps` times, timed on
    the device (the launches queued behind a short sleep)."""
    from synth import gemm_operands
    import numpy as np
    w = workloads.FULL["gemm_tiles_p4"]
    P, M, N, K = w["P"], w["rows"], w["cols"], w["K"]
    ops = []
    for p in range(P):
        a, bt = gemm_operands(seed, p, 1, M, N, K)
        ops.append((torch.from_numpy(a.view(np.int16)).cuda(), torch.from_numpy(bt.view(np.int16)).cuda()))
    out = torch.zeros(P * M * N, dtype=torch.int16, device="cuda")
    prod = torch.cuda.Stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for i in range(reps + 2):
        torch.cuda.synchronize()
        queue_behind_sleep(torch, prod)
        e0.record(prod)
        for p in range(P):
            tc.gemm_bf16(ops[p][0], ops[p][1], out[p * M * N:], ldc=N, M=M, N=N,
                         programs=w["programs"], group_m=w["group_m"], stream=prod)
        e1.record(prod)
        e1.synchronize()
        if i >= 2:
            ts.append(e0.elapsed_time(e1))
    ms = statistics.median(ts)
    # The library GEMM (torch.mm, hipBLASLt) on the same operands and shape,
    # for context: C = A @ B with B given as its transpose Bt [N, K].
    bf = torch.bfloat16
    lib_out = [torch.empty(M, N, dtype=bf, device="cuda") for _ in range(P)]
    lts = []
    with torch.cuda.stream(prod):
        for i in range(reps + 2):
            torch.cuda.synchronize()
            queue_behind_sleep(torch, prod)
            e0.record(prod)
            for p in range(P):
                torch.mm(ops[p][0].view(bf).view(M, K), ops[p][1].view(bf).view(N, K).t(), out=lib_out[p])
            e1.record(prod)
            e1.synchronize()
            if i >= 2:
                lts.append(e0.elapsed_time(e1))
    lib_ms = statistics.median(lts)
    flops = 2.0 * M * N * K * P
    return {"metric": "bf16 GEMM producer (M=N=2000, K=1024, 4 ranks back to back)",
            "ms": ms, "tflops": flops / (ms * 1e-3) / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, "reps": reps,
            "library_mm_ms": lib_ms, "library_mm_tflops": flops / (lib_ms * 1e-3) / 1e12}


def run_barrier(torch, tc, workloads):
    w = workloads.FULL["barrier_p8"]
    P, G = w["P"], w["gens"]
    W = torch.zeros((P, P), dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    first, res = 1, []
    for i in range(4):
        e0.record(s)
        tc.barrier(W, P, first, G, status, stream=s)
        e1.record(s)
        e1.synchronize()
        first += G
        if i:
            res.append(e0.elapsed_time(e1) * 1e3 / G)
    assert int(status.item()) == 0
    return dict(us_per_generation=statistics.median(res), P=P, generations=G)


def run_small_round(torch, tc, workloads, seed, name, rounds, premark=False, oneshot=False):
    """Full rounds of a small workload: start, the fill with in-kernel marks,
    wait.  With premark (for counter collection, which runs kernels one at
    a time) the fill and its marks precede start().  The fill is one CTA per
    writer (the workload's producer as specified), or with oneshot one CTA
    per 16 KiB block, each writer's share still marked once."""
    w = workloads.FULL[name]
    views, rep, B = rank_setup(w, torch, tc)
    plan = tc.TriggeredPlan(rep, build_sched(w, views, tc))
    prod = torch.cuda.Stream()
    times = []
    for i in range(rounds + 5):
        a = time.perf_counter()
        if premark:
            h = plan.current_handle()
            plan.fill(h, views, seed, kind=w["elem"], mark=False, oneshot=oneshot, stream=prod)
            plan.mark_all(h, stream=prod)
            plan.start(prod)
        else:
            h = plan.start(prod)
            plan.fill(h, views, seed, kind=w["elem"], mark=True, oneshot=oneshot, stream=prod)
        plan.wait(30.0)
        plan.next_round()
        if i >= 5:
            times.append((time.perf_counter() - a) * 1e6)
    plan.close()
    P = w["P"]
    med = statistics.median(times)
    return dict(us_per_round_median=med, us_p10=sorted(times)[len(times) // 10],
                us_p90=sorted(times)[9 * len(times) // 10],
                delivered_gbs=P * (P - 1) * (B // P) / (med * 1e-6) / 1e9)


def cpu_baseline(workloads, seed, budget_s=12.0):
    """The oracle, as it stands, on a bounded sample of the headline workload:
    the same P, chunking and writers with 1/96 of the rows per rank."""
    import numpy as np
    from oracle import plan as oplan
    from oracle import schedule as osched
    from oracle import values as ovalues
    w = workloads.FULL["u32_chunks_1p5g_p4"]
    P, cols = w["P"], w["cols"]
    rows = w["rows"] // 96
    nb = rows * cols * 4
    ov = [osched.View(p * nb, rows, cols, cols, 4) for p in range(P)]
    reps = [np.full(P * nb, 0xA5, dtype=np.uint8) for _ in range(P)]
    sim = oplan.PlanSim(reps, [osched.chunks(v, w["n"], w["writers"]) for v in ov])

    def produce(p, r):
        sim.rep[p][p * nb:(p + 1) * nb] = ovalues.block_bytes("u32", seed, p, r, rows * cols)
    t0 = time.perf_counter()
    n = 0
    while True:
        oplan.run_round(sim, produce)
        sim.next_round()
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = (time.perf_counter() - t0) / n
    return {"value": P * (P - 1) * nb / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "s_per_round": dt,
            "sample": f"P={P}, {rows}x{cols} u32 per rank ({nb / 2**20:.0f} MiB, 1/96 of the rows), "
                      f"chunks({w['n']}), {w['writers']} writers, {n} full oracle rounds "
                      f"(produce + marks + in-order copies + wait) in {dt * n:.1f} s on one core"}


def oracle_per_config(workloads, seed, budget_s=2.0):
    """The oracle, as it stands, timed per workload on one host core: seconds
    per round (at least one round, then as many as fit in budget_s).  The
    small workloads run at their full sizes; the 1.5 GiB one is the sample
    that cpu_baseline times (its full-size figure is that scaled by the row
    ratio).  The GEMM workload's round is the plan simulation fed each
    rank's block, with the fp32 reference GEMMs timed beside it."""
    import numpy as np
    import torch
    from oracle import barrier as obarrier
    from oracle import gemm as ogemm
    from oracle import plan as oplan
    from oracle import schedule as osched
    from oracle import values as ovalues
    from synth import gemm_operands, shuffled_order
    e_of = {"u32": 4, "bf16": 2, "u8": 1}

    def timed(fn):
        t0 = time.perf_counter()
        n = 0
        while True:
            fn()
            n += 1
            if time.perf_counter() - t0 > budget_s:
                return (time.perf_counter() - t0) / n, n

    def sim_of(w):
        e = e_of[w["elem"]]
        P, rows, cols = w["P"], w["rows"], w["cols"]
        nb = rows * cols * e
        ov = [osched.View(p * nb, rows, cols, cols, e) for p in range(P)]
        if w["builder"] == "whole":
            sch = [osched.whole(v, w["writers"]) for v in ov]
        elif w["builder"] == "chunks":
            sch = [osched.chunks(v, w["n"], w["writers"]) for v in ov]
        else:
            tm, tn = -(-rows // w["bm"]), -(-cols // w["bn"])
            order = ([osched.tile_of(i, tm, tn, w["group_m"]) for i in range(tm * tn)]
                     if w.get("group_m") else None)
            sch = [osched.tile_chunks(v, w["bm"], w["bn"], w["tiles_per_chunk"], order) for v in ov]
        reps = [np.full(P * nb, 0xA5, dtype=np.uint8) for _ in range(P)]
        return oplan.PlanSim(reps, sch), nb

    def fill_round(name, order_of=None):
        w = workloads.FULL[name]
        sim, nb = sim_of(w)
        P, e = w["P"], e_of[w["elem"]]

        def produce(p, r):
            sim.rep[p][p * nb:(p + 1) * nb] = ovalues.block_bytes(w["elem"], seed, p, r, nb // e)

        def one():
            marks = order_of(sim) if order_of else None
            oplan.run_round(sim, produce, mark_order=marks)
            sim.next_round()
        dt, n = timed(one)
        return {"s_per_round": dt, "rounds": n, "delivered_bytes": P * (P - 1) * nb}

    out = {}
    threads = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        out["bf16_chunks_p2"] = fill_round("bf16_chunks_p2")
        out["u32_whole_p8"] = fill_round("u32_whole_p8")

        def shuffled(sim):
            n = max(sim.n)
            return [(p, int(c)) for p in range(sim.P) for c in shuffled_order(seed, p, sim.round, n)
                    for _ in range(sim.writers(p, int(c)))]
        out["u32_tiles_shuffled_p8"] = fill_round("u32_tiles_shuffled_p8", shuffled)

        w = workloads.FULL["gemm_tiles_p4"]
        P, M, N, K = w["P"], w["rows"], w["cols"], w["K"]
        sim, nb = sim_of(w)
        ops = [gemm_operands(seed, p, 1, M, N, K) for p in range(P)]
        t0 = time.perf_counter()
        refs = [ogemm.gemm_ref(a, bt) for a, bt in ops]
        ref_s = time.perf_counter() - t0
        blocks = [(r.view(np.uint32) >> np.uint32(16)).astype(np.uint16).view(np.uint8).reshape(-1)
                  for r in refs]

        def produce(p, r):
            sim.rep[p][p * nb:(p + 1) * nb] = blocks[p]

        def one():
            oplan.run_round(sim, produce)
            sim.next_round()
        dt, n = timed(one)
        out["gemm_tiles_p4"] = {"s_per_round": dt, "rounds": n, "delivered_bytes": P * (P - 1) * nb,
                                "fp32_reference_gemms_s": ref_s}

        wb = workloads.FULL["barrier_p8"]
        t0 = time.perf_counter()
        obarrier.run(wb["P"], wb["gens"])
        obarrier.reveal(wb["P"], 1, wb["gens"])
        out["barrier_p8"] = {"s_per_1000_generations": time.perf_counter() - t0}
    finally:
        torch.set_num_threads(threads)
    return out


def cpu_copy_baseline(workloads, sample_bytes=256 << 20, reps=5):
    """One GPU's share of the headline round done by host cores with
    numpy.copyto: a source block copied into P - 1 destinations, on one core
    and on every core the process may use (threads over slices).  A bounded
    sample of the 1.5 GiB block; reported as delivered GB/s.  Context only."""
    import concurrent.futures
    import numpy as np
    w = workloads.FULL["u32_chunks_1p5g_p4"]
    P = w["P"]
    src = np.frombuffer(np.random.default_rng(1).bytes(sample_bytes), dtype=np.uint8)
    dst = [np.empty(sample_bytes, dtype=np.uint8) for _ in range(P - 1)]
    cores = len(os.sched_getaffinity(0))

    def one(lo, hi):
        for d in dst:
            np.copyto(d[lo:hi], src[lo:hi])

    def timed(nthreads):
        step = -(-sample_bytes // nthreads)
        best = float("inf")
        with concurrent.futures.ThreadPoolExecutor(max_workers=nthreads) as ex:
            for _ in range(reps):
                t0 = time.perf_counter()
                list(ex.map(lambda i: one(i * step, min(sample_bytes, (i + 1) * step)), range(nthreads)))
                best = min(best, time.perf_counter() - t0)
        return (P - 1) * sample_bytes / best / 1e9

    return {"unit": "GB/s", "one_core": round(timed(1), 2), "all_cores": round(timed(cores), 2),
            "cores": cores, "kind": "numpy.copyto",
            "sample": f"{sample_bytes >> 20} MiB source copied to {P - 1} destinations, best of {reps}"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="u32_chunks_1p5g_p4")
    ap.add_argument("--engine-ctas", type=int, default=0)
    ap.add_argument("--piece-bytes", type=int, default=0)
    ap.add_argument("--overlap-engine-ctas", type=int, default=0)
    ap.add_argument("--overlap-cus", type=int, default=0,
                    help="confine the copy engine of the GEMM overlap run to the first N CUs "
                         "(0: every CU, shared with the producer)")
    ap.add_argument("--placement-trials", type=int, default=0,
                    help="also measure the copy engine on N fresh allocations of the replicas")
    ap.add_argument("--gemm-only", action="store_true",
                    help="time only the 4 GEMM producers, with no plan (for counter collection)")
    ap.add_argument("--fill", choices=("waves", "oneshot"), default="oneshot",
                    help="producer grid of the headline step: persistent writers or one CTA per 16 KiB block")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--premark", action="store_true",
                    help="issue the marks before start() (for counter collection)")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run an elementwise kernel reading and writing 1 GiB each, "
                         "the reference for scaling HBM byte counters")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--overlap-only", action="store_true",
                    help="time only the GEMM producers with and without the copy engine")
    ap.add_argument("--small-round", default=None, metavar="WORKLOAD",
                    help="time only full rounds (start, fill with in-kernel marks, wait) of a small "
                         "workload, --steps rounds (for per-kernel traces and counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the P ranks of the "
              "all-gather are simulated as P replicas in one GPU's HBM.", file=sys.stderr)
        sys.exit(2)
    import torch
    import triggered_copy_amd as tc
    from synth import BASE_SEED, workloads
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    tc.lib()
    if args.gemm_only:
        print(json.dumps(run_gemm_only(torch, tc, workloads, BASE_SEED, args.steps)), flush=True)
        return
    if args.overlap_only:
        r = run_overlap(torch, tc, workloads, BASE_SEED, cu_mask=overlap_mask(torch, args.overlap_cus),
                        engine_ctas=args.overlap_engine_ctas)
        r["engine_cus"] = args.overlap_cus or "all"
        print(json.dumps(r), flush=True)
        return

    if args.calibrate:
        x = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            torch.add(x, 1.0, out=y)
        torch.cuda.synchronize()
        del x, y
        torch.cuda.empty_cache()
    if args.small_round:
        r = run_small_round(torch, tc, workloads, BASE_SEED, args.small_round, args.steps,
                            premark=args.premark)
        print(json.dumps(dict(workload=args.small_round, rounds=args.steps, **r)), flush=True)
        return
    h = run_headline(args, torch, tc, workloads, BASE_SEED)
    w = h["w"]
    extras = {}
    if not args.no_extras:
        log("overlap: 4 GEMM producers with and without the copy engine")
        extras["gemm_overlap"] = run_overlap(torch, tc, workloads, BASE_SEED,
                                             cu_mask=overlap_mask(torch, args.overlap_cus),
                                             engine_ctas=args.overlap_engine_ctas)
        extras["gemm_overlap"]["engine_cus"] = args.overlap_cus or "all"
        # The same rounds with a smaller engine (122 CTAs, one wave per 192 KiB
        # delivered): less copying beside the producers, a longer round.
        log("overlap: the same with 122 engine CTAs")
        extras["gemm_overlap_122"] = run_overlap(torch, tc, workloads, BASE_SEED,
                                                 cu_mask=overlap_mask(torch, args.overlap_cus),
                                                 engine_ctas=122)
        log("GEMM producers alone, device-timed, and the library GEMM")
        extras["gemm_only"] = run_gemm_only(torch, tc, workloads, BASE_SEED, 100)
        log("in-kernel consumers: after wait() vs waiting on the device")
        extras["gemm_consumer"] = run_consumer_overlap(torch, tc, workloads, BASE_SEED)
        log("barrier: 8 ranks x 1000 generations")
        extras["barrier_p8"] = run_barrier(torch, tc, workloads)
        log("small rounds")
        extras["bf16_chunks_p2_round"] = run_small_round(torch, tc, workloads, BASE_SEED, "bf16_chunks_p2", 200)
        extras["u32_whole_p8_round"] = run_small_round(torch, tc, workloads, BASE_SEED, "u32_whole_p8", 50)
        extras["bf16_chunks_p2_round_oneshot_fill"] = run_small_round(
            torch, tc, workloads, BASE_SEED, "bf16_chunks_p2", 200, oneshot=True)
        extras["u32_whole_p8_round_oneshot_fill"] = run_small_round(
            torch, tc, workloads, BASE_SEED, "u32_whole_p8", 50, oneshot=True)
        extras["overlapped_triggered_round"] = {"ms": h.get("overlapped_round_ms"),
                                                "delivered_gbs": h.get("overlapped_delivered_gbs")}
        if args.workload == "u32_chunks_1p5g_p4":
            # The same buffers as one whole() chunk per rank: regions of 1 GiB
            # and 0.5 GiB (the 1 GiB split), 192 writers.
            log("the 1.5 GiB workload as whole(): 1 GiB + 0.5 GiB regions")
            import copy
            a2 = copy.copy(args)
            a2.workload, a2.steps, a2.warmup, a2.no_extras, a2.premark = \
                "u32_whole_1p5g_p4", 5, 1, True, False
            hw = run_headline(a2, torch, tc, workloads, BASE_SEED)
            extras["u32_whole_1p5g_p4"] = {
                "value_gbs": round(hw["value"], 2), "ms_per_step": round(hw["ms_per_step"], 4),
                "engine_ms_mean": round(hw["engine_ms_mean"], 4),
                "engine_frac": round(hw["achieved"] / HBM_PEAK_GBS, 4), "engine_ctas": hw["engine_ctas"]}
    if args.placement_trials:
        log(f"copy engine on {args.placement_trials} fresh replica allocations")
        extras["engine_frac_per_allocation"] = run_placement_trials(torch, tc, workloads, BASE_SEED,
                                                                     args.placement_trials)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: the oracle on a bounded sample")
        cpu = cpu_baseline(workloads, BASE_SEED)
        log("cpu baseline: the oracle per workload, one core")
        per = oracle_per_config(workloads, BASE_SEED)
        per["u32_chunks_1p5g_p4"] = {"s_per_round_sample": cpu["s_per_round"],
                                     "s_per_round_full_estimate": cpu["s_per_round"] * 96,
                                     "sample": "1/96 of the rows"}
        cpu["per_config"] = per
        cpu.pop("s_per_round")
        log("cpu copy baseline: numpy.copyto of one GPU's share, sampled")
        extras["cpu_copy_baseline"] = cpu_copy_baseline(workloads)
    line = {
        "metric": METRIC,
        "value": round(h["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": args.workload, "P": w["P"], "bytes_per_rank": h["S"],
                   "builder": w["builder"], "chunks": w.get("n", 1), "writers": w["writers"],
                   "marks": "deferred (fill, start, mark kernel)", "fill": args.fill,
                   "engine_ctas": h["engine_ctas"], "pieces_per_round": h["pieces"]},
        "roofline": {"bound": "hbm", "achieved": round(h["achieved"], 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(h["achieved"] / HBM_PEAK_GBS, 4),
                     "traffic": counted_traffic(args.workload, h["engine_ctas"], h["piece_bytes"]),
                     "kernel": "engine_kernel", "algo_bytes_per_launch": h["algo_bytes"],
                     "launch_ms_mean": round(h["engine_ms_mean"], 4),
                     "launch_ms_median": round(h["engine_ms_median"], 4),
                     "launch_ms_p10": round(h["engine_ms_p10"], 4),
                     "launch_ms_p90": round(h["engine_ms_p90"], 4)},
        "hbm_frac": round(h["achieved"] / HBM_PEAK_GBS, 4),
        "engine_window_ms_median": round(h["window_ms_median"], 4),
        "overlap_slowdown_pct": (round(extras["gemm_overlap"]["slowdown_pct"], 2)
                                 if "gemm_overlap" in extras else None),
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
