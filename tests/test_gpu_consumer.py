"""GPU parity of the in-kernel consumer: a GEMM over every rank's replica of
the gathered rows, queued right behind its producers, waiting on the device
per 128-row block for the chunks those rows hold while the copy engine is
still delivering them.  The result must equal the
fp32 reference on the gathered rows of the same round (stale rows from the
round before, or the sentinel, would not), and every wait must succeed.  The
row dependencies the library computes must contain the oracle's exact set.
"""

import numpy as np
import pytest
import torch

import triggered_copy_amd as tc
from oracle import consumer as ocons
from oracle import gemm as ogemm
from oracle import schedule as osched
from synth import BASE_SEED, gemm_operands, workloads
from tests.gpu_common import Pair, log

pytestmark = pytest.mark.gpu

SMALL_CU_SHARE = 64   # consumer programs for the small case


def _deps_device(pair, gathered_tv, gathered_ov):
    start, pairs = pair.plan.row_deps(gathered_tv, 128)
    exact = ocons.row_deps(pair.os, gathered_ov, 128)
    assert len(start) == len(exact) + 1
    for b, want in enumerate(exact):
        got = sorted(tuple(int(x) for x in pr) for pr in pairs[start[b]:start[b + 1]])
        assert got == want, f"row block {b}: library {got} vs oracle {want}"
    return (torch.from_numpy(start.astype(np.int32)).cuda(),
            torch.from_numpy(np.ascontiguousarray(pairs).astype(np.int32).reshape(-1)).cuda())


def _check_outputs(Y, status, X_bits, wt_bits, what):
    assert int(status.sum().item()) == 0, f"{what}: a wait ran out of polls: {status.tolist()}"
    ref = ogemm.gemm_ref(X_bits, wt_bits)
    for q, y in enumerate(Y):
        got = ogemm.bf16_bits_to_f32(y.cpu().numpy().view(np.uint16)).reshape(ref.shape)
        ok, worst, rel = ogemm.within_tolerance(got, ref, 1e-2)
        assert ok, f"{what}: consumer of rank {q}: worst {worst}, relative Frobenius {rel}"


def test_consumer_waits_for_filled_tiles():
    # Ragged bf16 tiles filled by the hash producer; 231 gathered rows, 2 row blocks.
    w = dict(P=3, rows=77, cols=64, elem="bf16", builder="tile_chunks", bm=32, bn=32,
             tiles_per_chunk=3, rounds=2)
    pair = Pair(w)
    try:
        R, K, N = 3 * 77, 64, 40
        gtv = tc.View(0, R, K, K, 2, 0)
        gov = osched.View(0, R, K, K, 2)
        ds, dp = _deps_device(pair, gtv, gov)
        rng = np.random.default_rng(5)
        wt_bits = (rng.standard_normal((N, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        wt = torch.from_numpy(wt_bits.view(np.int16)).cuda()
        for r in (1, 2):
            log(f"consumer after fill, round {r}")
            Y = [torch.zeros(R * N, dtype=torch.int16, device="cuda") for _ in range(3)]
            status = torch.zeros((3, len(ds) - 1), dtype=torch.int32, device="cuda")
            torch.cuda.synchronize()
            h = pair.plan.start(pair.stream)
            pair.plan.fill(h, pair.tv, pair.seed, kind="bf16", stream=pair.stream)
            for q in range(3):   # behind the producer: they wait for the engine's copies
                tc.gemm_consume_bf16(h, q, ds, dp, pair.rep[q], wt, Y[q], M=R, N=N, K=K,
                                     status=status[q], programs=SMALL_CU_SHARE, stream=pair.stream)
            pair.plan.wait(10.0)
            torch.cuda.synchronize()
            pair.oracle_round()
            pair.compare(f"consumer round {r}")
            X_bits = pair.sim.rep[0][:R * K * 2].view(np.uint16).reshape(R, K)
            _check_outputs(Y, status, X_bits, wt_bits, f"round {r}")
            pair.plan.next_round()
            pair.sim.next_round()
    finally:
        pair.close()


@pytest.mark.parametrize("consumer_stream", ["producers", "own"])
def test_consumer_of_gemm_producers(consumer_stream):
    # The 4-rank GEMM producer workload; each rank's consumer multiplies the
    # gathered [8000, 2000] rows by a [2000, 256] weight while the producers
    # and the copy engine still run.  The consumers go on the producers'
    # stream, or on a stream of their own behind an event recorded after the
    # producers (so that wait() sees the producers' stream drain as soon as
    # the producers end).
    w = workloads.FULL["gemm_tiles_p4"]
    P, M, N, K = w["P"], w["rows"], w["cols"], w["K"]
    pair = Pair(w, oracle_bytes=False)
    try:
        R, N2 = P * M, 256
        gtv = tc.View(0, R, N, N, 2, 0)
        gov = osched.View(0, R, N, N, 2)
        ds, dp = _deps_device(pair, gtv, gov)
        rng = np.random.default_rng(9)
        wt_bits = (rng.standard_normal((N2, N)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        wt = torch.from_numpy(wt_bits.view(np.int16)).cuda()
        ops = []
        for p in range(P):
            a, bt = gemm_operands(BASE_SEED, p, 1, M, N, K)
            ops.append((torch.from_numpy(a.view(np.int16)).cuda(), torch.from_numpy(bt.view(np.int16)).cuda()))
        Y = [torch.zeros(R * N2, dtype=torch.int16, device="cuda") for _ in range(P)]
        status = torch.zeros((P, len(ds) - 1), dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        h = pair.plan.start(pair.stream)
        for p in range(P):
            tc.gemm_bf16(ops[p][0], ops[p][1], pair.rep[p][p * M * N * 2:], ldc=N, M=M, N=N,
                         programs=w["programs"], group_m=w["group_m"], handle=h, rank=p,
                         first_chunk=0, tiles_per_chunk=w["tiles_per_chunk"], stream=pair.stream)
        cons = pair.stream
        if consumer_stream == "own":
            cons = torch.cuda.Stream()
            produced = torch.cuda.Event()
            produced.record(pair.stream)
            cons.wait_event(produced)
        log(f"GEMM producers, consumers on the {consumer_stream} stream")
        for q in range(P):
            tc.gemm_consume_bf16(h, q, ds, dp, pair.rep[q], wt, Y[q], M=R, N=N2, K=N,
                                 status=status[q], programs=256, stream=cons)
        pair.plan.wait(30.0)
        torch.cuda.synchronize()
        # The gathered rows: each rank's own block as its producer wrote it.
        host = pair.rep.cpu().numpy()
        X_bits = np.concatenate([host[p][p * M * N * 2:(p + 1) * M * N * 2].view(np.uint16)
                                 for p in range(P)]).reshape(R, N)
        for q in range(P):
            assert np.array_equal(host[q][:R * N * 2].view(np.uint16).reshape(R, N), X_bits), \
                f"replica {q} is not the gathered rows"
        _check_outputs(Y, status, X_bits, wt_bits, "GEMM producers")
    finally:
        pair.close()


def test_row_deps_random_schedules():
    # The library's dependency lists against the oracle's exact sets, on
    # random small schedules (strided views, 1-D and 2-D pieces, small
    # pieces that split regions) and random block heights.
    rng = np.random.default_rng(21)
    for trial in range(12):
        P = int(rng.integers(1, 5))
        rows, cols = int(rng.integers(1, 40)), int(rng.integers(1, 48))
        e = int(rng.choice([1, 2, 4]))
        stride = cols + int(rng.integers(0, 4))
        w = dict(P=P, rows=rows, cols=cols, stride=stride, elem={1: "u8", 2: "bf16", 4: "u32"}[e],
                 builder="whole", writers=1, rounds=1)
        pair = Pair(w, oracle_bytes=False, piece_bytes=int(rng.choice([256, 512, 8192])))
        try:
            ts, os_ = [], []
            for p in range(P):
                kind = int(rng.integers(0, 3))
                if kind == 0:
                    ts.append(tc.whole(pair.tv[p], 1))
                    os_.append(osched.whole(pair.ov[p], 1))
                elif kind == 1:
                    n = int(rng.integers(1, rows + 1))
                    ts.append(tc.chunks(pair.tv[p], n, 1))
                    os_.append(osched.chunks(pair.ov[p], n, 1))
                else:
                    bm, bn, tpc = int(rng.integers(1, 9)), int(rng.integers(1, 9)), int(rng.integers(1, 4))
                    ts.append(tc.tile_chunks(pair.tv[p], (bm, bn), tpc))
                    os_.append(osched.tile_chunks(pair.ov[p], bm, bn, tpc, None))
            pair.plan.close()
            pair.plan = tc.TriggeredPlan(pair.rep, ts, backstop_s=20.0)
            pair.os = os_
            tr = int(rng.integers(1, 20))
            gtv = tc.View(0, P * rows, cols, stride, e, 0)
            gov = osched.View(0, P * rows, cols, stride, e)
            start, pairs = pair.plan.row_deps(gtv, tr)
            exact = ocons.row_deps(os_, gov, tr)
            assert len(start) == len(exact) + 1
            for b, want in enumerate(exact):
                got = sorted(tuple(int(x) for x in pr) for pr in pairs[start[b]:start[b + 1]])
                assert got == want, f"trial {trial} block {b}: {got} vs {want}"
        finally:
            pair.close()
