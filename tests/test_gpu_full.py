"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses.

* GEMM producer: within rtol 1e-2 of the fp32 CPU reference; replicas,
  gates and cursors bit-exact against the oracle fed each rank's GPU block.
* 8 ranks x 4 MiB whole chunk, 8 writers, 10 rounds; the extra-mark run.
* 4 ranks x 1.5 GiB (chunks of 0.5 GiB; one whole chunk cut at 1 GiB):
  replicas compared with each other in full, and every element of replica 0
  with the oracle's values (streamed from the oracle's C twin of its value
  hash); gates and cursors bit-exact against the counters-only oracle.
* 8 ranks of 2-D tiles completed in a shuffled order, stepped one chunk at a
  time: after every step the gates equal the oracle's (head-of-line order).
"""

import numpy as np
import pytest
import torch

import triggered_copy_amd as tc
from oracle import cvalues
from oracle import gemm as ogemm
from oracle import plan as oplan
from synth import BASE_SEED, gemm_operands, workloads
from tests.gpu_common import Pair, log, oracle_produce, require_gpu, wait_until

pytestmark = pytest.mark.gpu


def _u16_to_dev(a):
    return torch.from_numpy(a.view(np.int16)).cuda()


@pytest.mark.parametrize("M,N,K,programs,group_m", [(300, 264, 128, 7, 2), (2000, 2000, 1024, 256, 8),
                                                    (128, 128, 64, 1, 1), (1, 8, 8, 3, 8)])
def test_gemm_matches_reference(M, N, K, programs, group_m):
    require_gpu()
    log(f"gemm {M}x{N}x{K} programs={programs}")
    a, bt = gemm_operands(BASE_SEED, 0, 1, M, N, K)
    C_out = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    tc.gemm_bf16(_u16_to_dev(a), _u16_to_dev(bt), C_out, programs=programs, group_m=group_m)
    torch.cuda.synchronize()
    got = ogemm.bf16_bits_to_f32(C_out.cpu().numpy().view(np.uint16))
    ok, worst, frob = ogemm.within_tolerance(got, ogemm.gemm_ref(a, bt), 1e-2)
    assert ok, (worst, frob)


def test_gemm_checks_operand_memory():
    # Operands are checked on the host before the launch: a C in host memory
    # is refused, and so is a shape whose rows run past an operand's
    # allocation (M far beyond what A holds).
    require_gpu()
    M, N, K = 64, 64, 64
    a, bt = gemm_operands(BASE_SEED, 0, 1, M, N, K)
    A, Bt = _u16_to_dev(a), _u16_to_dev(bt)
    host_c = torch.zeros((M, N), dtype=torch.int16).pin_memory()
    with pytest.raises(tc.InvalidArgument):
        tc.gemm_bf16(A, Bt, host_c)
    C_out = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    with pytest.raises(tc.BoundsError):
        tc.gemm_bf16(A, Bt, C_out, M=(1 << 32) - 1)
    tc.gemm_bf16(A, Bt, C_out)
    torch.cuda.synchronize()
    got = ogemm.bf16_bits_to_f32(C_out.cpu().numpy().view(np.uint16))
    ok, worst, frob = ogemm.within_tolerance(got, ogemm.gemm_ref(a, bt), 1e-2)
    assert ok, (worst, frob)


def test_gemm_tiles_p4_full():
    w = workloads.FULL["gemm_tiles_p4"]
    pair = Pair(w)
    P, M, N, K = w["P"], w["rows"], w["cols"], w["K"]
    try:
        for r in range(1, w["rounds"] + 1):
            log(f"gemm_tiles_p4 round {r}")
            ops = [gemm_operands(BASE_SEED, p, r, M, N, K) for p in range(P)]
            dev = [(_u16_to_dev(a), _u16_to_dev(bt)) for a, bt in ops]
            torch.cuda.synchronize()
            h = pair.plan.start(pair.stream)
            for p in range(P):
                C_out = pair.rep[p][p * M * N * 2:]
                tc.gemm_bf16(dev[p][0], dev[p][1], C_out, ldc=N, M=M, N=N, programs=w["programs"],
                             group_m=w["group_m"], handle=h, rank=p, first_chunk=0,
                             tiles_per_chunk=w["tiles_per_chunk"], stream=pair.stream)
            pair.plan.wait(20.0)
            torch.cuda.synchronize()
            host = pair.rep.cpu().numpy()
            blocks = []
            for p in range(P):
                blk = host[p][p * M * N * 2:(p + 1) * M * N * 2]
                got = ogemm.bf16_bits_to_f32(blk.view(np.uint16).reshape(M, N))
                ok, worst, frob = ogemm.within_tolerance(got, ogemm.gemm_ref(*ops[p]), 1e-2)
                assert ok, (p, worst, frob)
                blocks.append(blk.copy())

            def produce(p, rr):   # the oracle is fed each rank's GPU block
                pair.sim.rep[p][p * M * N * 2:(p + 1) * M * N * 2] = blocks[p]
            oplan.run_round(pair.sim, produce)
            pair.compare(f"gemm_tiles_p4 round {r}")
            pair.plan.next_round()
            pair.sim.next_round()
    finally:
        pair.close()


def test_u32_whole_p8_ten_rounds():
    w = workloads.FULL["u32_whole_p8"]
    pair = Pair(w)
    try:
        for r in range(1, w["rounds"] + 1):
            log(f"u32_whole_p8 round {r}")
            pair.gpu_round_fill()
            pair.oracle_round()
            pair.compare(f"u32_whole_p8 round {r}")
            if r < w["rounds"]:
                pair.plan.next_round()
                pair.sim.next_round()
        g = pair.plan.gates().view(np.uint64).reshape(w["P"], -1, 8)
        for p in range(w["P"]):
            assert (int(g[p, p, 2]), int(g[p, p, 0])) == (80, 10)
            assert all(int(g[q, p, 1]) == 10 for q in range(w["P"]) if q != p)
    finally:
        pair.close()


def test_u32_whole_p8_extra_mark_round7():
    w = workloads.FULL["u32_whole_p8"]
    pair = Pair(w)
    er, rank = w["extra_round"], w["extra_rank"]
    try:
        for r in range(1, er + 1):
            log(f"u32_whole_p8 extra-mark run round {r}")
            h = pair.plan.start(pair.stream)
            pair.plan.fill(h, pair.tv, pair.seed, kind="u32", stream=pair.stream)
            if r < er:
                pair.plan.wait(10.0)
                pair.oracle_round()
                pair.compare(f"extra-mark run round {r}")
                pair.plan.next_round()
                pair.sim.next_round()
                continue
            pair.plan.mark(h, rank, 0, 1, stream=pair.stream)
            with pytest.raises(tc.ExtraMarksError) as ei:
                pair.plan.wait(10.0)
            with pytest.raises(oplan.PlanError) as eo:
                pair.oracle_round(extra=[(rank, 0)])
            assert ei.value.chunks == eo.value.chunks == [(rank, 0)]
            assert pair.plan.state == "FAILED"
            torch.cuda.synchronize()
            assert np.array_equal(pair.plan.gates(), pair.sim.gate_bytes())
            g = pair.plan.gates().view(np.uint64).reshape(w["P"], -1, 8)
            assert int(g[rank, rank, 2]) == 8 * er + 1
    finally:
        pair.close()


class _FullCheck:
    """Every element of every rank's block against the oracle's values,
    streamed in slices of 2^26 elements: replica 0's words are read back
    into pinned host memory while the C oracle (oracle/values.c) writes the
    expected words of the same slice, so host memory stays bounded.  The
    other replicas are compared with replica 0 in full on the device."""

    SLICE = 1 << 26

    def __init__(self):
        self.got = torch.empty(self.SLICE, dtype=torch.int32).pin_memory()
        self.want = np.empty(self.SLICE, dtype=np.uint32)
        self.neq = np.empty(self.SLICE, dtype=bool)

    def __call__(self, pair, w, r):
        P, rows, cols = w["P"], w["rows"], w["cols"]
        n = rows * cols
        for q in range(1, P):
            assert torch.equal(pair.rep[0], pair.rep[q]), f"replica {q} differs from replica 0"
        words = pair.rep[0].view(torch.int32)
        got_np = self.got.numpy().view(np.uint32)
        for p in range(P):
            for lo in range(0, n, self.SLICE):
                k = min(self.SLICE, n - lo)
                self.got[:k].copy_(words[p * n + lo:p * n + lo + k])
                cvalues.u32_pattern_into(self.want[:k], pair.seed, p, r, lo)
                np.not_equal(got_np[:k], self.want[:k], out=self.neq[:k])
                if self.neq[:k].any():
                    bad = np.flatnonzero(self.neq[:k])
                    raise AssertionError(f"round {r}, rank {p}: {bad.size} elements differ from the "
                                         f"oracle, first at index {lo + int(bad[0])}")


@pytest.mark.parametrize("oneshot", [False, True], ids=["writer_ctas", "oneshot"])
@pytest.mark.parametrize("name", ["u32_chunks_1p5g_p4", "u32_whole_1p5g_p4"])
def test_u32_1p5g_p4_full(name, oneshot):
    # Writer CTAs (one per writer slot) or the one-shot grid (one CTA per
    # 16 KiB block, the share's last block marking), at the full size.
    w = workloads.FULL[name]
    check = _FullCheck()
    pair = Pair(w, oracle_bytes=False)
    try:
        for r in range(1, w["rounds"] + 1):
            deferred = r == 2
            log(f"{name} round {r} ({'deferred' if deferred else 'in-kernel'} marks, oneshot={oneshot})")
            pair.gpu_round_fill(mark=not deferred, timeout=30.0, oneshot=oneshot)
            pair.oracle_round()
            pair.compare(f"{name} round {r}")
            check(pair, w, r)
            log(f"{name} round {r}: every element of the 4 x 1.5 GiB blocks equals the oracle's")
            pair.plan.next_round()
            pair.sim.next_round()
    finally:
        pair.close()


def test_u32_tiles_shuffled_p8_rounds():
    w = workloads.FULL["u32_tiles_shuffled_p8"]
    pair = Pair(w)
    try:
        for r in range(1, w["rounds"] + 1):
            log(f"u32_tiles_shuffled_p8 round {r}")
            orders, dev = pair.orders_device(r)
            pair.gpu_round_fill(serial=True, order=dev, order_stride=orders.shape[1])
            mark_order = [(p, int(c)) for p in range(pair.P) for c in orders[p]
                          for _ in range(pair.sim.writers(p, int(c)))]
            pair.oracle_round(mark_order=mark_order)
            pair.compare(f"shuffled round {r}")
            pair.plan.next_round()
            pair.sim.next_round()
    finally:
        pair.close()


def _random_builder_workload(rng):
    P = int(rng.integers(2, 6))
    elem = str(rng.choice(["u8", "bf16", "u32"]))
    rows, cols = int(rng.integers(5, 48)), int(rng.integers(5, 70))
    w = dict(P=P, rows=rows, cols=cols, elem=elem, rounds=2)
    if rng.random() < 0.4:
        w["stride"] = cols + int(rng.integers(1, 9))
    b = int(rng.integers(0, 3))
    if b == 0:
        w.update(builder="whole", writers=int(rng.integers(1, 4)))
    elif b == 1:
        w.update(builder="chunks", n=int(rng.integers(1, min(rows, 6) + 1)), writers=int(rng.integers(1, 4)))
    else:
        w.update(builder="tile_chunks", bm=int(rng.integers(4, 20)), bn=int(rng.integers(4, 24)),
                 tiles_per_chunk=int(rng.integers(1, 5)))
        if rng.random() < 0.5:
            w["group_m"] = int(rng.integers(1, 4))
    return w


@pytest.mark.parametrize("case", range(16))
def test_random_builders_marked_one_at_a_time(case):
    # Random views (u8/bf16/u32, padded strides), builders, writer counts and
    # tile orders; every mark of the round issued on its own, in a seeded
    # random order across ranks and chunks.  After each mark the gate rows
    # and queue cursors must equal the oracle's (a gate opens only on its
    # last writer's mark; arrivals only in schedule order); after each round
    # the replicas are compared byte for byte.
    rng = np.random.default_rng(500 + case)
    w = _random_builder_workload(rng)
    pair = Pair(w, seed=BASE_SEED + 77 * case, engine_ctas=int(rng.integers(1, 9)))
    try:
        for r in (1, 2):
            h = pair.plan.start(pair.stream)
            pair.plan.fill(h, pair.tv, pair.seed, kind=w["elem"], mark=False, stream=pair.stream)
            pair.sim.start()
            for p in range(pair.P):
                oracle_produce(pair.sim.rep[p], pair.ov[p], w["elem"], pair.seed, p, r)
            marks = [(p, c) for p in range(pair.P) for c in range(pair.sim.n[p])
                     for _ in range(pair.sim.writers(p, c))]
            marks = [marks[i] for i in rng.permutation(len(marks))]
            log(f"random builders case {case} round {r}: {w} engine, {len(marks)} single marks")
            for p, c in marks:
                pair.plan.mark(h, p, c, 1, stream=pair.stream)
                pair.sim.mark(p, c)
                want_g = pair.sim.gate_bytes()
                ok = wait_until(lambda: np.array_equal(pair.plan.cursors(), pair.sim.cur)
                                and np.array_equal(pair.plan.gates(), want_g), 5.0)
                assert ok, f"case {case} round {r} after mark ({p},{c})"
            pair.plan.wait(10.0)
            pair.sim.wait()
            pair.compare(f"random builders case {case} round {r}")
            pair.plan.next_round()
            pair.sim.next_round()
    finally:
        pair.close()


def test_head_of_line_stepped_p8():
    w = workloads.FULL["u32_tiles_shuffled_p8"]
    pair = Pair(w)
    try:
        for r in (1, 2):
            orders, _ = pair.orders_device(r)
            h = pair.plan.start(pair.stream)
            pair.plan.fill(h, pair.tv, pair.seed, kind="u32", mark=False, stream=pair.stream)
            pair.sim.start()
            for p in range(pair.P):
                oracle_produce(pair.sim.rep[p], pair.ov[p], "u32", pair.seed, p, r)
            n = orders.shape[1]
            for k in range(n):
                for p in range(pair.P):
                    c = int(orders[p][k])
                    wr = pair.sim.writers(p, c)
                    pair.plan.mark(h, p, c, wr, stream=pair.stream)
                    for _ in range(wr):
                        pair.sim.mark(p, c)
                    want_g = pair.sim.gate_bytes()
                    ok = wait_until(lambda: np.array_equal(pair.plan.cursors(), pair.sim.cur)
                                    and np.array_equal(pair.plan.gates(), want_g), 5.0)
                    assert ok, f"round {r} step ({p},{c}): cursors {pair.plan.cursors()[p].tolist()} " \
                               f"vs oracle {pair.sim.cur[p].tolist()}"
            log(f"head-of-line round {r}: {n * pair.P} steps matched")
            pair.plan.wait(10.0)
            pair.sim.wait()
            pair.compare(f"stepped round {r}")
            pair.plan.next_round()
            pair.sim.next_round()
    finally:
        pair.close()
