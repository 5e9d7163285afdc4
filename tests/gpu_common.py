"""Shared set-up for the GPU parity tests: one workload run on the HIP path
and on the CPU oracle from the same seeded inputs."""

import sys
import time

import numpy as np
import torch

import triggered_copy_amd as tc
from oracle import plan as oplan
from oracle import schedule as osched
from oracle import values as ovalues
from synth import BASE_SEED, SENTINEL, shuffled_order

ELEM = {"u32": 4, "bf16": 2, "u8": 1}


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X")
    tc.lib()


def log(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def rank_views(w):
    """(tc views, oracle views) of every rank's rows of `out`."""
    e = ELEM[w["elem"]]
    stride = w.get("stride", w["cols"])
    tv, ov = [], []
    for p in range(w["P"]):
        off = p * w["rows"] * stride * e
        tv.append(tc.View(off, w["rows"], w["cols"], stride, e, 0))
        ov.append(osched.View(off, w["rows"], w["cols"], stride, e))
    return tv, ov


def tile_order(w):
    if w.get("group_m"):
        tm, tn = -(-w["rows"] // w["bm"]), -(-w["cols"] // w["bn"])
        return [osched.tile_of(s, tm, tn, w["group_m"]) for s in range(tm * tn)]
    return None


def build_schedules(w, tv, ov):
    ts, os_ = [], []
    for v, o in zip(tv, ov):
        b = w["builder"]
        if b == "whole":
            ts.append(tc.whole(v, w["writers"]))
            os_.append(osched.whole(o, w["writers"]))
        elif b == "chunks":
            ts.append(tc.chunks(v, w["n"], w["writers"]))
            os_.append(osched.chunks(o, w["n"], w["writers"]))
        else:
            order = tile_order(w)
            ts.append(tc.tile_chunks(v, (w["bm"], w["bn"]), w["tiles_per_chunk"], order=order))
            os_.append(osched.tile_chunks(o, w["bm"], w["bn"], w["tiles_per_chunk"], order))
    return ts, os_


def buffer_bytes(w):
    e = ELEM[w["elem"]]
    b = w["P"] * w["rows"] * w.get("stride", w["cols"]) * e
    return (b + 255) // 256 * 256


def oracle_produce(rep, v, kind, seed, p, r):
    """Write rank p's round-r values into replica array ``rep`` (oracle)."""
    e = ELEM[kind]
    vals = ovalues.block_bytes(kind, seed, p, r, v.rows * v.cols).reshape(v.rows, v.cols * e)
    if v.row_stride == v.cols:
        rep[v.byte_offset:v.byte_offset + v.rows * v.cols * e] = vals.reshape(-1)
    else:
        for i in range(v.rows):
            a = v.byte_offset + i * v.row_stride * e
            rep[a:a + v.cols * e] = vals[i]


def oracle_produce_regions(rep, v, sched, kind, seed, p, r):
    """As oracle_produce, but only the bytes of ``sched``'s regions: what a
    producer that writes exactly its scheduled regions leaves."""
    tmp = rep.copy()
    oracle_produce(tmp, v, kind, seed, p, r)
    for ch in sched.chunks:
        for off, rows, rb, pitch in ch.regions:
            for i in range(rows):
                a = off + i * pitch
                rep[a:a + rb] = tmp[a:a + rb]


def gate_array(sim):
    return sim.gate_bytes()


class Pair:
    """A plan on the GPU and its oracle twin over the same workload."""

    def __init__(self, w, seed=BASE_SEED, oracle_bytes=True, **plan_kw):
        require_gpu()
        self.w, self.seed = w, seed
        self.P = w["P"]
        self.B = buffer_bytes(w)
        self.tv, self.ov = rank_views(w)
        self.ts, self.os = build_schedules(w, self.tv, self.ov)
        self.rep = torch.full((self.P, self.B), SENTINEL, dtype=torch.uint8, device="cuda")
        plan_kw.setdefault("backstop_s", 20.0)
        self.plan = tc.TriggeredPlan(self.rep, self.ts, **plan_kw)
        if oracle_bytes:
            reps = [np.full(self.B, SENTINEL, dtype=np.uint8) for _ in range(self.P)]
            self.sim = oplan.PlanSim(reps, self.os)
        else:
            self.sim = oplan.PlanSim(None, self.os, buffer_bytes=self.B)
        self.stream = torch.cuda.Stream()     # the producers' stream (not the legacy default)
        torch.cuda.synchronize()              # the sentinel fill ran on the default stream

    def oracle_round(self, mark_order=None, extra=(), withheld=()):
        w = self.w

        def produce(p, r):
            if self.sim.rep is not None:
                oracle_produce(self.sim.rep[p], self.ov[p], w["elem"], self.seed, p, r)
        oplan.run_round(self.sim, produce, mark_order=mark_order, extra_marks=extra, withheld=withheld)

    def orders_device(self, r):
        """Seeded per-rank chunk completion orders for round r, [P, n] on the GPU."""
        n = max(len(s.chunks) for s in self.os)
        arr = np.stack([shuffled_order(self.seed, p, r, n) for p in range(self.P)])
        return arr, torch.from_numpy(arr.astype(np.int32)).cuda()

    def gpu_round_fill(self, mark=True, serial=False, order=None, order_stride=0, timeout=10.0,
                       **fill_kw):
        h = self.plan.start(self.stream)
        self.plan.fill(h, self.tv, self.seed, kind=self.w["elem"], mark=mark, serial=serial,
                       order=order, order_stride=order_stride, stream=self.stream, **fill_kw)
        if not mark:
            self.plan.mark_all(h, stream=self.stream)
        self.plan.wait(timeout)
        return h

    def undelivered_mask(self, q):
        """Bytes of replica q that belong to chunks not yet delivered to q.
        Their content is unpinned: the engine may copy an open chunk before
        an earlier chunk's arrival is signalled (arrivals stay in order)."""
        m = np.zeros(self.B, dtype=bool)
        for p in range(self.P):
            if p == q:
                continue
            for c in range(int(self.sim.cur[p, q]), self.sim.n[p]):
                for off, rows, rb, pitch in self.os[p].chunks[c].regions:
                    for i in range(rows):
                        m[off + i * pitch: off + i * pitch + rb] = True
        return m

    def compare(self, what="", partial=False):
        torch.cuda.synchronize()
        g = self.plan.gates()
        og = gate_array(self.sim)
        assert g.shape == og.shape
        bad = np.argwhere((g != og).any(axis=2))
        assert bad.size == 0, f"{what}: gate rows differ at (table, chunk) {bad[:8].tolist()}"
        cur = self.plan.cursors()
        assert np.array_equal(cur, self.sim.cur), f"{what}: cursors {cur.tolist()} vs {self.sim.cur.tolist()}"
        if self.sim.rep is not None:
            host = self.rep.cpu().numpy()
            for q in range(self.P):
                neq = host[q] != self.sim.rep[q]
                if partial:
                    neq &= ~self.undelivered_mask(q)
                if neq.any():
                    diff = np.flatnonzero(neq)
                    raise AssertionError(f"{what}: replica {q} differs at {diff.size} bytes, first {diff[:8]}")

    def close(self):
        self.plan.close()


def wait_until(fn, timeout_s=5.0):
    t0 = time.time()
    while time.time() - t0 < timeout_s:
        if fn():
            return True
        time.sleep(0.0005)
    return fn()
