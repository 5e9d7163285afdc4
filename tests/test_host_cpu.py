"""Host logic of the C library against the oracle (CPU only, no GPU calls).

* the library loads and exports every function include/*.h declares;
* schedule builders produce region/chunk tables bit-identical to the oracle's;
* plan-creation validation agrees with the oracle's, code for code;
* the grouped step->tile order equals the oracle's.
"""

import ctypes as C
import os
import random
import re

import numpy as np
import pytest

import triggered_copy_amd as tc
from triggered_copy_amd import _lib
from oracle import schedule as osched
from synth import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_function():
    lib = tc.lib()
    declared = set()
    for name in os.listdir(os.path.join(ROOT, "include")):
        if name.endswith(".h"):
            text = open(os.path.join(ROOT, "include", name)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            for m in re.finditer(r"^(?:int|void|const char\*)\s+(tc_\w+)\s*\(", text, flags=re.M):
                declared.add(m.group(1))
    assert declared, "no declarations found"
    for name in sorted(declared):
        assert hasattr(lib, name), f"{name} declared but not exported"
    assert declared == set(_lib.EXPORTS)
    assert b"gfx950" in lib.tc_version()


def test_header_is_plain_c_and_a_c_program_links(tmp_path):
    # include/tc.h is usable from C: the C round-trip program compiles with
    # -Werror and links against the library and the HIP runtime.
    from tests import c_abi_build
    exe = c_abi_build.build(str(tmp_path))
    assert os.path.exists(exe)


def _oview(v):
    return osched.View(v.byte_offset, v.rows, v.cols, v.row_stride, v.elem_bytes)


def _otables(s):
    ct, rt = s.tables()
    return (np.array(ct, dtype=np.uint64).reshape(-1, 3), np.array(rt, dtype=np.uint64).reshape(-1, 4))


def _same(cs, os_):
    ch, rg = cs.tables()
    och, org = _otables(os_)
    assert np.array_equal(ch, och)
    assert np.array_equal(rg, org)


def _random_view(rnd):
    e = rnd.choice([1, 2, 4, 8])
    cols = rnd.randint(1, 40)
    return tc.View(rnd.randint(0, 1000), rnd.randint(1, 40), cols, cols + rnd.choice([0, 0, 3, 17]), e, 0)


def test_builders_match_oracle_random():
    rnd = random.Random(10)
    for _ in range(300):
        v = _random_view(rnd)
        ov = _oview(v)
        w = rnd.randint(1, 5)
        _same(tc.whole(v, w), osched.whole(ov, w))
        n = rnd.randint(1, v.rows)
        _same(tc.chunks(v, n, w), osched.chunks(ov, n, w))
        bm, bn, T = rnd.randint(1, 9), rnd.randint(1, 9), rnd.randint(1, 7)
        tm, tn = -(-v.rows // bm), -(-v.cols // bn)
        order = list(range(tm * tn))
        rnd.shuffle(order)
        _same(tc.tile_chunks(v, (bm, bn), T, order=order), osched.tile_chunks(ov, bm, bn, T, order))
        _same(tc.tile_chunks(v, (bm, bn), T), osched.tile_chunks(ov, bm, bn, T))


def test_builders_match_oracle_named_workloads():
    for name, w in workloads.ALL.items():
        if "rows" not in w:
            continue
        e = {"u32": 4, "bf16": 2, "u8": 1}[w["elem"]]
        stride = w.get("stride", w["cols"])
        for p in range(w["P"]):
            v = tc.View(p * w["rows"] * stride * e, w["rows"], w["cols"], stride, e, 0)
            ov = _oview(v)
            if w["builder"] == "whole":
                _same(tc.whole(v, w["writers"]), osched.whole(ov, w["writers"]))
            elif w["builder"] == "chunks":
                _same(tc.chunks(v, w["n"], w["writers"]), osched.chunks(ov, w["n"], w["writers"]))
            else:
                tm, tn = -(-w["rows"] // w["bm"]), -(-w["cols"] // w["bn"])
                g = w.get("group_m")
                order = [osched.tile_of(s, tm, tn, g) for s in range(tm * tn)] if g else None
                _same(tc.tile_chunks(v, (w["bm"], w["bn"]), w["tiles_per_chunk"], order=order),
                      osched.tile_chunks(ov, w["bm"], w["bn"], w["tiles_per_chunk"], order))


def test_large_split_matches_oracle():
    v = tc.View(0, 786432, 512, 512, 4, 0)
    ch, rg = tc.whole(v, 192).tables()
    assert rg.tolist() == [[0, 1, 1 << 30, 1 << 30], [1 << 30, 1, 1 << 29, 1 << 29]]
    # A 2-D window over 1 GiB: whole rows per piece, as the oracle cuts it.
    v2 = tc.View(64, 3000, 262144, 524288, 4, 0)
    _same(tc.whole(v2, 1), osched.whole(_oview(v2), 1))


def test_from_arrays_and_append_match_oracle():
    regions = [(0, 1, 100, 100), (128, 3, 16, 48), (1000, 1, (1 << 30) + 5, (1 << 30) + 5)]
    chunks = [(0, 2, 2), (2, 1, 1)]
    _same(tc.from_arrays(chunks, regions), osched.from_tables(chunks, regions))
    empty = tc.from_arrays([], [])
    assert len(empty) == 0
    a = tc.from_arrays([(0, 1, 1)], [(0, 1, 8, 8)])
    a.append(tc.from_arrays([(0, 1, 3)], [(8, 2, 4, 6)]))
    ch, rg = a.tables()
    assert ch.tolist() == [[0, 1, 1], [1, 1, 3]]
    assert rg.tolist() == [[0, 1, 8, 8], [8, 2, 4, 6]]
    with pytest.raises(tc.InvalidArgument):
        tc.from_arrays([(1, 1, 1)], [(0, 1, 8, 8), (8, 1, 8, 8)])
    with pytest.raises(tc.InvalidArgument):
        tc.from_arrays([(0, 1, 0)], [(0, 1, 8, 8)])


def test_builder_errors():
    v = tc.View(0, 4, 4, 4, 4, 0)
    with pytest.raises(tc.InvalidArgument):
        tc.whole(v, 0)
    with pytest.raises(tc.InvalidArgument):
        tc.chunks(v, 5)
    with pytest.raises(tc.InvalidArgument):
        tc.tile_chunks(v, (2, 2), 2, order=[0, 1, 1, 3])
    with pytest.raises(tc.InvalidArgument):
        tc.whole(tc.View(0, 0, 4, 4, 4, 0))
    with pytest.raises(tc.InvalidArgument):
        tc.whole(tc.View(0, 4, 4, 3, 4, 0))
    # extents whose byte arithmetic would wrap 64 bits are refused, not wrapped
    with pytest.raises(tc.InvalidArgument):
        tc.whole(tc.View(0, 1 << 40, 4, 1 << 40, 4, 0))
    with pytest.raises(tc.InvalidArgument):
        tc.chunks(tc.View((1 << 63) + 16, 4, 4, 4, 4, 0), 2)
    with pytest.raises(tc.InvalidArgument):
        tc.from_arrays([(0, 1, 1)], [(0, 1 << 40, 16, 1 << 40)])
    with pytest.raises(tc.InvalidArgument):
        tc.from_arrays([(0, 1, 1)], [((1 << 64) - 64, 1, 128, 128)])


def test_order_grouped_matches_oracle():
    for tm in range(1, 18):
        for tn in range(1, 18):
            for g in (1, 2, 3, 8, 20):
                got = tc.order_grouped(tm, tn, g)
                assert got.tolist() == [osched.tile_of(s, tm, tn, g) for s in range(tm * tn)]


def _validate(P, B, scheds, own=None):
    ptrs = (C.c_void_p * P)(*[s.ptr.value if s is not None else None for s in scheds])
    d = _lib.PlanDesc()
    d.nranks = P
    d.flags = _lib.CHECK_OWN_ROWS if own else 0
    d.buffer_bytes = B
    d.schedules = C.cast(ptrs, C.POINTER(C.c_void_p))
    d.rows_per_rank_bytes = own or 0
    return tc.lib().tc_plan_validate(C.byref(d))


def test_validation_matches_oracle_random():
    rnd = random.Random(11)
    codes = {None: 0, "EINVAL": _lib.EINVAL, "EBOUNDS": _lib.EBOUNDS, "EOVERLAP": _lib.EOVERLAP}
    seen = set()
    for _ in range(600):
        P = rnd.randint(1, 4)
        B = rnd.choice([64, 96, 128])
        own = rnd.choice([None, None, B // P if P > 1 else None])
        cs, os_ = [], []
        for p in range(P):
            if rnd.random() < 0.15:
                cs.append(None)
                os_.append(None)
                continue
            regs = []
            for _ in range(rnd.randint(1, 3)):
                rows = rnd.randint(1, 3)
                rb = rnd.randint(1, 9)
                pitch = rb + rnd.randint(0, 6) if rows > 1 else rb
                off = rnd.randint(0, B)
                regs.append((off, rows, rb, pitch))
            ct = [(0, len(regs), rnd.randint(1, 2))]
            cs.append(tc.from_arrays(ct, regs))
            os_.append(osched.from_tables(ct, regs))
        try:
            osched.validate(B, os_, own)
            want = None
        except osched.ScheduleError as e:
            want = e.code
        got = _validate(P, B, cs, own)
        assert got == codes[want], (want, tc.lib().tc_last_error())
        seen.add(want)
    assert seen == {None, "EBOUNDS", "EOVERLAP"}


def test_validation_whole_out_everywhere_rejected():
    P, rows, cols = 4, 8, 16
    B = P * rows * cols * 4
    out = tc.View(0, P * rows, cols, cols, 4, 0)
    assert _validate(P, B, [tc.whole(out) for _ in range(P)]) == _lib.EOVERLAP
    mine = [tc.whole(tc.View(p * rows * cols * 4, rows, cols, cols, 4, 0)) for p in range(P)]
    assert _validate(P, B, mine) == 0
    assert _validate(P, B, mine, own=rows * cols * 4) == 0
    shifted = [tc.whole(tc.View(p * rows * cols * 4 + 4, rows, cols, cols, 4, 0)) for p in range(P - 1)]
    assert _validate(P - 1, B, shifted, own=rows * cols * 4) == _lib.EBOUNDS


def test_workspace_bytes():
    v = tc.View(0, 64, 64, 64, 4, 0)
    s = [tc.chunks(v, 4), None]
    ptrs = (C.c_void_p * 2)(s[0].ptr.value, None)
    out = C.c_uint64()
    assert tc.lib().tc_plan_workspace_bytes(2, ptrs, 0, C.byref(out)) == 0
    assert out.value >= 2 * 4 * 64 and out.value % 256 == 0


def test_bench_refuses_more_than_one_gpu():
    # The P ranks are simulated on one GPU: --gpus N > 1 exits with a message.
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
