"""The no-allocation plan (tc_plan_create_noalloc), through the C boundary,
against the ordinary plan (tc_plan_create) on the same workloads.

Two calls in a row, the second with a smaller input: a plan over a larger
workload is created in the library's static workspace, run and closed; then
a plan over a smaller one reuses the same array, which still holds the
first plan's state.  Every round's replicas, gate rows and queue cursors
must equal the ordinary plan's bit for bit (and the oracle's).  Also: a
second open no-allocation plan on the device is refused, and so is a plan
whose workspace would not fit."""

import numpy as np
import pytest
import torch

import triggered_copy_amd as tc
from synth import workloads
from tests.gpu_common import Pair, log, require_gpu

pytestmark = pytest.mark.gpu


def _run(w, noalloc, rounds):
    """Every round's (replicas, gates, cursors) of workload w, and the plan's
    check against the oracle after each round."""
    pair = Pair(w, noalloc=noalloc)
    out = []
    try:
        for r in range(1, rounds + 1):
            pair.gpu_round_fill()
            pair.oracle_round()
            pair.compare(f"{'noalloc' if noalloc else 'workspace'} round {r}")
            torch.cuda.synchronize()
            out.append((pair.rep.cpu().numpy().copy(), pair.plan.gates(), pair.plan.cursors()))
            pair.plan.next_round()
            pair.sim.next_round()
    finally:
        pair.close()
    return out


@pytest.mark.parametrize("names", [("u32_whole_p8", "bf16_chunks_p2")])
def test_noalloc_plan_matches_the_workspace_plan_twice(names):
    require_gpu()
    for i, name in enumerate(names):
        w = dict(workloads.ALL[name])
        rounds = 3
        log(f"no-allocation plan, call {i + 1}: {name}, {rounds} rounds")
        got = _run(w, True, rounds)
        want = _run(w, False, rounds)
        for r, ((rg, gg, cg), (rw, gw, cw)) in enumerate(zip(got, want), 1):
            assert np.array_equal(rg, rw), f"{name} round {r}: replicas differ"
            assert np.array_equal(gg, gw), f"{name} round {r}: gate rows differ"
            assert np.array_equal(cg, cw), f"{name} round {r}: cursors differ"


def test_noalloc_refuses_a_second_plan_and_an_oversized_one():
    require_gpu()
    w = dict(workloads.SMALL["u32_chunks_ragged_p3"])
    a = Pair(w, noalloc=True)
    try:
        with pytest.raises(tc.StateError, match="already open"):
            tc.TriggeredPlan(a.rep, a.ts, noalloc=True)
        a.gpu_round_fill()
        a.oracle_round()
        a.compare("noalloc beside a refused second plan")
    finally:
        a.close()
    # 2 ranks x 128 MiB in 256-byte pieces: about 32 MiB of piece descriptors
    # alone, past the static workspace.
    rep = torch.zeros((2, 256 << 20), dtype=torch.uint8, device="cuda")
    views = [tc.View(p * (128 << 20), 1 << 15, 4096, 4096, 1, 0) for p in range(2)]
    with pytest.raises(tc.WorkspaceTooSmall, match="no-allocation"):
        tc.TriggeredPlan(rep, [tc.whole(v) for v in views], piece_bytes=256, noalloc=True)
    # the device's array is free again for the next plan
    b = Pair(dict(workloads.SMALL["u32_whole_p5"]), noalloc=True)
    try:
        b.gpu_round_fill()
        b.oracle_round()
        b.compare("noalloc after the refusals")
    finally:
        b.close()
