"""The C-ABI from a plain C program (tests/c_abi/round_trip.c): device
buffers from hipMalloc, no Python binding, two rounds of three ranks checked
for delivery, no stale data and gate rows."""

import subprocess

import pytest

from tests import c_abi_build
from tests.gpu_common import log, require_gpu

pytestmark = pytest.mark.gpu


def test_plain_c_round_trip(tmp_path):
    require_gpu()
    exe = c_abi_build.build(str(tmp_path))
    log("c_abi round_trip: 3 ranks, 3 rounds")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "OK" in r.stdout
