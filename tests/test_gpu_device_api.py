"""The exported device calls from a kernel outside the library.

tests/device_api/user_kernels.hip includes include/tc_device.h only and
builds a small all-gather of per-rank payloads on tc_notify / tc_wait_ge
("Barrier: Signals Only", The idea and Walkthrough).  The signal window must
end equal to the oracle's barrier after the same generations, and every
payload a rank read after its wait must be the one its peer wrote in that
generation (release before notify, acquire after the wait)."""

import ctypes as C
import os

import numpy as np
import pytest
import torch

from oracle import barrier as obarrier
from tests.gpu_common import log, require_gpu

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "device_api", "libtc_user_kernels.so")


def _lib():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built (run __graft_entry__.build())")
    lib = C.CDLL(LIB)
    lib.tcu_gather.restype = C.c_int
    lib.tcu_gather.argtypes = [C.c_void_p, C.c_uint32, C.c_uint32, C.c_uint32, C.c_void_p,
                               C.c_void_p, C.c_uint32, C.c_void_p, C.c_void_p]
    return lib


def _payload(g, rank, t):
    v = (np.uint64(g) * np.uint64(2654435761)) & np.uint64(0xFFFFFFFF)
    v = v ^ (np.uint64(rank) << np.uint64(24)) ^ (t.astype(np.uint64) * np.uint64(40503))
    return (v & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.int32)


@pytest.mark.parametrize("P,gens", [(8, 300), (2, 50), (5, 120)])
def test_user_kernel_gathers_on_notify_and_wait_ge(P, gens):
    require_gpu()
    lib = _lib()
    W = torch.zeros((P, P), dtype=torch.int32, device="cuda")
    stage = torch.zeros((2, P, 256), dtype=torch.int32, device="cuda")
    out = torch.zeros((gens, P, P, 256), dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    for first in (1, gens + 1):          # a second run continues the generation count
        log(f"user gather P={P} generations {first}..{first + gens - 1}")
        rc = lib.tcu_gather(W.data_ptr(), P, first, gens, stage.data_ptr(), out.data_ptr(), 1 << 22,
                            status.data_ptr(), C.c_void_p(s))
        assert rc == 0
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert np.array_equal(W.cpu().numpy(), obarrier.run(P, first + gens - 1))
        got = out.cpu().numpy()
        t = np.arange(256)
        for i in range(gens):
            g = first + i
            want = np.stack([_payload(g, s_, t) for s_ in range(P)])
            for m in range(P):
                assert np.array_equal(got[i, m], want), f"generation {g}: rank {m} read stale words"
