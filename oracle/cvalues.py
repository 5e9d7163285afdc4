"""The oracle's value hash in plain C (``oracle/values.c``), for tests that
check every element of the largest workloads.  TEST INFRASTRUCTURE ONLY, as
the rest of this package.  The library is built with gcc by ``build()``
(``__graft_entry__.build()`` calls it), or on first use if it is missing."""

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "values.c")
LIB = os.path.join(HERE, "liboracle_values.so")

_lib = None


def build() -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-shared", "-fPIC", "-pthread",
           SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building {SRC} failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = C.CDLL(LIB)
        L.oracle_splitmix64_stream.argtypes = [C.c_uint64, C.c_uint64, C.c_void_p]
        L.oracle_splitmix64_stream.restype = None
        L.oracle_u32_pattern.argtypes = [C.c_uint64, C.c_uint32, C.c_uint32, C.c_uint64, C.c_uint64,
                                         C.c_void_p, C.c_uint32]
        L.oracle_u32_pattern.restype = C.c_int
        _lib = L
    return _lib


def threads() -> int:
    """Host threads to use: the cores this process may run on, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def splitmix64_stream(seed: int, n: int):
    out = np.zeros(n, dtype=np.uint64)
    lib().oracle_splitmix64_stream(seed & ((1 << 64) - 1), n, out.ctypes.data)
    return [int(x) for x in out]


def u32_pattern_into(out: np.ndarray, seed: int, rank: int, rnd: int, first: int, nthreads=None):
    """Fills the uint32 array ``out`` with elements first .. first+len-1."""
    assert out.dtype == np.uint32 and out.flags.c_contiguous
    rc = lib().oracle_u32_pattern(seed & ((1 << 64) - 1), rank, rnd, first, out.size, out.ctypes.data,
                                  nthreads or threads())
    if rc != 0:
        raise ValueError("rank, round or index outside the key layout")
    return out
