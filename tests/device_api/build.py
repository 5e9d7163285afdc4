"""Builds tests/device_api/libtc_user_kernels.so: user kernels that include
include/tc_device.h and nothing else of the library, for the GPU tests of
the exported device calls.  Compiled in-tree for gfx950 with the library's
own flags, by __graft_entry__.build()."""

import os
import subprocess

from triggered_copy_amd import build as tcbuild

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "user_kernels.hip")
LIB = os.path.join(HERE, "libtc_user_kernels.so")


def build(verbose: bool = True) -> str:
    tmp = LIB + ".tmp"
    cmd = [tcbuild.hipcc(), "-x", "hip", SRC, "-shared", "-o", tmp] + tcbuild.common_flags()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building {SRC} failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB
