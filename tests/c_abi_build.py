"""Builds tests/c_abi/round_trip.c, a plain C user of include/tc.h, with gcc
against the in-tree library and the HIP runtime.  Used by the CPU test (it
must compile and link) and the GPU test (it must run and pass)."""

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "round_trip.c")
LIBDIR = os.path.join(ROOT, "triggered_copy_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out_dir):
    exe = os.path.join(out_dir, "round_trip")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SRC,
           "-o", exe, "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-L", LIBDIR, "-ltriggered_copy",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", f"-Wl,-rpath,{LIBDIR}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the C program failed:\n{r.stdout}{r.stderr}")
    return exe
