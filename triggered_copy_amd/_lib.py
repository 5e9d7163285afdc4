"""ctypes declarations of the C boundary (include/tc.h).  Marshalling only."""

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtriggered_copy.so")

TC_MAX_RANKS = 16
NOALLOC_WORKSPACE_BYTES = 32 << 20
GATE_ROW_BYTES = 64

OK, EINVAL, EBOUNDS, EOVERLAP, ENOMEM, EHIP, ESTATE, ETIMEOUT, EEXTRA, EROUNDS, ENODEV, ECORRUPT = \
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10, -11
STATE_NAMES = {0: "READY", 1: "STARTED", 2: "DONE", 3: "FAILED", 4: "CLOSED", 5: "CLOSING"}
CHECK_OWN_ROWS = 1
FILL_U32, FILL_BF16, FILL_U8 = 0, 1, 2
FILL_PARALLEL, FILL_SERIAL, FILL_WAVES, FILL_ONESHOT = 0, 1, 2, 3
MARK_INKERNEL, MARK_NONE = 0, 1

u32, u64, vp = C.c_uint32, C.c_uint64, C.c_void_p


class View(C.Structure):
    _fields_ = [("byte_offset", u64), ("rows", u64), ("cols", u64), ("row_stride", u64),
                ("elem_bytes", u32), ("rsvd", u32)]


class Region(C.Structure):
    _fields_ = [("offset", u64), ("rows", u64), ("row_bytes", u64), ("pitch", u64)]


class Chunk(C.Structure):
    _fields_ = [("first_region", u32), ("num_regions", u32), ("writers", u32), ("rsvd", u32)]


class Handle(C.Structure):
    _fields_ = [("gates", u64), ("gate_stride", u64), ("writers", u64), ("marks", u64), ("round", u32),
                ("nranks", u32), ("chunk_base", u32 * (TC_MAX_RANKS + 1)), ("rsvd", u32)]


class PlanDesc(C.Structure):
    _fields_ = [("nranks", u32), ("flags", u32), ("replicas", C.POINTER(vp)),
                ("buffer_bytes", u64), ("schedules", C.POINTER(vp)), ("workspace", vp),
                ("workspace_bytes", u64), ("rows_per_rank_bytes", u64),
                ("cu_mask", C.POINTER(u32)), ("cu_mask_words", u32), ("engine_ctas", u32),
                ("piece_bytes", u64), ("engine_backstop_us", u64)]


class Stats(C.Structure):
    _fields_ = [("engine_ms", C.c_float), ("launches", u32), ("engine_ctas", u32),
                ("window_ticks", u64), ("bytes_moved", u64), ("bytes_read", u64),
                ("pieces", u64), ("G", u32), ("engine_checked", u32)]


class FillDesc(C.Structure):
    _fields_ = [("views", C.POINTER(View)), ("seed", u64), ("kind", u32), ("mark_mode", u32),
                ("mode", u32), ("rsvd", u32), ("order", vp), ("order_stride", u32),
                ("ctas", u32)]


_SIGS = {
    "tc_schedule_whole": [C.POINTER(View), u32, C.POINTER(vp)],
    "tc_schedule_chunks": [C.POINTER(View), u32, u32, C.POINTER(vp)],
    "tc_schedule_tile_chunks": [C.POINTER(View), u32, u32, u32, C.POINTER(u32), u32, C.POINTER(vp)],
    "tc_schedule_from_arrays": [C.POINTER(Chunk), u32, C.POINTER(Region), u32, C.POINTER(vp)],
    "tc_schedule_append": [vp, vp],
    "tc_schedule_get": [vp, C.POINTER(C.POINTER(Chunk)), C.POINTER(u32),
                        C.POINTER(C.POINTER(Region)), C.POINTER(u32)],
    "tc_order_grouped": [u32, u32, u32, C.POINTER(u32)],
    "tc_plan_workspace_bytes": [u32, C.POINTER(vp), u64, C.POINTER(u64)],
    "tc_plan_validate": [C.POINTER(PlanDesc)],
    "tc_plan_create": [C.POINTER(PlanDesc), C.POINTER(vp)],
    "tc_plan_create_noalloc": [C.POINTER(PlanDesc), C.POINTER(vp)],
    "tc_plan_start": [vp, vp, C.POINTER(Handle)],
    "tc_plan_wait": [vp, u64],
    "tc_plan_handle": [vp, C.POINTER(Handle)],
    "tc_plan_next_round": [vp],
    "tc_plan_close": [vp, C.POINTER(C.c_int)],
    "tc_plan_state": [vp, C.POINTER(C.c_int), C.POINTER(u32)],
    "tc_plan_problems": [vp, C.POINTER(u32), u32, C.POINTER(u32)],
    "tc_plan_read_gates": [vp, vp, u64],
    "tc_plan_read_cursors": [vp, C.POINTER(u32)],
    "tc_plan_stats": [vp, C.POINTER(Stats)],
    "tc_plan_engine_stream": [vp, C.POINTER(vp)],
    "tc_plan_debug_set_round": [vp, u32],
    "tc_produce_fill": [vp, C.POINTER(Handle), C.POINTER(FillDesc), vp],
    "tc_mark_all": [vp, C.POINTER(Handle), vp],
    "tc_mark": [vp, C.POINTER(Handle), u32, u32, u32, vp],
    "tc_gemm_bf16": [vp, vp, vp, u32, u32, u32, u64, u32, u32, C.POINTER(Handle), u32, u32, u32, vp],
    "tc_consume_copy": [vp, C.POINTER(Handle), u32, vp, u32, vp, vp],
    "tc_plan_row_deps": [vp, C.POINTER(View), u32, C.POINTER(u32), C.POINTER(u32), u32,
                         C.POINTER(u32), C.POINTER(u32)],
    "tc_gemm_consume_bf16": [C.POINTER(Handle), u32, vp, vp, u32, vp, vp, u64, vp, vp, u32, u32, u32,
                             u64, u32, u32, vp],
    "tc_barrier_run": [vp, u32, u32, u32, vp, vp, vp, u32, vp, vp],
}

EXPORTS = sorted(list(_SIGS) + ["tc_schedule_free", "tc_last_error", "tc_version", "tc_release"])

_lib = None


def load() -> C.CDLL:
    """Loads the in-tree HIP library.  There is no fallback: without it the
    package cannot run."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m triggered_copy_amd.build` (hipcc, gfx950)")
    lib = C.CDLL(LIB_PATH)
    for name, args in _SIGS.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = C.c_int
    lib.tc_schedule_free.argtypes = [vp]
    lib.tc_schedule_free.restype = None
    lib.tc_last_error.argtypes = []
    lib.tc_last_error.restype = C.c_char_p
    lib.tc_version.argtypes = []
    lib.tc_version.restype = C.c_char_p
    lib.tc_release.argtypes = []
    lib.tc_release.restype = C.c_int
    _lib = lib
    return lib
