"""Triggered (gated) chunked all-gather on MI355X: Python binding.

Thin marshalling over the C boundary declared in ``include/tc.h``; every step
of the path runs in the HIP library ``libtriggered_copy.so`` (built in-tree
for gfx950).  PyTorch is used only for device memory and streams.

Pages (title -- section): "Triggered Plans" (Iris documentation) -- Model,
The kernel author's contract, Memory ordering, Gates and rounds; "Triggered
SDMA Plans" (Iris pull request) -- API; "Barrier: Signals Only" (pypto
documentation) -- Walkthrough.
"""

import atexit
import ctypes as C
import weakref

import numpy as np

from . import _lib
from ._lib import (FILL_BF16, FILL_U8, FILL_U32, MARK_INKERNEL, MARK_NONE,  # noqa: F401
                   FILL_PARALLEL, FILL_SERIAL, FILL_WAVES, FILL_ONESHOT,
                   GATE_ROW_BYTES, TC_MAX_RANKS, Handle, View)

__all__ = ["View", "Schedule", "whole", "chunks", "tile_chunks", "from_arrays", "order_grouped",
           "view_of", "TriggeredPlan", "prepare_all_gather", "gemm_bf16", "gemm_consume_bf16",
           "barrier", "release",
           "TriggeredCopyError",
           "PlanTimeout", "ExtraMarksError", "StateError", "RoundLimitError"]


# ------------------------------------------------------------------ errors

class TriggeredCopyError(RuntimeError):
    code = None

    def __init__(self, msg, code=None, chunks=()):
        super().__init__(msg)
        if code is not None:
            self.code = code
        self.chunks = list(chunks)


class InvalidArgument(TriggeredCopyError):
    code = _lib.EINVAL


class BoundsError(TriggeredCopyError):
    code = _lib.EBOUNDS


class OverlapError(TriggeredCopyError):
    code = _lib.EOVERLAP


class WorkspaceTooSmall(TriggeredCopyError):
    code = _lib.ENOMEM


class HipError(TriggeredCopyError):
    code = _lib.EHIP


class StateError(TriggeredCopyError):
    code = _lib.ESTATE


class PlanTimeout(TriggeredCopyError):
    code = _lib.ETIMEOUT


class ExtraMarksError(TriggeredCopyError):
    code = _lib.EEXTRA


class RoundLimitError(TriggeredCopyError):
    code = _lib.EROUNDS


class NoDevice(TriggeredCopyError):
    code = _lib.ENODEV


class CorruptGates(TriggeredCopyError):
    code = _lib.ECORRUPT


_ERRORS = {c.code: c for c in (InvalidArgument, BoundsError, OverlapError, WorkspaceTooSmall,
                               HipError, StateError, PlanTimeout, ExtraMarksError,
                               RoundLimitError, NoDevice, CorruptGates)}


def lib():
    return _lib.load()


# Plans not yet closed.  At interpreter exit they are closed and the
# library's process-lifetime engine streams are released, while the HIP
# runtime is still whole: freeing them from finalizers during the runtime's
# own teardown is not safe.
_LIVE = weakref.WeakSet()


@atexit.register
def _close_all_at_exit():
    if _lib._lib is None:
        return
    for _ in range(3):                   # a CLOSING plan finishes once the plan before it closes
        for plan in list(_LIVE):
            try:
                plan.close()
            except Exception:
                pass
        if not _LIVE:
            break
    if not _LIVE:
        _lib._lib.tc_release()


def release():
    """Destroys the library's cached engine streams (tc_release).  Every
    plan must be closed first."""
    _check(lib().tc_release())


def _check(rc, chunks=()):
    if rc != _lib.OK:
        msg = lib().tc_last_error().decode(errors="replace")
        raise _ERRORS.get(rc, TriggeredCopyError)(msg, rc, chunks)


def _stream_ptr(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return C.c_void_p(getattr(stream, "cuda_stream", stream))


# --------------------------------------------------------------- schedules

def view_of(t, base=None, elem_bytes=None) -> View:
    """The view of tensor ``t`` relative to ``base`` (``base=out`` of the
    page's builders).  1-D tensors are one row.  Only a row stride is allowed
    (the last dimension must be contiguous)."""
    base = t if base is None else base
    e = elem_bytes or t.element_size()
    if t.dim() == 1:
        rows, cols, stride = 1, t.shape[0], t.shape[0]
        if t.stride(0) != 1:
            raise InvalidArgument("1-D view must be contiguous")
    elif t.dim() == 2:
        rows, cols = t.shape
        if t.stride(1) != 1:
            raise InvalidArgument("last dimension must be contiguous")
        stride = t.stride(0)
    else:
        raise InvalidArgument("views are 1-D or 2-D")
    off = t.data_ptr() - base.data_ptr()
    if off < 0:
        raise InvalidArgument("view starts before its base")
    return View(off, rows, cols, stride, e, 0)


def _as_view(v, base):
    if isinstance(v, View):
        return v
    if isinstance(v, (tuple, list)):                 # (byte_offset, rows, cols, stride, elem)
        return View(*v, 0)
    return view_of(v, base)


class Schedule:
    """One rank's chunks (owned host memory in the library)."""

    def __init__(self, ptr):
        self._ptr = C.c_void_p(ptr)

    @property
    def ptr(self):
        return self._ptr

    def __del__(self):
        # At interpreter exit the module globals may already be gone.
        lib_mod = globals().get("_lib")
        if getattr(self, "_ptr", None) and self._ptr.value and lib_mod is not None \
                and getattr(lib_mod, "_lib", None) is not None:
            lib_mod._lib.tc_schedule_free(self._ptr)
            self._ptr = C.c_void_p(0)

    def tables(self):
        """(chunks [n, 3] = first_region, num_regions, writers;
            regions [m, 4] = offset, rows, row_bytes, pitch) as uint64 numpy."""
        cp, nc = C.POINTER(_lib.Chunk)(), C.c_uint32()
        rp, nr = C.POINTER(_lib.Region)(), C.c_uint32()
        _check(lib().tc_schedule_get(self._ptr, C.byref(cp), C.byref(nc), C.byref(rp), C.byref(nr)))
        ch = np.zeros((nc.value, 3), dtype=np.uint64)
        for i in range(nc.value):
            ch[i] = (cp[i].first_region, cp[i].num_regions, cp[i].writers)
        rg = np.zeros((nr.value, 4), dtype=np.uint64)
        if nr.value:
            raw = np.ctypeslib.as_array(C.cast(rp, C.POINTER(C.c_uint64)), shape=(nr.value * 4,))
            rg[:] = raw.reshape(nr.value, 4)
        return ch, rg

    def append(self, other: "Schedule") -> "Schedule":
        _check(lib().tc_schedule_append(self._ptr, other._ptr))
        return self

    def __len__(self):
        return len(self.tables()[0])


def _new(fn, *args) -> Schedule:
    out = C.c_void_p()
    _check(fn(*args, C.byref(out)))
    return Schedule(out.value)


def whole(mine, writers: int = 1, base=None) -> Schedule:
    """One chunk, marked once by each of ``writers`` programs."""
    v = _as_view(mine, base)
    return _new(lib().tc_schedule_whole, C.byref(v), writers)


def chunks(mine, n: int, writers: int = 1, base=None) -> Schedule:
    """One chunk per row block (tensor_split rule), completed in order."""
    v = _as_view(mine, base)
    return _new(lib().tc_schedule_chunks, C.byref(v), n, writers)


def tile_chunks(mine, tile, tiles_per_chunk: int, order=None, base=None) -> Schedule:
    """One region per tile, consecutive steps grouped into chunks; ``order``
    is the producer's step->tile map (a sequence, or a callable of the step)."""
    v = _as_view(mine, base)
    bm, bn = tile
    if order is not None:
        nt = -(-v.rows // bm) * -(-v.cols // bn)
        if callable(order):
            order = [order(i) for i in range(nt)]
        arr = (C.c_uint32 * len(order))(*[int(x) for x in order])
        return _new(lib().tc_schedule_tile_chunks, C.byref(v), bm, bn, tiles_per_chunk, arr, len(order))
    return _new(lib().tc_schedule_tile_chunks, C.byref(v), bm, bn, tiles_per_chunk, None, 0)


def from_arrays(chunk_table, region_table) -> Schedule:
    """Hand-built schedule: rows (first_region, num_regions, writers) over
    rows (offset, rows, row_bytes, pitch).  Empty tables = sends nothing."""
    ct = list(chunk_table)
    rt = list(region_table)
    ca = (_lib.Chunk * max(1, len(ct)))(*[_lib.Chunk(int(a), int(b), int(c), 0) for a, b, c in ct])
    ra = (_lib.Region * max(1, len(rt)))(*[_lib.Region(*[int(x) for x in r]) for r in rt])
    return _new(lib().tc_schedule_from_arrays, ca, len(ct), ra, len(rt))


def order_grouped(tm: int, tn: int, group_m: int) -> np.ndarray:
    out = (C.c_uint32 * (tm * tn))()
    _check(lib().tc_order_grouped(tm, tn, group_m, out))
    return np.frombuffer(out, dtype=np.uint32).copy()


# ------------------------------------------------------------------- plans

class TriggeredPlan:
    """A triggered all-gather over P replica buffers of one GPU.

    ``replicas``: a [P, B] uint8 CUDA tensor or a list of P CUDA tensors of
    equal byte size (256-byte aligned).  ``schedules``: P schedules (None =
    that rank sends nothing).  The workspace is a torch allocation unless
    given; with ``noalloc=True`` the plan is made by tc_plan_create_noalloc
    and uses the library's static per-device workspace instead (one such
    plan per device at a time).  Use as a context manager; leaving the block
    closes the plan.
    """

    def __init__(self, replicas, schedules, *, own_rows_bytes=None, cu_mask=None,
                 engine_ctas=0, piece_bytes=0, backstop_s=30.0, workspace=None, noalloc=False):
        import torch
        if isinstance(replicas, torch.Tensor) and replicas.dim() == 2:
            reps = [replicas[p] for p in range(replicas.shape[0])]
        else:
            reps = list(replicas)
        P = len(reps)
        if not 1 <= P <= TC_MAX_RANKS or len(schedules) != P:
            raise InvalidArgument("need 1..16 replicas and one schedule per replica")
        nbytes = reps[0].numel() * reps[0].element_size()
        for r in reps:
            if r.numel() * r.element_size() != nbytes or not r.is_cuda:
                raise InvalidArgument("replicas must be CUDA tensors of equal size")
            if not r.is_contiguous() or r.device != reps[0].device:
                raise InvalidArgument("replicas must be contiguous and on one device")
        self.P, self.buffer_bytes = P, nbytes
        self._keep = (reps, list(schedules))
        sched_ptrs = (C.c_void_p * P)(*[s.ptr.value if s is not None else None for s in schedules])
        self._sched_ptrs = sched_ptrs
        if noalloc and workspace is not None:
            raise InvalidArgument("a no-allocation plan takes no workspace")
        if workspace is None and not noalloc:
            ws_need = C.c_uint64()
            _check(lib().tc_plan_workspace_bytes(P, sched_ptrs, piece_bytes, C.byref(ws_need)))
            workspace = torch.empty(ws_need.value, dtype=torch.uint8, device=reps[0].device)
        self.workspace = workspace
        rep_ptrs = (C.c_void_p * P)(*[r.data_ptr() for r in reps])
        self._rep_ptrs = rep_ptrs
        d = _lib.PlanDesc()
        d.nranks = P
        d.flags = _lib.CHECK_OWN_ROWS if own_rows_bytes else 0
        d.replicas = C.cast(rep_ptrs, C.POINTER(C.c_void_p))
        d.buffer_bytes = nbytes
        d.schedules = C.cast(sched_ptrs, C.POINTER(C.c_void_p))
        d.workspace = workspace.data_ptr() if workspace is not None else None
        d.workspace_bytes = workspace.numel() if workspace is not None else 0
        d.rows_per_rank_bytes = own_rows_bytes or 0
        if cu_mask is not None:
            m = (C.c_uint32 * len(cu_mask))(*cu_mask)
            self._mask = m
            d.cu_mask = C.cast(m, C.POINTER(C.c_uint32))
            d.cu_mask_words = len(cu_mask)
        d.engine_ctas = engine_ctas
        d.piece_bytes = piece_bytes
        d.engine_backstop_us = int(backstop_s * 1e6)
        self._desc = d
        ptr = C.c_void_p()
        create = lib().tc_plan_create_noalloc if noalloc else lib().tc_plan_create
        with torch.cuda.device(reps[0].device):  # the plan's streams live on the replicas' device
            _check(create(C.byref(d), C.byref(ptr)))
        self._p = ptr
        self.handle = None
        _LIVE.add(self)

    # -- context manager
    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
        return False

    def close(self):
        """Closes the plan; mid-round, every chunk is sent as it stands.
        Returns "CLOSED", or "CLOSING" when this plan's copies are queued
        behind another plan's waiting ones: close that plan, then call
        close() here again."""
        if getattr(self, "_p", None) is None or not self._p.value:
            return "CLOSED"
        closing = C.c_int(0)
        rc = lib().tc_plan_close(self._p, C.byref(closing))
        if rc == _lib.OK and closing.value:
            return "CLOSING"
        if rc == _lib.OK:
            self._p = C.c_void_p(0)
            _LIVE.discard(self)
        _check(rc)
        return "CLOSED"

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- round
    def start(self, stream=None) -> Handle:
        h = Handle()
        _check(lib().tc_plan_start(self._p, _stream_ptr(stream), C.byref(h)))
        self.handle = h
        return h

    def current_handle(self) -> Handle:
        """This round's handle without starting it (for data written before
        start() and marked after it)."""
        h = Handle()
        _check(lib().tc_plan_handle(self._p, C.byref(h)))
        return h

    def wait(self, timeout_s: float = 30.0):
        rc = lib().tc_plan_wait(self._p, int(timeout_s * 1e6))
        if rc in (_lib.ETIMEOUT, _lib.EEXTRA, _lib.ECORRUPT):
            _check(rc, self.problems())
        _check(rc)

    def next_round(self):
        _check(lib().tc_plan_next_round(self._p))

    # -- introspection
    @property
    def state(self) -> str:
        s, r = C.c_int(), C.c_uint32()
        _check(lib().tc_plan_state(self._p, C.byref(s), C.byref(r)))
        return _lib.STATE_NAMES[s.value]

    @property
    def round(self) -> int:
        s, r = C.c_int(), C.c_uint32()
        _check(lib().tc_plan_state(self._p, C.byref(s), C.byref(r)))
        return r.value

    def problems(self):
        n = C.c_uint32()
        _check(lib().tc_plan_problems(self._p, None, 0, C.byref(n)))
        buf = (C.c_uint32 * max(1, 2 * n.value))()
        _check(lib().tc_plan_problems(self._p, buf, n.value, C.byref(n)))
        return [(buf[2 * i], buf[2 * i + 1]) for i in range(n.value)]

    @property
    def G(self) -> int:
        return self.stats()["G"]

    def gates(self) -> np.ndarray:
        """[P, G, 64] uint8 snapshot of every gate table."""
        G = self.G
        out = np.zeros((self.P, G, GATE_ROW_BYTES), dtype=np.uint8)
        if G:
            _check(lib().tc_plan_read_gates(self._p, out.ctypes.data_as(C.c_void_p), out.nbytes))
        return out

    def cursors(self) -> np.ndarray:
        out = np.zeros((self.P, self.P), dtype=np.uint32)
        _check(lib().tc_plan_read_cursors(self._p, out.ctypes.data_as(C.POINTER(C.c_uint32))))
        return out

    def stats(self) -> dict:
        s = _lib.Stats()
        _check(lib().tc_plan_stats(self._p, C.byref(s)))
        return {k: getattr(s, k) for k, _ in s._fields_}

    def engine_stream(self) -> int:
        out = C.c_void_p()
        _check(lib().tc_plan_engine_stream(self._p, C.byref(out)))
        return out.value

    def debug_set_round(self, r: int):
        _check(lib().tc_plan_debug_set_round(self._p, r))

    # -- synthetic producers / consumer on this plan
    def fill(self, handle, views, seed, kind="u32", mark=True, serial=False, order=None,
             order_stride=0, waves=False, ctas=0, oneshot=False, stream=None):
        """Hash-fill producer.  serial: one CTA per rank in order[];
        waves: a persistent grid of `ctas` CTAs completing every rank's
        chunk 0, then every rank's chunk 1, ...; oneshot: one CTA per
        16 KiB block of every writer's share, in the waves order (plans of
        byte-range chunks and contiguous views only); otherwise one CTA per
        writer."""
        kinds = {"u32": FILL_U32, "bf16": FILL_BF16, "u8": FILL_U8}
        va = (View * self.P)(*[_as_view(v, None) for v in views])
        d = _lib.FillDesc()
        d.views = C.cast(va, C.POINTER(View))
        d.seed = seed
        d.kind = kinds[kind]
        d.mark_mode = MARK_INKERNEL if mark else MARK_NONE
        if serial + waves + oneshot > 1:
            raise ValueError("fill: pick one of serial, waves, oneshot")
        d.mode = (FILL_SERIAL if serial else FILL_WAVES if waves else
                  FILL_ONESHOT if oneshot else FILL_PARALLEL)
        d.order = order.data_ptr() if order is not None else None
        d.order_stride = order_stride
        d.ctas = ctas
        _check(lib().tc_produce_fill(self._p, C.byref(handle), C.byref(d), _stream_ptr(stream)))

    def mark_all(self, handle, stream=None):
        _check(lib().tc_mark_all(self._p, C.byref(handle), _stream_ptr(stream)))

    def mark(self, handle, rank, chunk, count=1, stream=None):
        _check(lib().tc_mark(self._p, C.byref(handle), rank, chunk, count, _stream_ptr(stream)))

    def row_deps(self, view, tile_rows=128):
        """(start [nblocks + 1], pairs [npairs, 2] = (src, chunk)) as uint32
        numpy: the chunks each block of tile_rows rows of ``view`` waits for."""
        v = _as_view(view, None)
        nb, npairs = C.c_uint32(), C.c_uint32()
        _check(lib().tc_plan_row_deps(self._p, C.byref(v), tile_rows, None, None, 0,
                                      C.byref(nb), C.byref(npairs)))
        start = np.zeros(nb.value + 1, dtype=np.uint32)
        pairs = np.zeros((max(1, npairs.value), 2), dtype=np.uint32)
        u32p = C.POINTER(C.c_uint32)
        _check(lib().tc_plan_row_deps(self._p, C.byref(v), tile_rows,
                                      start.ctypes.data_as(u32p), pairs.ctypes.data_as(u32p),
                                      npairs.value, C.byref(nb), C.byref(npairs)))
        return start, pairs[:npairs.value]

    def consume_copy(self, handle, dst, out, status, max_polls=1 << 20, stream=None):
        _check(lib().tc_consume_copy(self._p, C.byref(handle), dst, C.c_void_p(out.data_ptr()),
                                     max_polls, C.c_void_p(status.data_ptr()), _stream_ptr(stream)))


# -------------------------------------------------------------- producers

def prepare_all_gather(replicas, rows, cols, elem_bytes, schedules=None, writers=1, **plan_kw):
    """The in-place all-gather plan: rank p owns rows [p * rows, (p + 1) * rows)
    of a [P * rows, cols] buffer (one replica per rank), sends them as one
    whole() chunk with ``writers`` marks unless ``schedules`` are given, and
    the plan checks that no rank's schedule leaves its own rows.  Returns
    (plan, views)."""
    P = replicas.shape[0] if hasattr(replicas, "shape") and len(replicas.shape) == 2 else len(replicas)
    own = rows * cols * elem_bytes
    views = [View(p * own, rows, cols, cols, elem_bytes, 0) for p in range(P)]
    if schedules is None:
        schedules = [whole(v, writers) for v in views]
    return TriggeredPlan(replicas, schedules, own_rows_bytes=own, **plan_kw), views


def gemm_bf16(A, Bt, C_out, *, ldc=None, programs=256, group_m=8, handle=None, rank=0,
              first_chunk=0, tiles_per_chunk=256, M=None, N=None, stream=None):
    """C_out[M, N] (row stride ldc) = A[M, K] @ Bt[N, K].T in bf16 / fp32 acc.
    ``C_out`` may be any CUDA tensor whose data_ptr is the tile origin."""
    if not (A.is_contiguous() and Bt.is_contiguous()):
        raise InvalidArgument("gemm_bf16: A and Bt must be contiguous (row-major, K innermost)")
    M = M or A.shape[0]
    K = A.shape[1]
    N = N or Bt.shape[0]
    ldc = ldc or N
    h = C.byref(handle) if handle is not None else None
    _check(lib().tc_gemm_bf16(C.c_void_p(A.data_ptr()), C.c_void_p(Bt.data_ptr()),
                              C.c_void_p(C_out.data_ptr()), M, N, K, ldc, programs, group_m, h,
                              rank, first_chunk, tiles_per_chunk, _stream_ptr(stream)))


def gemm_consume_bf16(handle, dst, dep_start, dep_pairs, X, Wt, Y, *, M, N, K, ldx=None, ldy=None,
                      status=None, max_polls=1 << 20, programs=128, group_m=8, stream=None):
    """Y[M, N] = X[M, K] @ Wt[N, K].T where X is rank ``dst``'s replica of
    gathered rows; each 128-row block first waits for its chunks
    (``dep_start`` / ``dep_pairs``: device uint32 copies of
    ``TriggeredPlan.row_deps(view, 128)``)."""
    ptr = (lambda t: C.c_void_p(t.data_ptr()) if t is not None else None)
    _check(lib().tc_gemm_consume_bf16(C.byref(handle), dst, ptr(dep_start), ptr(dep_pairs), max_polls,
                                      ptr(status), ptr(X), ldx or K, ptr(Wt), ptr(Y), M, N, K, ldy or N,
                                      programs, group_m, _stream_ptr(stream)))


def barrier(W, P, first_gen, n_gen, status, *, x=None, y=None, snap=None, max_polls=1 << 22,
            stream=None):
    """Runs generations first_gen .. first_gen+n_gen-1 of the dedicated-row
    barrier on the int32 [P, P] CUDA tensor ``W`` (asynchronous)."""
    ptr = (lambda t: C.c_void_p(t.data_ptr()) if t is not None else None)
    _check(lib().tc_barrier_run(ptr(W), P, first_gen, n_gen, ptr(x), ptr(y), ptr(snap), max_polls,
                                ptr(status), _stream_ptr(stream)))
