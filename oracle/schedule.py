"""Regions, chunks and schedules (oracle side).

Follows "Triggered Plans", section *Model*: a *region* is the unit of one
copy (bytes back to back, or a 2-D window of a strided tensor) and lands at
the identical offset in every peer's buffer; a *chunk* bundles regions, in order,
under one writers count; a *schedule* is one rank's list of chunks in the
order its producer finishes them.  The
builders ``whole``, ``chunks`` and ``tile_chunks`` and the 1 GiB split of
linear copies come from the same section and from *Requirements and limits*.
Validation follows *The kernel author's contract* (a failed create keeps
nothing) and *Requirements and limits* (no byte may be sent by two
different ranks); the own-rows check is the all-gather wrapper's, described at the end
of *Model*.

Readings where the pages are silent (each listed in the design notes):

* normal form: a region is ``(offset, rows, row_bytes, pitch)``; it is linear
  (``rows == 1``, ``pitch == row_bytes``) when it has one row or its rows are
  back to back; otherwise 2-D;
* linear regions are cut into pieces of exactly 2**30 bytes from the start,
  remainder last; a 2-D region over 2**30 bytes is cut into groups of whole
  rows of at most 2**30 bytes (each group normalised again);
* ``chunks(n)`` uses the tensor_split rule (the first ``rows % n`` blocks get
  one extra row) and rejects ``n > rows``;
* ``tile_chunks`` gives each chunk one writer per tile it holds (the producer
  marks once per step), and defaults ``order`` to row-major;
* the grouped step->tile order (the body the page elides for ``tile_of``) is
  the usual GROUP_M swizzle written out in ``tile_of`` below.
"""

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

GIB = 1 << 30

# Error codes shared in meaning (not in code) with the C boundary.
EINVAL = "EINVAL"
EBOUNDS = "EBOUNDS"
EOVERLAP = "EOVERLAP"


class ScheduleError(Exception):
    def __init__(self, code: str, msg: str = ""):
        super().__init__(f"{code}: {msg}")
        self.code = code


@dataclass(frozen=True)
class View:
    """A 2-D window of the base buffer: rows x cols elements, row stride in
    elements, starting ``byte_offset`` bytes into the buffer (``base=out``)."""
    byte_offset: int
    rows: int
    cols: int
    row_stride: int
    elem_bytes: int


Region = Tuple[int, int, int, int]          # (offset, rows, row_bytes, pitch)


@dataclass
class Chunk:
    regions: List[Region]
    writers: int


@dataclass
class Schedule:
    chunks: List[Chunk] = field(default_factory=list)

    def tables(self):
        """Flattened (chunk table, region table) in the boundary's layout:
        chunk = (first_region, num_regions, writers)."""
        ct, rt = [], []
        for ch in self.chunks:
            ct.append((len(rt), len(ch.regions), ch.writers))
            rt.extend(ch.regions)
        return ct, rt


def _normal(off: int, rows: int, row_bytes: int, pitch: int) -> Region:
    if rows == 1 or row_bytes == pitch:
        n = rows * row_bytes
        return (off, 1, n, n)
    return (off, rows, row_bytes, pitch)


def split_region(reg: Region) -> List[Region]:
    """Apply the 1 GiB rule to one normal-form region."""
    off, rows, row_bytes, pitch = reg
    if rows == 1:
        n = row_bytes
        return [(off + k, 1, min(GIB, n - k), min(GIB, n - k)) for k in range(0, n, GIB)]
    if rows * row_bytes <= GIB:
        return [reg]
    if row_bytes > GIB:                      # every row alone is over the cap
        out = []
        for i in range(rows):
            out.extend(split_region((off + i * pitch, 1, row_bytes, row_bytes)))
        return out
    per = GIB // row_bytes
    out = []
    for i in range(0, rows, per):
        g = _normal(off + i * pitch, min(per, rows - i), row_bytes, pitch)
        out.extend(split_region(g))
    return out


def window_regions(v: View, r0: int, r1: int, c0: int, c1: int) -> List[Region]:
    """Regions covering rows [r0, r1) x cols [c0, c1) of view ``v``."""
    if not (0 <= r0 < r1 <= v.rows and 0 <= c0 < c1 <= v.cols):
        raise ScheduleError(EINVAL, "empty or out-of-view window")
    e = v.elem_bytes
    off = v.byte_offset + (r0 * v.row_stride + c0) * e
    return split_region(_normal(off, r1 - r0, (c1 - c0) * e, v.row_stride * e))


def _check_view(v: View):
    if v.rows == 0 or v.cols == 0 or v.elem_bytes == 0 or v.row_stride < v.cols:
        raise ScheduleError(EINVAL, "bad view")


def whole(v: View, writers: int = 1) -> Schedule:
    """One chunk holding the whole view; ``writers`` = programs that mark it."""
    _check_view(v)
    if writers == 0:
        raise ScheduleError(EINVAL, "writers must be positive")
    return Schedule([Chunk(window_regions(v, 0, v.rows, 0, v.cols), writers)])


def row_blocks(rows: int, n: int) -> List[Tuple[int, int]]:
    """tensor_split rule: n blocks, the first rows % n one row longer."""
    if n == 0 or n > rows:
        raise ScheduleError(EINVAL, "need 1 <= n <= rows")
    q, r = divmod(rows, n)
    out, start = [], 0
    for k in range(n):
        size = q + (1 if k < r else 0)
        out.append((start, start + size))
        start += size
    return out


def chunks(v: View, n: int, writers: int = 1) -> Schedule:
    """One chunk per row block, completed in order."""
    _check_view(v)
    if writers == 0:
        raise ScheduleError(EINVAL, "writers must be positive")
    return Schedule([Chunk(window_regions(v, a, b, 0, v.cols), writers)
                     for a, b in row_blocks(v.rows, n)])


def tile_of(step: int, tiles_m: int, tiles_n: int, group_m: int) -> int:
    """Grouped step->tile order: walk ``group_m`` tile-rows column by column
    before moving to the next band of rows."""
    width = group_m * tiles_n
    group = step // width
    first_m = group * group_m
    size_m = min(tiles_m - first_m, group_m)
    tm = first_m + (step % width) % size_m
    tn = (step % width) // size_m
    return tm * tiles_n + tn


def tile_chunks(v: View, bm: int, bn: int, tiles_per_chunk: int,
                order: Optional[Sequence[int]] = None) -> Schedule:
    """One region per tile (clipped at the edges); consecutive steps grouped
    ``tiles_per_chunk`` at a time; ``order[step]`` is the producer's tile."""
    _check_view(v)
    if bm == 0 or bn == 0 or tiles_per_chunk == 0:
        raise ScheduleError(EINVAL, "zero tile or chunk size")
    tm_count = -(-v.rows // bm)
    tn_count = -(-v.cols // bn)
    nt = tm_count * tn_count
    if order is None:
        order = list(range(nt))
    order = list(order)
    if len(order) != nt or sorted(order) != list(range(nt)):
        raise ScheduleError(EINVAL, "order is not a permutation of the tiles")
    out = []
    for k in range(0, nt, tiles_per_chunk):
        steps = range(k, min(nt, k + tiles_per_chunk))
        regs = []
        for s in steps:
            t = order[s]
            tm, tn = divmod(t, tn_count)
            regs.extend(window_regions(v, tm * bm, min(v.rows, (tm + 1) * bm),
                                       tn * bn, min(v.cols, (tn + 1) * bn)))
        out.append(Chunk(regs, len(steps)))
    return Schedule(out)


def from_tables(chunk_table, region_table) -> Schedule:
    """A hand-built schedule: (first_region, num_regions, writers) rows over a
    region table.  Chunks must cover the region table in order."""
    out, pos = [], 0
    for first, num, w in chunk_table:
        if first != pos or num == 0 or w == 0:
            raise ScheduleError(EINVAL, "chunk table must tile the region table")
        regs = []
        for r in region_table[first:first + num]:
            off, rows, row_bytes, pitch = r
            if rows == 0 or row_bytes == 0 or (rows > 1 and pitch < row_bytes):
                raise ScheduleError(EINVAL, "bad region")
            regs.extend(split_region(_normal(off, rows, row_bytes, pitch)))
        out.append(Chunk(regs, w))
        pos += num
    if pos != len(region_table):
        raise ScheduleError(EINVAL, "regions left over")
    return Schedule(out)


# ----------------------------------------------------------------- validation

def region_intervals(reg: Region) -> List[Tuple[int, int]]:
    """Half-open byte intervals of one region, one per row."""
    off, rows, row_bytes, pitch = reg
    return [(off + i * pitch, off + i * pitch + row_bytes) for i in range(rows)]


def _merged(intervals):
    out = []
    for a, b in sorted(intervals):
        if out and a <= out[-1][1]:
            out[-1][1] = max(out[-1][1], b)
        else:
            out.append([a, b])
    return out


def _intersects(xs, ys) -> bool:
    i = j = 0
    while i < len(xs) and j < len(ys):
        a0, a1 = xs[i]
        b0, b1 = ys[j]
        if a0 < b1 and b0 < a1:
            return True
        if a1 <= b1:
            i += 1
        else:
            j += 1
    return False


def validate(buffer_bytes: int, schedules: Sequence[Optional[Schedule]],
             own_rows_bytes: Optional[int] = None) -> None:
    """Plan-creation checks; raises ScheduleError and keeps nothing.

    * every chunk has writers > 0 and at least one region (EINVAL);
    * every region byte lies inside [0, buffer_bytes) (EBOUNDS);
    * with ``own_rows_bytes``: rank p's bytes lie in its rows
      [p*own_rows_bytes, (p+1)*own_rows_bytes) (EBOUNDS);
    * no byte is sent by two ranks (EOVERLAP).  One rank may repeat bytes.
    """
    per_rank = []
    for p, s in enumerate(schedules):
        ivs = []
        for ch in (s.chunks if s is not None else []):
            if ch.writers == 0 or not ch.regions:
                raise ScheduleError(EINVAL, f"rank {p}: chunk without writers or regions")
            for reg in ch.regions:
                off, rows, row_bytes, pitch = reg
                if rows == 0 or row_bytes == 0 or (rows > 1 and pitch < row_bytes):
                    raise ScheduleError(EINVAL, f"rank {p}: bad region {reg}")
                end = off + (rows - 1) * pitch + row_bytes
                if off < 0 or end > buffer_bytes:
                    raise ScheduleError(EBOUNDS, f"rank {p}: region {reg} outside buffer")
                if own_rows_bytes is not None:
                    lo, hi = p * own_rows_bytes, (p + 1) * own_rows_bytes
                    if off < lo or end > hi:
                        raise ScheduleError(EBOUNDS, f"rank {p}: region {reg} outside own rows")
                ivs.extend(region_intervals(reg))
        per_rank.append(_merged(ivs))
    for p in range(len(per_rank)):
        for q in range(p + 1, len(per_rank)):
            if _intersects(per_rank[p], per_rank[q]):
                raise ScheduleError(EOVERLAP, f"ranks {p} and {q} send the same bytes")
