"""Which chunks a consumer of the gathered rows must wait for (oracle side).

After "Triggered Plans" (Iris documentation), sections *Memory ordering*
(consumer side: read a chunk only after its arrival) and *Model* (a chunk is
a group of regions landing at the same offsets in every peer's buffer).  A
consumer that reads the rows of a view of the gathered buffer in blocks of
``tile_rows`` rows must wait, before a block, for every chunk with a byte in
those rows.  The exact set, computed from byte intervals.

The reference for the consumer's arithmetic is ``oracle.gemm.gemm_ref`` on
the gathered rows.
"""

from typing import List, Optional, Sequence, Tuple

from .schedule import Schedule, View, region_intervals


def row_block_intervals(v: View, tile_rows: int) -> List[List[Tuple[int, int]]]:
    """Per block of tile_rows rows of the view: its rows' byte intervals."""
    e, pitch = v.elem_bytes, v.row_stride * v.elem_bytes
    nb = -(-v.rows // tile_rows)
    out = []
    for b in range(nb):
        rows = range(b * tile_rows, min(v.rows, (b + 1) * tile_rows))
        out.append([(v.byte_offset + r * pitch, v.byte_offset + r * pitch + v.cols * e) for r in rows])
    return out


def row_deps(schedules: Sequence[Optional[Schedule]], v: View,
             tile_rows: int) -> List[List[Tuple[int, int]]]:
    """deps[b] = sorted (rank, chunk) pairs with a byte in block b's rows."""
    blocks = row_block_intervals(v, tile_rows)
    deps = []
    for ivs in blocks:
        lo, hi = ivs[0][0], ivs[-1][1]
        found = []
        for p, s in enumerate(schedules):
            if s is None:
                continue
            for c, ch in enumerate(s.chunks):
                hit = False
                for reg in ch.regions:
                    for a, b in region_intervals(reg):
                        if b <= lo or a >= hi:
                            continue
                        if any(a < y and x < b for x, y in ivs):
                            hit = True
                            break
                    if hit:
                        break
                if hit:
                    found.append((p, c))
        deps.append(sorted(found))
    return deps
