"""The dedicated-row notify/wait barrier, sequentially (oracle side).

After "Barrier: Signals Only" (pypto documentation), sections *The idea*,
*Walkthrough* and *Edge cases*: every rank adds 1 (AtomicAdd) to the cell of
its own row in every other rank's signal window, then waits until each other
row of its own window reaches the threshold (Ge).  A rank never notifies
itself, so after one barrier rank r's window reads 1 everywhere except 0 in
its own row.  The counters are monotonic, so a reused window takes a
per-generation threshold: generation g waits for ``>= g``.

Reading for P simulated ranks on one device: the P windows are stacked as
``W[P, P]`` int32, ``W[q, s]`` = the cell of row s in rank q's window, written
only by rank s.

The data reveal of the same page (each rank writes its own slot, all pass
the barrier, each then picks up its right-hand neighbour's slot, so that
y[r] = x[(r + 1) % N]) is
kept with a double-buffered stage ``x[g % 2][m]`` so that generations can
follow each other without a second barrier.
"""

import numpy as np


def run(P: int, n_gen: int, first_gen: int = 1, W: np.ndarray = None):
    """Sequential barrier: every rank notifies, then every wait must pass.
    Returns W after generations first_gen .. first_gen + n_gen - 1."""
    if W is None:
        W = np.zeros((P, P), dtype=np.int64)
    W = W.astype(np.int64, copy=True)
    for g in range(first_gen, first_gen + n_gen):
        for m in range(P):                          # notify phase of rank m
            for q in range(P):
                if q != m:
                    W[q, m] += 1
        for m in range(P):                          # wait phase of rank m
            for s in range(P):
                if s != m and not W[m, s] >= g:
                    raise AssertionError(f"rank {m} would wait forever on row {s}")
    return W


def closed_form(P: int, gens: int) -> np.ndarray:
    """W after ``gens`` generations from zero: g everywhere off the diagonal."""
    return gens * (np.ones((P, P), dtype=np.int64) - np.eye(P, dtype=np.int64))


def stage_value(g: int, m: int) -> int:
    """Value rank m stages in generation g for the data reveal (any value
    distinct per (g, m) works; this one fits int32 for g < 2**23)."""
    return (g << 8) | m


def reveal(P: int, first_gen: int, n_gen: int) -> np.ndarray:
    """y[g - first_gen, m] = the value rank (m + 1) % P staged in generation g."""
    y = np.zeros((n_gen, P), dtype=np.int64)
    for i, g in enumerate(range(first_gen, first_gen + n_gen)):
        for m in range(P):
            y[i, m] = stage_value(g, (m + 1) % P)
    return y
