"""Step-by-step simulation of a triggered plan on P simulated ranks (oracle).

What is simulated, after "Triggered Plans":

* *Model*: a round is ``start()``, every chunk marked ready by its writers,
  ``wait()``; one plan serves every round, set up once.
* *Gates and rounds*: a chunk's 64-byte gate row carries ``ready``,
  ``arrival`` and the count of writers' marks; the copy side compares the
  lower half of ``ready`` with the round using ``>=``; the first round is 1,
  each ``next_round()`` adds 1 and nothing ever clears a gate, hence at most
  2**32 - 1 rounds per plan.
* *Memory ordering*: the writer counter is incremented once per mark; the
  writer whose increment completes the round's count opens the gate by
  writing the round number into ``ready``.
* The diagram at the top of the page and "Triggered SDMA Plans", *Design
  notes*: per peer, one queue that runs, in prepared order, for each chunk:
  poll ``ready >= round``, copy every region, add 1 to the chunk's arrival
  counter on that peer.
* *The kernel author's contract*: a queue keeps its prepared order (a chunk
  that finishes early still waits behind those listed before it); ``wait()`` raises on extra
  marks, and a timeout reports which chunks are still missing marks or copies.

Readings (where the pages are silent):

* gate row: ``ready`` u64 at byte 0, ``arrival`` u64 at byte 8, writer
  counter u64 at byte 16, bytes 24..63 zero; little-endian;
* the writer counter is cumulative: the last writer of round r is the one
  whose increment makes it r * writers;
* a rank's own chunk gets no arrival (nothing is copied to itself);
* an extra mark is reported at that round's ``wait()``, which moves the plan
  to FAILED; a timeout leaves it STARTED, so a later mark and ``wait()`` can
  still succeed;
* the queue cursor ``cur[p][q]`` counts chunks of rank p delivered to q this
  round and is reset by ``start()``.
"""

from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

from .schedule import Schedule, ScheduleError, validate

ROUND_LIMIT = (1 << 32) - 1
GATE_ROW_BYTES = 64
GATE_WORDS = GATE_ROW_BYTES // 8
READY, ARRIVAL, WRITERS = 0, 1, 2          # u64 word index in a gate row

READY_STATE, STARTED, DONE, FAILED, CLOSED = "READY", "STARTED", "DONE", "FAILED", "CLOSED"


class PlanError(Exception):
    def __init__(self, code: str, msg: str = "", chunks: Sequence[Tuple[int, int]] = ()):
        super().__init__(f"{code}: {msg}")
        self.code = code
        self.chunks = list(chunks)


def copy_region(dst: np.ndarray, src: np.ndarray, reg) -> None:
    """Copy one region's bytes from ``src`` to ``dst`` at the same offsets."""
    off, rows, row_bytes, pitch = reg
    for i in range(rows):
        a = off + i * pitch
        dst[a:a + row_bytes] = src[a:a + row_bytes]


class PlanSim:
    """P replicas (uint8 numpy arrays of equal size), one schedule per rank.

    With ``replicas=None`` (and ``buffer_bytes`` given) only gates, cursors
    and delivery logs are simulated: the copies are skipped, which changes no
    counter (counters never depend on the bytes copied)."""

    def __init__(self, replicas: Optional[List[np.ndarray]], schedules: Sequence[Optional[Schedule]],
                 own_rows_bytes: Optional[int] = None, buffer_bytes: Optional[int] = None):
        self.P = len(replicas) if replicas is not None else len(schedules)
        if self.P == 0 or len(schedules) != self.P:
            raise PlanError("EINVAL", "one schedule per rank")
        if replicas is None:
            size = buffer_bytes
        else:
            size = replicas[0].size
            if any(r.size != size for r in replicas):
                raise PlanError("EINVAL", "replicas differ in size")
        try:
            validate(size, schedules, own_rows_bytes)
        except ScheduleError as e:
            raise PlanError(e.code, str(e)) from None
        self.rep = replicas
        self.sched = [s if s is not None else Schedule() for s in schedules]
        self.n = [len(s.chunks) for s in self.sched]
        self.base = np.concatenate([[0], np.cumsum(self.n)]).astype(int).tolist()
        self.G = self.base[-1]
        # gates[q, g] = 64-byte row of global chunk g in rank q's gate table
        self.gates = np.zeros((self.P, self.G, GATE_WORDS), dtype=np.uint64)
        self.cur = np.zeros((self.P, self.P), dtype=np.uint32)
        self.round = 1
        self.state = READY_STATE
        self.log: Dict[Tuple[int, int], List[int]] = {}

    # ------------------------------------------------------------ helpers
    def g(self, p: int, c: int) -> int:
        return self.base[p] + c

    def writers(self, p: int, c: int) -> int:
        return self.sched[p].chunks[c].writers

    # -------------------------------------------------------------- round
    def start(self) -> int:
        if self.state != READY_STATE:
            raise PlanError("ESTATE", f"start() in state {self.state}")
        self.state = STARTED
        self.cur[:] = 0
        self.log = {(p, q): [] for p in range(self.P) for q in range(self.P) if p != q}
        return self.round

    def mark(self, p: int, c: int, advance: bool = True) -> None:
        """One ``mark_ready`` by one writer of rank p's chunk c."""
        if self.state != STARTED:
            raise PlanError("ESTATE", "mark outside a started round")
        row = self.gates[p, self.g(p, c)]
        row[WRITERS] += np.uint64(1)
        if int(row[WRITERS]) == self.round * self.writers(p, c):
            row[READY] = np.uint64(self.round)
        if advance:
            self.advance()

    def gate_open(self, p: int, c: int) -> bool:
        ready_lo = int(self.gates[p, self.g(p, c), READY]) & 0xFFFFFFFF
        return ready_lo >= self.round

    def step_queue(self, p: int, q: int) -> bool:
        """Run the head of queue p->q once if its gate is open."""
        c = int(self.cur[p, q])
        if c >= self.n[p] or not self.gate_open(p, c):
            return False
        if self.rep is not None:
            for reg in self.sched[p].chunks[c].regions:
                copy_region(self.rep[q], self.rep[p], reg)
        self.gates[q, self.g(p, c), ARRIVAL] += np.uint64(1)
        self.cur[p, q] = c + 1
        self.log[(p, q)].append(c)
        return True

    def advance(self) -> None:
        """Run every queue until no head gate is open (a fixed point)."""
        progressed = True
        while progressed:
            progressed = False
            for p in range(self.P):
                for q in range(self.P):
                    if p != q:
                        while self.step_queue(p, q):
                            progressed = True

    def problems(self) -> Tuple[List[Tuple[int, int]], List[Tuple[int, int]]]:
        """(extra, short) lists of (rank, chunk) as ``wait()`` sees them."""
        extra, short = [], []
        r = self.round
        for p in range(self.P):
            for c in range(self.n[p]):
                g = self.g(p, c)
                own = self.gates[p, g]
                want = r * self.writers(p, c)
                if int(own[WRITERS]) > want:
                    extra.append((p, c))
                    continue
                arrived = all(int(self.gates[q, g, ARRIVAL]) >= r
                              for q in range(self.P) if q != p)
                if int(own[WRITERS]) < want or (int(own[READY]) & 0xFFFFFFFF) < r or not arrived:
                    short.append((p, c))
        return extra, short

    def wait(self) -> None:
        if self.state != STARTED:
            raise PlanError("ESTATE", f"wait() in state {self.state}")
        self.advance()
        extra, short = self.problems()
        if extra:
            self.state = FAILED
            raise PlanError("EEXTRA", "chunks got extra marks", extra)
        if short:
            raise PlanError("ETIMEOUT", "chunks still short", short)
        self.state = DONE

    def next_round(self) -> None:
        if self.state != DONE:
            raise PlanError("ESTATE", f"next_round() in state {self.state}")
        if self.round >= ROUND_LIMIT:
            raise PlanError("EROUNDS", "round limit reached")
        self.round += 1
        self.state = READY_STATE

    def close(self) -> None:
        self.state = CLOSED

    # ---------------------------------------------------------- snapshots
    def gate_bytes(self) -> np.ndarray:
        """All gate tables as bytes, [P, G, 64], little-endian."""
        return self.gates.astype("<u8").view(np.uint8).reshape(self.P, self.G, GATE_ROW_BYTES)


def run_round(sim: PlanSim, produce: Callable[[int, int], None],
              mark_order: Optional[Sequence[Tuple[int, int]]] = None,
              extra_marks: Sequence[Tuple[int, int]] = (),
              withheld: Sequence[Tuple[int, int]] = ()) -> None:
    """One round: start; every rank writes its block (``produce(p, round)``);
    the writers' marks are applied in ``mark_order`` (default: rank-major,
    schedule order, all writers of a chunk together) plus ``extra_marks``,
    minus one mark per entry of ``withheld``; then ``wait()``."""
    sim.start()
    for p in range(sim.P):
        produce(p, sim.round)
    if mark_order is None:
        mark_order = [(p, c) for p in range(sim.P) for c in range(sim.n[p])
                      for _ in range(sim.writers(p, c))]
    marks = list(mark_order)
    for pc in withheld:
        marks.remove(pc)
    marks.extend(extra_marks)
    for p, c in marks:
        sim.mark(p, c)
    sim.wait()


def expected_after_round(schedules, blocks: List[np.ndarray], before: List[np.ndarray]):
    """The plain definition of the result of a complete round: replica q is
    its earlier content ``before[q]`` with, at every byte of rank p's regions,
    rank p's produced byte (``blocks[p]`` is replica p after its producer ran;
    only its region bytes are used).  Bytes in no region keep their earlier
    value.  No two ranks share a byte, so the order over p does not matter."""
    out = []
    for q in range(len(before)):
        rq = before[q].copy()
        for p, s in enumerate(schedules):
            if s is None:
                continue
            for ch in s.chunks:
                for reg in ch.regions:
                    copy_region(rq, blocks[p], reg)
        out.append(rq)
    return out
