"""Oracle of one sharded step Arg -> Compute(A) -> sparse exchange -> Compute(B) -> Result.

Test infrastructure only (see the package docstring).

Source: the PATHWAYS page ("PATHWAYS: Asynchronous Distributed Dataflow for
ML"), section 4.3 "Coordination implementation": a chain of two N-sharded
computations is the four-node graph Arg -> Compute(A) -> Compute(B) -> Result;
every node emits output tuples tagged with a destination shard; the runtime
sends messages among dynamically chosen subsets of shards along the sharded
edge and uses progress tracking to decide when a shard has received all of
its messages. Sections 4.4 and 4.5: computations take buffer futures as
inputs and a successor starts once its input future is ready.

Readings where the page is silent (each also listed in the design notes):
  * order inside a destination: stable in global source order
    g = s * T + i (source shard, then position);
  * completion is count based: the expected count of destination d is the
    number of tuples tagged d; its future fires when that many arrived, and
    fires with an empty segment when the count is 0;
  * one destination per tuple; the payload row is the routing unit.

The result is a stable sort of the tuples by destination, a plain definition
with exactly one correct output; it is written out here as a counting sort
(count -> exclusive scan -> place in order).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .numerics import to_f32

# Node ids of the step graph, in topological order.
ARG, A, EXCH, B, RESULT = "Arg", "A", "exchange", "B", "Result"


# --------------------------------------------------------------------------
# Elementwise node bodies (the workloads' A and B)
# --------------------------------------------------------------------------

def op_identity():
    return ("identity",)


def op_affine(a: float, b: float):
    """y = a * x + b, evaluated in fp64 and rounded once to fp32."""
    return ("affine", float(a), float(b))


def op_rowsum():
    """One value per tuple: the sum of its payload, fp64 then rounded to fp32."""
    return ("rowsum",)


def apply_op(op, x32: np.ndarray) -> np.ndarray:
    """Apply an elementwise node body to fp32 tuples ``x32`` [n, P]."""
    kind = op[0]
    if kind == "identity":
        return np.array(x32, dtype=np.float32, copy=True)
    if kind == "affine":
        a, b = op[1], op[2]
        return to_f32(np.float64(a) * x32.astype(np.float64) + np.float64(b))
    if kind == "rowsum":
        return to_f32(x32.astype(np.float64).sum(axis=1))
    raise ValueError(f"unknown op {op!r}")


# --------------------------------------------------------------------------
# Histogram, exclusive scan, stable placement
# --------------------------------------------------------------------------

def check_dest(dest: np.ndarray, num_dest: int) -> None:
    if dest.size and (dest.min() < 0 or dest.max() >= num_dest):
        raise ValueError("destination outside [0, num_dest)")


def histogram(dest: np.ndarray, num_dest: int, num_src: int, tuples_per_src: int) -> np.ndarray:
    """counts[s][d] = number of tuples of source shard s tagged with destination d."""
    check_dest(dest, num_dest)
    assert dest.size == num_src * tuples_per_src
    counts = np.zeros((num_src, num_dest), dtype=np.int64)
    for s in range(num_src):
        seg = dest[s * tuples_per_src:(s + 1) * tuples_per_src]
        counts[s] = np.bincount(seg, minlength=num_dest)[:num_dest]
    return counts


def exclusive_scan(totals: np.ndarray) -> np.ndarray:
    """offsets[0] = 0, offsets[d + 1] = offsets[d] + totals[d]  (length N + 1)."""
    offsets = np.zeros(len(totals) + 1, dtype=np.int64)
    for d in range(len(totals)):
        offsets[d + 1] = offsets[d] + int(totals[d])
    return offsets


def stable_place(dest: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """src_index: the slots of destination d, offsets[d] .. offsets[d+1]-1, hold the
    global indices of the tuples tagged d in ascending source order."""
    num_dest = len(offsets) - 1
    src_index = np.empty(dest.size, dtype=np.int64)
    for d in range(num_dest):
        idx = np.flatnonzero(dest == d)
        if idx.size != offsets[d + 1] - offsets[d]:
            raise AssertionError("count / placement mismatch")
        src_index[offsets[d]:offsets[d + 1]] = idx
    return src_index


# --------------------------------------------------------------------------
# Futures: a table of (node, shard) -> epoch with exactly-once firing
# --------------------------------------------------------------------------

@dataclass
class FutureTable:
    """Buffer futures of the step graph. A future fires at most once per
    (node, shard, epoch); consumers may read a buffer only after its future
    fired (sections 4.4-4.5 of the dataflow page)."""
    epoch: int = 1
    fired: dict = field(default_factory=dict)     # (node, shard) -> epoch
    fire_count: dict = field(default_factory=dict)  # (node, shard, epoch) -> count
    order: list = field(default_factory=list)     # firing order

    def fire(self, node, shard):
        key = (node, shard, self.epoch)
        n = self.fire_count.get(key, 0)
        if n:
            raise AssertionError(f"future {key} fired twice")
        self.fire_count[key] = 1
        self.fired[(node, shard)] = self.epoch
        self.order.append((node, shard))

    def ready(self, node, shard) -> bool:
        return self.fired.get((node, shard)) == self.epoch

    def require(self, node, shard):
        if not self.ready(node, shard):
            raise AssertionError(f"read of {node}[{shard}] before its future fired")


# --------------------------------------------------------------------------
# The step
# --------------------------------------------------------------------------

@dataclass
class ExchangeResult:
    y: np.ndarray            # [G, P] exchanged A(x) rows, destination-major
    src_index: np.ndarray    # [G] int64, global source index of each slot
    counts: np.ndarray       # [num_src, N] int64
    offsets: np.ndarray      # [N + 1] int64
    expected: np.ndarray     # [N] int64
    b_out: np.ndarray | None # B's output (rowsum: [G]; affine: [G, P]) or None
    futures: FutureTable
    arrived_at_fire: dict    # destination -> arrivals counted when its future fired


def exchange_step(x: np.ndarray, dest: np.ndarray, num_dest: int, num_src: int,
                  a_op=op_identity(), b_op=None, epoch: int = 1) -> ExchangeResult:
    """Run Arg -> A -> exchange -> B -> Result sequentially, node by node and
    shard by shard, over a future table.

    x: [G, P] fp32 tuples, shard-major (tuple g = s*T + i, T = G / num_src);
    dest: [G] int.
    """
    g_total = dest.size
    if x.shape[0] != g_total or num_src <= 0 or g_total % num_src:
        raise ValueError("x / dest / num_src shapes disagree")
    T = g_total // num_src
    ft = FutureTable(epoch=epoch)

    # Arg: the caller's sharded buffer is bound; its per-shard futures are ready.
    for s in range(num_src):
        ft.fire(ARG, s)

    # Compute(A): per source shard, gated on the Arg future.
    ax = np.empty_like(x, dtype=np.float32)
    for s in range(num_src):
        ft.require(ARG, s)
        ax[s * T:(s + 1) * T] = apply_op(a_op, x[s * T:(s + 1) * T])
        ft.fire(A, s)

    # Destination tags -> per-destination expected totals and segment offsets.
    counts = histogram(dest, num_dest, num_src, T)
    expected = counts.sum(axis=0)
    offsets = exclusive_scan(expected)
    src_index = stable_place(dest, offsets)

    # Progress tracking: destinations expecting nothing are complete at once;
    # others complete when their arrivals reach the expected count. Sources
    # deliver in order; each source's tuples for d form one batched message.
    arrived = np.zeros(num_dest, dtype=np.int64)
    arrived_at_fire = {}
    for d in range(num_dest):
        if expected[d] == 0:
            arrived_at_fire[d] = 0
            ft.fire(EXCH, d)
    for s in range(num_src):
        ft.require(A, s)
    y = ax[src_index]                       # the tuples land in their slots ...
    for s in range(num_src):                # ... and are counted per (source, destination) batch
        for d in np.flatnonzero(counts[s]):
            arrived[d] += counts[s][d]
            if arrived[d] == expected[d]:
                arrived_at_fire[int(d)] = int(arrived[d])
                ft.fire(EXCH, int(d))

    # Compute(B): per destination shard, gated on its exchange future.
    b_out = None
    if b_op is not None:
        parts = []
        for d in range(num_dest):
            ft.require(EXCH, d)
            parts.append(apply_op(b_op, y[offsets[d]:offsets[d + 1]]))
            ft.fire(B, d)
        b_out = np.concatenate(parts) if parts else np.zeros(0, np.float32)
    else:
        for d in range(num_dest):
            ft.require(EXCH, d)
            ft.fire(B, d)

    # Result: complete once every B shard is.
    for d in range(num_dest):
        ft.require(B, d)
    ft.fire(RESULT, -1)
    return ExchangeResult(y, src_index, counts, offsets, expected, b_out, ft, arrived_at_fire)
