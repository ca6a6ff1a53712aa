"""Invariant checkers for exchange outputs and future tables (test infrastructure only).

They state, independently of how an exchange was computed, what any correct
result must satisfy (PATHWAYS page, section 4.3: tuples tagged with a
destination are delivered to that destination; a shard's input is complete
once all of its messages arrived; plus the stable reading of the order):

  * src_index is a permutation of [0, G);
  * destinations along the output are non-decreasing and segment d spans
    offsets[d] .. offsets[d+1];
  * inside a segment, source indices ascend (stability);
  * counts sum to G and their column sums are the segment lengths;
  * each output row equals A applied to the row it came from;
  * every future fired exactly once, and only when the expected count had
    arrived.

Each checker raises AssertionError with a message naming the first breach.
"""
from __future__ import annotations

import numpy as np


def check_exchange(dest, num_dest, src_index, offsets, counts=None, y=None, ax=None) -> None:
    dest = np.asarray(dest).astype(np.int64)
    src_index = np.asarray(src_index).astype(np.int64)
    offsets = np.asarray(offsets).astype(np.int64)
    g = dest.size
    if src_index.size != g:
        raise AssertionError(f"src_index has {src_index.size} entries, expected {g}")
    if offsets.size != num_dest + 1 or offsets[0] != 0 or offsets[-1] != g:
        raise AssertionError("offsets do not span [0, G]")
    if np.any(np.diff(offsets) < 0):
        raise AssertionError("offsets decrease")
    if g:
        if src_index.min() < 0 or src_index.max() >= g:
            raise AssertionError("src_index out of range")
        seen = np.zeros(g, dtype=np.int64)
        np.add.at(seen, src_index, 1)
        if np.any(seen != 1):
            bad = int(np.flatnonzero(seen != 1)[0])
            raise AssertionError(f"src_index is not a permutation (tuple {bad} appears {seen[bad]} times)")
        seg_of_slot = np.repeat(np.arange(num_dest), np.diff(offsets))
        d_at = dest[src_index]
        if np.any(d_at != seg_of_slot):
            j = int(np.flatnonzero(d_at != seg_of_slot)[0])
            raise AssertionError(f"slot {j} holds a tuple for destination {d_at[j]} inside segment {seg_of_slot[j]}")
        same = seg_of_slot[1:] == seg_of_slot[:-1]
        if np.any(same & (src_index[1:] <= src_index[:-1])):
            j = int(np.flatnonzero(same & (src_index[1:] <= src_index[:-1]))[0])
            raise AssertionError(f"source order broken inside a segment at slot {j}")
    if counts is not None:
        counts = np.asarray(counts).astype(np.int64)
        if counts.sum() != g:
            raise AssertionError("counts do not sum to G")
        if np.any(counts.sum(axis=0) != np.diff(offsets)):
            raise AssertionError("count columns disagree with segment lengths")
    if y is not None and ax is not None and g:
        yv = np.asarray(y).reshape(g, -1).view(np.uint32)
        av = np.asarray(ax).reshape(g, -1).view(np.uint32)
        if not np.array_equal(yv, av[src_index]):
            j = int(np.flatnonzero(np.any(yv != av[src_index], axis=1))[0])
            raise AssertionError(f"payload of slot {j} is not the bits of its source row")


def check_fires(fire_count, expected_fires=1) -> None:
    """Every (node, shard) fired exactly ``expected_fires`` times."""
    fc = np.asarray(fire_count)
    if np.any(fc != expected_fires):
        j = np.argwhere(fc != expected_fires)[0]
        raise AssertionError(f"future {tuple(int(v) for v in j)} fired {fc[tuple(j)]} times, expected {expected_fires}")


def check_futures_at_fire(arrived_at_fire: dict, expected) -> None:
    """Each destination's future fired only when its expected count had arrived."""
    expected = np.asarray(expected)
    for d in range(expected.size):
        if d not in arrived_at_fire:
            raise AssertionError(f"destination {d} never fired")
        if arrived_at_fire[d] != expected[d]:
            raise AssertionError(f"destination {d} fired at {arrived_at_fire[d]} of {expected[d]} arrivals")
