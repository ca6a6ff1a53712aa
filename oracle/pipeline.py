"""Oracle of the GPipe forward pipeline over S stages and M microbatches (test infrastructure only).

Sources: the PATHWAYS page ("PATHWAYS: Asynchronous Distributed Dataflow for
ML"), section 5.3 "Large-scale model performance" and Table 2: a model split
into S balanced stages on distinct device sets, run with a GPipe-like
schedule over M microbatches (S = 16, M = 64 among the measured settings);
the NEST page ("Nest: Network- and Memory-Aware Device Placement for
Distributed Deep Learning"), Algorithm 1: a pipeline of s stages and mbs
microbatches takes t_stage * (mbs + s - 1) plus synchronisation, i.e.
M + S - 1 stage slots from the first microbatch entering to the last leaving.

Readings: each stage is f_s(h) = bf16(GELU(fp32(h . W_s))) with W_s stored
[in][out] and distinct per stage; forward only; stage s runs its
microbatches in ascending order and microbatch m enters stage s once stage
s - 1 finished it. The values do not depend on the schedule.
"""
from __future__ import annotations

import numpy as np

from .numerics import gelu, to_bf16, to_f32


def stage(h: np.ndarray, w: np.ndarray) -> np.ndarray:
    """bf16(GELU(fp32(h . W))) with the dot products in fp64."""
    a = to_f32(h.astype(np.float64) @ w.astype(np.float64))
    return to_bf16(to_f32(gelu(a)))


def forward(x: np.ndarray, w: np.ndarray, keep_all: bool = False):
    """Run every stage on rows x [..., d]; returns the last output or, with
    ``keep_all``, the list of all S stage outputs."""
    outs = []
    h = x
    for s in range(w.shape[0]):
        h = stage(h, w[s])
        if keep_all:
            outs.append(h)
    return outs if keep_all else h


def gpipe_schedule(stages: int, microbatches: int):
    """Lock-step GPipe fill/drain: at every tick each stage runs the next
    microbatch whose input is ready (finished by stage s - 1 in an earlier
    tick). Returns the list of ticks, each a list of (stage, microbatch)."""
    done_tick = {}
    next_mb = [0] * stages
    ticks = []
    t = 0
    while any(n < microbatches for n in next_mb):
        items = []
        for s in range(stages):
            m = next_mb[s]
            if m >= microbatches:
                continue
            if s == 0 or done_tick.get((s - 1, m), t) < t:
                items.append((s, m))
        for s, m in items:
            done_tick[(s, m)] = t
            next_mb[s] += 1
        if not items:
            raise AssertionError("schedule made no progress")
        ticks.append(items)
        t += 1
    return ticks
