"""Oracle of the chained step Arg -> A -> B -> Result repeated K times (test infrastructure only).

Source: the PATHWAYS page ("PATHWAYS: Asynchronous Distributed Dataflow for
ML"): section 5.1 "Single-controller dispatch overheads" (a trivial
computation repeated with each result fed into the next, submitted one call
per computation, as one chained call, or as one fused node), section 4.3
(two N-sharded computations form Arg -> Compute(A) -> Compute(B) -> Result,
with N tuples between adjacent nodes under data parallelism), sections
4.4-4.5 (buffer futures gate each computation).

Readings:
  * Result of step k is the Arg of step k + 1;
  * each shard's tuple is its whole buffer and goes to the same shard
    (identity routing), so the exchange between A and B moves nothing;
  * A and B are separate nodes with separate futures; a node's output is an
    fp32 buffer, so each node rounds once to fp32.

The executor runs the graph sequentially, node after node, over a future
table holding the epoch (= step number) each (node, shard) last fired for;
it asserts every read is of a fired input and every future fires once per
step. It is vectorised over shards (whole-node firing), which is the same
sequence of events as a shard-by-shard loop because shards are independent.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .exchange import apply_op, op_affine


@dataclass
class ChainResult:
    state: np.ndarray        # [N, E] fp32: the Result after the last step
    fut_a: np.ndarray        # [N] epoch A last fired for
    fut_b: np.ndarray        # [N] epoch B last fired for
    fires_a: np.ndarray      # [N] total fires of A
    fires_b: np.ndarray      # [N] total fires of B
    history: list            # states after steps 1..record (fp32 copies)


def chain(x0: np.ndarray, steps: int, a_op=op_affine(1.0, 1.0), b_op=op_affine(0.5, 0.0),
          record: int = 0) -> ChainResult:
    """Run ``steps`` chained Arg -> A -> B -> Result steps over [N, E] fp32 shards."""
    x = np.array(x0, dtype=np.float32, copy=True)
    n = x.shape[0]
    fut_a = np.zeros(n, dtype=np.int64)   # epoch 0 = never fired
    fut_b = np.zeros(n, dtype=np.int64)   # B "epoch 0" stands for the initial Arg
    fires_a = np.zeros(n, dtype=np.int64)
    fires_b = np.zeros(n, dtype=np.int64)
    history = []
    for k in range(1, steps + 1):
        # A of step k reads the Result of step k - 1.
        if not np.all(fut_b == k - 1):
            raise AssertionError("A read an input whose future has not fired")
        if np.any(fut_a >= k):
            raise AssertionError("A future fired twice in one step")
        a = apply_op(a_op, x)
        fut_a[:] = k
        fires_a += 1
        # B of step k reads A of step k.
        if not np.all(fut_a == k):
            raise AssertionError("B read an input whose future has not fired")
        if np.any(fut_b >= k):
            raise AssertionError("B future fired twice in one step")
        x = apply_op(b_op, a)
        fut_b[:] = k
        fires_b += 1
        if k <= record:
            history.append(x.copy())
    return ChainResult(x, fut_a, fut_b, fires_a, fires_b, history)

