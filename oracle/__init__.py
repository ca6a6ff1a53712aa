"""CPU oracle for the sharded-dataflow hot path -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously correct restatement of what the
hot path computes, written from the PATHWAYS page ("PATHWAYS: Asynchronous
Distributed Dataflow for ML"), section 4.3 "Coordination implementation"
(sharded dataflow graph, destination-tagged tuples, sparse exchange with
progress tracking), sections 4.4-4.5 (buffer futures, parallel asynchronous
dispatch), section 5.1 (chained computations), section 5.3 / Table 2 (GPipe
pipeline) and section 6.3 (data-dependent routing, mixture of experts).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it. The HIP library never does; it shares no code,
headers, tables or helpers with this package. The one module both sides use
is ``pw_inputs`` (seeded random draws only).

Arithmetic is fp64 unless the workload fixes a storage precision, in which
case results are rounded once to that precision where the method stores a
buffer (fp32 node outputs, bf16 activations).

Modules:
  numerics  -- fp32 / bf16 rounding, exact GELU
  exchange  -- histogram, exclusive scan, stable counting-sort exchange,
               elementwise A/B, the sequential step executor over futures
  chain     -- the chained Arg->A->B->Result executor over a future table
  moe       -- router, top-2 gate, dispatch, expert FFN, gated combine
  pipeline  -- stage function and the GPipe fill/drain schedule
  invariants-- checkers for exchange outputs and future tables

Parity status per function is stated in its docstring: every function here
is pinned by a ``-m "not gpu"`` test in ``tests/test_oracle_*.py`` except
where a docstring says "parity unpinned".
"""
