"""Seeded synthetic inputs for the five sharded-dataflow workloads.

This module is shared by the CPU oracle and the HIP path, so it holds only
random draws and their shapes, never any of the method's arithmetic
(no exchange, no routing, no GEMM, no rounding rule of the method: the one
dtype cast below is torch's own fp32 -> bf16 conversion of freshly drawn
values).

Every array of workload ``k`` comes from
``numpy.random.default_rng(child)`` where ``child`` is spawned from
``SeedSequence(1000 + k)``; size variants (smaller parity cases, the chain's
N sweep) add their sizes to the spawn key, so a case is reproducible from
its name and sizes alone.

Workloads (value distributions and shapes as the dataflow page's
evaluation describes them; sizes are the ones this library is measured on):

* exchange_uniform  - N shards x T tuples, payload P fp32 ~ U(-1, 1),
                      destination uniform in [0, N)        (small exchange)
* exchange_zipf     - N shards x T tuples, payload P fp32 ~ N(0, 1); each
                      source shard picks k distinct destinations with Zipf(s)
                      weights over shard ids, each tuple picks one of the k
                      uniformly                              (large exchange)
* chain             - N shards x E fp32 ~ U(-1, 1)          (chained steps)
* moe               - tokens x d bf16 ~ N(0, 1), router d x E, expert FFN
                      weights, all ~ N(0, 0.02) (standard deviation)
* pipeline          - M microbatches of R x d bf16 ~ N(0, 1), S stage
                      weights d x d ~ N(0, 0.02)
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "rng_for", "sha256", "ExchangeInputs", "exchange_uniform", "exchange_zipf",
    "zipf_weights", "chain_state", "MoEInputs", "moe", "PipelineInputs", "pipeline",
]


def rng_for(workload: int, *key: int) -> np.random.Generator:
    """Generator for one array of workload ``workload`` (1..5).

    ``key`` distinguishes arrays (and size variants) of the same workload.
    """
    ss = np.random.SeedSequence(1000 + int(workload), spawn_key=tuple(int(k) for k in key))
    return np.random.default_rng(ss)


_CHUNK_ROWS = 1 << 20


def _fill_chunked(shape, workload: int, key: tuple, draw) -> np.ndarray:
    """Fill a [rows, cols] float32 array chunk by chunk (1 Mi rows each), every
    chunk from its own generator spawned with the chunk index in its key, in
    parallel threads. The values depend only on (workload, key, shape)."""
    from concurrent.futures import ThreadPoolExecutor
    rows, cols = shape
    out = np.empty((rows, cols), dtype=np.float32)
    starts = list(range(0, rows, _CHUNK_ROWS))

    def work(i_start):
        i, start = i_start
        stop = min(rows, start + _CHUNK_ROWS)
        draw(rng_for(workload, *key, i), out[start:stop])

    if len(starts) <= 1:
        for i_s in enumerate(starts):
            work(i_s)
    else:
        with ThreadPoolExecutor(max_workers=min(16, len(starts))) as ex:
            list(ex.map(work, enumerate(starts)))
    return out


def sha256(a) -> str:
    """SHA-256 of an array's raw bytes (numpy array or CPU torch tensor)."""
    if hasattr(a, "numpy") and not isinstance(a, np.ndarray):
        a = a.contiguous().view(-1).view(__import__("torch").uint8).numpy()
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8).tobytes()).hexdigest()


@dataclass
class ExchangeInputs:
    x: np.ndarray          # [N*T, P] float32, shard-major (tuple g = s*T + i)
    dest: np.ndarray       # [N*T] int32
    num_shards: int
    tuples_per_shard: int
    choices: np.ndarray | None = None   # [N, k] destinations each source may use (zipf case)
    meta: dict = field(default_factory=dict)


def exchange_uniform(num_shards: int = 8, tuples_per_shard: int = 4096, payload: int = 64,
                     variant: int = 0) -> ExchangeInputs:
    """Payload ~ U(-1, 1) fp32, destination uniform over all shards."""
    key = (num_shards, tuples_per_shard, payload, variant)
    g = num_shards * tuples_per_shard
    x = rng_for(1, 0, *key).uniform(-1.0, 1.0, size=(g, payload)).astype(np.float32)
    dest = rng_for(1, 1, *key).integers(0, num_shards, size=g, dtype=np.int64).astype(np.int32)
    return ExchangeInputs(x, dest, num_shards, tuples_per_shard,
                          meta={"workload": "exchange_uniform", "key": key})


def zipf_weights(num_shards: int, s: float) -> np.ndarray:
    """Sampling weights proportional to (d + 1) ** -s over shard ids d."""
    w = (np.arange(1, num_shards + 1, dtype=np.float64)) ** (-float(s))
    return w / w.sum()


def exchange_zipf(num_shards: int = 256, tuples_per_shard: int = 65536, payload: int = 64,
                  k: int = 4, s: float = 1.1, variant: int = 0,
                  with_payload: bool = True) -> ExchangeInputs:
    """Payload ~ N(0, 1) fp32. Each source shard draws ``k`` distinct
    destination shards without replacement with Zipf(s) weights (its own id
    may be among them); each of its tuples picks one of those uniformly."""
    key = (num_shards, tuples_per_shard, payload, k, int(round(s * 1000)), variant)
    g = num_shards * tuples_per_shard
    kk = min(k, num_shards)
    w = zipf_weights(num_shards, s)
    rc = rng_for(2, 1, *key)
    choices = np.stack([rc.choice(num_shards, size=kk, replace=False, p=w)
                        for _ in range(num_shards)]).astype(np.int32)
    pick = rng_for(2, 2, *key).integers(0, kk, size=(num_shards, tuples_per_shard), dtype=np.int64)
    dest = np.take_along_axis(choices, pick, axis=1).reshape(g).astype(np.int32)
    if with_payload:
        x = _fill_chunked((g, payload), 2, (0, *key),
                          lambda r, o: r.standard_normal(size=o.shape, dtype=np.float32, out=o))
    else:
        x = np.zeros((0, payload), dtype=np.float32)
    return ExchangeInputs(x, dest, num_shards, tuples_per_shard, choices=choices,
                          meta={"workload": "exchange_zipf", "key": key})


def chain_state(num_shards: int = 2048, elems: int = 128, variant: int = 0) -> np.ndarray:
    """[N, E] float32 ~ U(-1, 1): the chain's initial Arg."""
    return rng_for(3, 0, num_shards, elems, variant).uniform(-1.0, 1.0, size=(num_shards, elems)).astype(np.float32)


def _bf16(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


@dataclass
class MoEInputs:
    x: "object"        # torch.bfloat16 [tokens, d]
    w_router: "object" # torch.bfloat16 [d, E]
    w1: "object"       # torch.bfloat16 [E, d, H]
    w2: "object"       # torch.bfloat16 [E, H, d]
    meta: dict = field(default_factory=dict)


def moe(tokens: int = 131072, d: int = 1024, experts: int = 64, hidden: int = 4096,
        variant: int = 0, with_experts: bool = True) -> MoEInputs:
    """Tokens ~ N(0, 1), router and expert weights ~ N(0, 0.02), all bf16
    (drawn in fp32, then torch's round-to-nearest-even cast)."""
    key = (tokens, d, experts, hidden, variant)
    normal = lambda r, o: r.standard_normal(size=o.shape, dtype=np.float32, out=o)
    x = _bf16(_fill_chunked((tokens, d), 4, (0, *key), normal))
    wr = _bf16(rng_for(4, 1, *key).standard_normal(size=(d, experts), dtype=np.float32) * np.float32(0.02))
    if with_experts:
        w1 = _fill_chunked((experts * d, hidden), 4, (2, *key), normal)
        w1 *= np.float32(0.02)
        w1 = _bf16(w1).reshape(experts, d, hidden)
        w2 = _fill_chunked((experts * hidden, d), 4, (3, *key), normal)
        w2 *= np.float32(0.02)
        w2 = _bf16(w2).reshape(experts, hidden, d)
    else:
        w1 = w2 = None
    return MoEInputs(x, wr, w1, w2, meta={"workload": "moe", "key": key})


@dataclass
class PipelineInputs:
    x: "object"   # torch.bfloat16 [M, R, d]
    w: "object"   # torch.bfloat16 [S, d, d]  (stored [in][out])
    meta: dict = field(default_factory=dict)


def pipeline(stages: int = 16, microbatches: int = 64, rows: int = 2048, d: int = 1024,
             variant: int = 0) -> PipelineInputs:
    """Microbatches ~ N(0, 1), per-stage weights ~ N(0, 0.02), all bf16."""
    key = (stages, microbatches, rows, d, variant)
    x = _fill_chunked((microbatches * rows, d), 5, (0, *key),
                      lambda r, o: r.standard_normal(size=o.shape, dtype=np.float32, out=o))
    x = _bf16(x).reshape(microbatches, rows, d)
    w = _bf16(rng_for(5, 1, *key).standard_normal(size=(stages, d, d), dtype=np.float32) * np.float32(0.02))
    return PipelineInputs(x, w, meta={"workload": "pipeline", "key": key})
