"""Oracle of the mixture-of-experts step (test infrastructure only).

Source: the PATHWAYS page ("PATHWAYS: Asynchronous Distributed Dataflow for
ML"), section 6.3 "Data-dependent vectorized control flow": examples or
sub-examples are routed, by a learned function, to the accelerators holding
different weight subsets (mixture of experts, Shazeer et al. 2017), which
needs fine-grained data-dependent exchanges; section 4.3: the exchange
itself (see ``oracle.exchange``).

Readings where the pages are silent:
  * router logits = X . W_r with W_r stored [d][E]; the product of two bf16
    values is exact, the sum is taken in fp64 and rounded once to fp32;
  * top-2 keeps the two largest logits, ties to the lower expert id; the
    gates are the softmax over the two kept logits (keep-top-k, then
    softmax), rounded to fp32;
  * each token emits two tuples, in (token, slot) order with slot 0 the
    top-1 expert; tuple g = 2 * token + slot; destination = expert;
  * expert FFN with no biases: H = bf16(GELU(fp32(X_e . W1_e))),
    Y_e = bf16(fp32(H . W2_e)), weights stored [in][out], GELU exact (erf);
  * combine: out[t] = bf16(g_0 * Y[slot of (t,0)] + g_1 * Y[slot of (t,1)]),
    summed in fp64 and rounded to fp32 then bf16; without a capacity limit
    no tuple is dropped.
  * with a capacity C per expert (section 4.5: a node whose resource needs
    depend on its predecessor's results; the usual way to give expert
    buffers a static bound): an expert keeps the first C of its tuples in
    tuple order g and drops the rest; the kept tuples are placed as without
    a limit (segments of min(n_e, C) rows, source order inside); a dropped
    tuple contributes nothing to its token's combine (its gate is not
    renormalised), so a token with both tuples dropped combines to zero.

Arrays are numpy float32 holding bf16-exact values where the workload is
bf16 (callers convert bf16 tensors with ``.float()``).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .exchange import exclusive_scan, histogram, stable_place
from .numerics import gelu, to_bf16, to_f32


def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """fp32 [T, E] = round_fp32(X . W_r) with the dot products in fp64."""
    return to_f32(x.astype(np.float64) @ w_router.astype(np.float64))


def top2(logits: np.ndarray):
    """(experts [T, 2] int64, kept logits [T, 2] fp32): the two largest
    logits of each row, larger first, ties going to the lower expert id."""
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")
    experts = order[:, :2].astype(np.int64)
    kept = np.take_along_axis(logits, experts, axis=1).astype(np.float32)
    return experts, kept


def gates(kept: np.ndarray) -> np.ndarray:
    """Softmax over the two kept logits of each token, fp64 rounded to fp32."""
    k = kept.astype(np.float64)
    m = k.max(axis=1, keepdims=True)
    e = np.exp(k - m)
    return to_f32(e / e.sum(axis=1, keepdims=True))


def expert_ffn(xe: np.ndarray, w1e: np.ndarray, w2e: np.ndarray) -> np.ndarray:
    """Y_e = bf16(fp32(H . W2_e)), H = bf16(GELU(fp32(X_e . W1_e)))."""
    a = to_f32(xe.astype(np.float64) @ w1e.astype(np.float64))
    h = to_bf16(to_f32(gelu(a)))
    return to_bf16(to_f32(h.astype(np.float64) @ w2e.astype(np.float64)))


def combine_rows(g: np.ndarray, y0: np.ndarray, y1: np.ndarray) -> np.ndarray:
    """bf16(fp32(g0 * y0 + g1 * y1)) per token; g [T, 2], y0/y1 [T, d]."""
    s = g[:, 0:1].astype(np.float64) * y0.astype(np.float64) + g[:, 1:2].astype(np.float64) * y1.astype(np.float64)
    return to_bf16(to_f32(s))


@dataclass
class MoEResult:
    logits: np.ndarray     # [T, E] fp32
    experts: np.ndarray    # [T, 2]
    gates: np.ndarray      # [T, 2] fp32
    dest: np.ndarray       # [2T] expert of tuple g = 2t + slot
    counts: np.ndarray     # [num_src, E]
    offsets: np.ndarray    # [E + 1]
    src_index: np.ndarray  # [2T] tuple index held by each dispatched slot
    y: np.ndarray | None   # [2T, d] expert outputs in dispatched order
    out: np.ndarray | None # [T, d] combined output


def capacity_keep(dest: np.ndarray, num_experts: int, capacity: int) -> np.ndarray:
    """keep[g]: tuple g is among the first `capacity` tuples of its expert in
    tuple order (capacity 0: no limit, every tuple kept)."""
    keep = np.ones(dest.size, dtype=bool)
    if capacity <= 0:
        return keep
    seen = np.zeros(num_experts, dtype=np.int64)
    for g in range(dest.size):
        e = dest[g]
        keep[g] = seen[e] < capacity
        seen[e] += 1
    return keep


def route(logits: np.ndarray, num_experts: int, num_src: int, capacity: int = 0):
    """Top-2, gates and the dispatch exchange from fp32 logits. counts are
    the routed tuples per (source, expert) before any capacity limit;
    offsets and src_index describe the kept tuples only."""
    experts, kept = top2(logits)
    g = gates(kept)
    dest = experts.reshape(-1)
    t = logits.shape[0]
    counts = histogram(dest, num_experts, num_src, (2 * t) // num_src)
    keep = capacity_keep(dest, num_experts, capacity)
    idx = np.flatnonzero(keep)
    offsets = exclusive_scan(np.bincount(dest[idx], minlength=num_experts)[:num_experts])
    src_index = idx[stable_place(dest[idx], offsets)]
    return experts, g, dest, counts, offsets, src_index


def moe_step(x, w_router, w1, w2, num_src: int = 1, logits=None, with_ffn: bool = True,
             capacity: int = 0) -> MoEResult:
    """The whole step on every token. ``logits`` may be given to recompute the
    routing from another implementation's fp32 logits. ``capacity``: tuples
    kept per expert (0: no limit)."""
    if logits is None:
        logits = router_logits(x, w_router)
    num_experts = w_router.shape[1]
    experts, g, dest, counts, offsets, src_index = route(logits, num_experts, num_src, capacity)
    y = out = None
    if with_ffn:
        t = x.shape[0]
        rows = x[src_index // 2]                       # payload of each dispatched tuple
        y = np.empty_like(rows)
        for e in range(num_experts):
            lo, hi = offsets[e], offsets[e + 1]
            if hi > lo:
                y[lo:hi] = expert_ffn(rows[lo:hi], w1[e], w2[e])
        pos = np.full(2 * t, -1, dtype=np.int64)       # slot of tuple g, -1 if dropped
        pos[src_index] = np.arange(src_index.size)
        zero = np.zeros((1, x.shape[1]), dtype=np.float32)
        yz = np.concatenate([y, zero])                 # row -1: a dropped tuple's zero contribution
        out = combine_rows(g, yz[pos[0::2]], yz[pos[1::2]])
    return MoEResult(logits, experts, g, dest, counts, offsets, src_index, y, out)


def moe_tokens(x, w_router, w1, w2, token_ids, logits=None):
    """Per-token path for sampled checks: route each token, run its two
    experts on its own row, combine. Returns (experts, gates, out) for the
    listed tokens; independent of other tokens because every step is
    row-wise."""
    token_ids = np.asarray(token_ids, dtype=np.int64)
    xs = x[token_ids]
    lg = router_logits(xs, w_router) if logits is None else np.asarray(logits, np.float32)[token_ids]
    experts, kept = top2(lg)
    g = gates(kept)
    y = np.empty((len(token_ids), 2, x.shape[1]), dtype=np.float32)
    for i in range(len(token_ids)):
        for j in range(2):
            e = experts[i, j]
            y[i, j] = expert_ffn(xs[i:i + 1], w1[e], w2[e])[0]
    return experts, g, combine_rows(g, y[:, 0], y[:, 1])
