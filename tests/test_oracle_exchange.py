"""Pins of the exchange oracle against brute force, a library stable sort,
invariants and exact arithmetic (CPU only).

PATHWAYS page, section 4.3: tuples tagged with destination shards are
exchanged along the sharded edge; progress tracking decides when a shard has
all of its messages. The reading pinned here: the output is the stable sort
of the tuples by destination in global source order.
"""
import itertools
import math

import numpy as np
import pytest

import pw_inputs
from oracle import exchange as ex
from oracle import invariants as inv


def brute_force(dest, num_dest):
    """Literal definition: for every destination in turn, walk the tuples in
    source order and append those tagged with it."""
    order, counts = [], []
    for d in range(num_dest):
        c = 0
        for g in range(len(dest)):
            if dest[g] == d:
                order.append(g)
                c += 1
        counts.append(c)
    return order, counts


def _oracle_light(dest, num_dest, num_src):
    t = len(dest) // num_src
    counts = ex.histogram(dest, num_dest, num_src, t)
    offsets = ex.exclusive_scan(counts.sum(axis=0))
    return counts, offsets, ex.stable_place(dest, offsets)


@pytest.mark.parametrize("num_dest,tuples", [(2, t) for t in range(1, 7)] + [(3, t) for t in range(1, 5)])
def test_exhaustive_against_brute_force(num_dest, tuples):
    """Every destination vector of N shards x T tuples (N=2: T<=6, N=3: T<=4)."""
    num_src = num_dest
    g = num_src * tuples
    for combo in itertools.product(range(num_dest), repeat=g):
        dest = np.array(combo, dtype=np.int32)
        counts, offsets, src_index = _oracle_light(dest, num_dest, num_src)
        order, bcounts = brute_force(combo, num_dest)
        assert src_index.tolist() == order, combo
        assert np.diff(offsets).tolist() == bcounts, combo
        for s in range(num_src):
            seg = combo[s * tuples:(s + 1) * tuples]
            assert counts[s].tolist() == [seg.count(d) for d in range(num_dest)], combo


def test_full_step_small_exhaustive_with_payload():
    """exchange_step (futures, A, B) on every N=2, T=3 input, rows checked
    against the brute-force order."""
    rng = np.random.default_rng(7)
    for combo in itertools.product(range(2), repeat=6):
        dest = np.array(combo, dtype=np.int32)
        x = rng.uniform(-1, 1, size=(6, 3)).astype(np.float32)
        r = ex.exchange_step(x, dest, 2, 2, a_op=ex.op_affine(2.0, 1.0), b_op=ex.op_rowsum())
        order, _ = brute_force(combo, 2)
        ax = (np.float32(2) * x + np.float32(1))
        assert np.array_equal(r.y.view(np.uint32), ax[order].view(np.uint32))
        for j, gsrc in enumerate(order):
            assert math.isclose(r.b_out[j], math.fsum(float(v) for v in ax[gsrc]), rel_tol=0, abs_tol=1e-6)


@pytest.mark.parametrize("case", ["uniform_small", "zipf_small", "uniform_c1", "all_to_one", "reversed", "identity"])
def test_against_library_stable_sort(case):
    """np.argsort(kind='stable') of the destinations is the same permutation."""
    if case == "uniform_small":
        inp = pw_inputs.exchange_uniform(5, 37, 4)
        dest, n, ns = inp.dest, 5, 5
    elif case == "zipf_small":
        inp = pw_inputs.exchange_zipf(64, 300, 4)
        dest, n, ns = inp.dest, 64, 64
    elif case == "uniform_c1":
        inp = pw_inputs.exchange_uniform(8, 4096, 64)
        dest, n, ns = inp.dest, 8, 8
    elif case == "all_to_one":
        dest, n, ns = np.full(64 * 33, 17, np.int32), 64, 64
    elif case == "reversed":
        n = ns = 16
        dest = np.repeat(np.arange(n - 1, -1, -1, dtype=np.int32), 21)
    else:
        n = ns = 16
        dest = np.repeat(np.arange(n, dtype=np.int32), 21)
    counts, offsets, src_index = _oracle_light(dest, n, ns)
    assert np.array_equal(src_index, np.argsort(dest, kind="stable"))
    assert np.array_equal(np.diff(offsets), np.bincount(dest, minlength=n))
    inv.check_exchange(dest, n, src_index, offsets, counts)


def test_step_futures_and_payload_c1():
    """The small uniform workload end to end: futures fire once, each only with
    all of its arrivals, A is bit exact, B within the fp32 summation bound."""
    inp = pw_inputs.exchange_uniform(8, 4096, 64)
    r = ex.exchange_step(inp.x, inp.dest, 8, 8, a_op=ex.op_affine(2.0, 1.0), b_op=ex.op_rowsum())
    ax = np.float32(2) * inp.x + np.float32(1)         # two fp32 roundings; 2x is exact
    inv.check_exchange(inp.dest, 8, r.src_index, r.offsets, r.counts, r.y, ax)
    inv.check_futures_at_fire(r.arrived_at_fire, r.expected)
    assert all(v == 1 for v in r.futures.fire_count.values())
    nodes = {(n, s) for n, s in r.futures.order}
    assert nodes == ({("Arg", s) for s in range(8)} | {("A", s) for s in range(8)}
                     | {("exchange", d) for d in range(8)} | {("B", d) for d in range(8)} | {("Result", -1)})
    pos = {k: i for i, k in enumerate(r.futures.order)}
    for d in range(8):
        assert pos[("exchange", d)] < pos[("B", d)] < pos[("Result", -1)]
    # B = per-tuple sum: against an exactly rounded sum (math.fsum), within one fp32 ulp
    ref = np.array([math.fsum(map(float, ax[g])) for g in r.src_index], dtype=np.float64)
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(r.b_out.astype(np.float64) - ref) <= ulp)


def test_empty_and_degenerate():
    # no tuples at all: every destination's future still fires, with an empty segment
    x = np.zeros((0, 4), np.float32)
    r = ex.exchange_step(x, np.zeros(0, np.int32), 5, 1)
    assert r.offsets.tolist() == [0] * 6
    inv.check_futures_at_fire(r.arrived_at_fire, r.expected)
    # one destination gets nothing
    dest = np.array([0, 2, 0, 2], np.int32)
    r = ex.exchange_step(np.ones((4, 1), np.float32), dest, 3, 2)
    assert r.expected.tolist() == [2, 0, 2] and r.arrived_at_fire[1] == 0
    with pytest.raises(ValueError):
        ex.exchange_step(np.ones((2, 1), np.float32), np.array([0, 3], np.int32), 3, 1)
    with pytest.raises(ValueError):
        ex.exchange_step(np.ones((2, 1), np.float32), np.array([0, -1], np.int32), 3, 1)


def test_affine_is_exact_fp32():
    """A = 2x + 1 and the chain's x + 1, x / 2: the fp64-then-round oracle equals
    plain fp32 arithmetic bit for bit (2x and x/2 are exact in fp32)."""
    x = pw_inputs.exchange_uniform(8, 4096, 64).x
    assert np.array_equal(ex.apply_op(ex.op_affine(2, 1), x).view(np.uint32),
                          (np.float32(2) * x + np.float32(1)).view(np.uint32))
    assert np.array_equal(ex.apply_op(ex.op_affine(1, 1), x).view(np.uint32), (x + np.float32(1)).view(np.uint32))
    assert np.array_equal(ex.apply_op(ex.op_affine(0.5, 0), x).view(np.uint32), (x * np.float32(0.5)).view(np.uint32))


# --------------------------------------------------------------------------
# The checkers themselves must catch planted mistakes
# --------------------------------------------------------------------------

def _good():
    inp = pw_inputs.exchange_uniform(4, 50, 2)
    counts, offsets, src_index = _oracle_light(inp.dest, 4, 4)
    return inp, counts, offsets, src_index


def test_invariants_catch_swapped_pair():
    inp, counts, offsets, si = _good()
    bad = si.copy()
    lo = offsets[1]
    bad[lo], bad[lo + 1] = bad[lo + 1], bad[lo]
    with pytest.raises(AssertionError, match="source order"):
        inv.check_exchange(inp.dest, 4, bad, offsets, counts)


def test_invariants_catch_dropped_tuple():
    inp, counts, offsets, si = _good()
    bad = si.copy()
    bad[3] = bad[4]
    with pytest.raises(AssertionError, match="permutation"):
        inv.check_exchange(inp.dest, 4, bad, offsets, counts)


def test_invariants_catch_wrong_segment_and_payload():
    inp, counts, offsets, si = _good()
    bad_off = offsets.copy()
    bad_off[2] += 1
    with pytest.raises(AssertionError):
        inv.check_exchange(inp.dest, 4, si, bad_off, counts)
    y = inp.x[si].copy()
    y[5, 1] = np.nextafter(y[5, 1], np.float32(9))
    with pytest.raises(AssertionError, match="payload"):
        inv.check_exchange(inp.dest, 4, si, offsets, counts, y, inp.x)


def test_future_table_catches_double_fire_and_early_read():
    ft = ex.FutureTable(epoch=3)
    ft.fire("A", 0)
    with pytest.raises(AssertionError, match="twice"):
        ft.fire("A", 0)
    with pytest.raises(AssertionError, match="before its future"):
        ft.require("B", 0)
    with pytest.raises(AssertionError):
        inv.check_fires(np.array([[1, 1], [1, 2]]))
    with pytest.raises(AssertionError):
        inv.check_futures_at_fire({0: 3, 1: 1}, [3, 2])


def test_planted_oracle_mistake_is_caught(monkeypatch):
    """Plant an off-by-one in the oracle's scan; the brute-force pin fails."""
    def bad_scan(totals):
        o = np.zeros(len(totals) + 1, np.int64)
        o[1:] = np.cumsum(totals)
        o[1:-1] += 1          # planted mistake
        return o
    monkeypatch.setattr(ex, "exclusive_scan", bad_scan)
    dest = np.array([1, 0, 1, 0], np.int32)
    with pytest.raises(AssertionError):
        counts, offsets, si = _oracle_light(dest, 2, 2)
        assert si.tolist() == brute_force(dest.tolist(), 2)[0]


def test_zipf_generator_structure():
    """Each source uses at most k distinct destinations, all from its own draw."""
    inp = pw_inputs.exchange_zipf(64, 500, 4)
    d = inp.dest.reshape(64, 500)
    for s in range(64):
        used = set(np.unique(d[s]).tolist())
        assert used <= set(inp.choices[s].tolist()) and len(inp.choices[s]) == 4
        assert len(set(inp.choices[s].tolist())) == 4
