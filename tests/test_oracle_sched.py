"""Pins of the multi-tenant dispatch oracle (PATHWAYS page, section 5.2,
Figure 9: proportional shares such as 1:1:1:1 and 1:2:4:8) to facts that
do not come from its code: closed forms of stride scheduling and orders
derived by hand."""
import os
from collections import Counter

from oracle import sched


def counts(order, upto):
    return Counter(c for c, _ in order[:upto])


def test_equal_shares_are_round_robin():
    # 1:1:1:1 with equal costs: every client in turn, lowest number first
    order = sched.backlogged_order([1, 1, 1, 1], [[1] * 5] * 4)
    assert [c for c, _ in order] == [0, 1, 2, 3] * 5
    # each client's programs leave in submission order
    for c in range(4):
        assert [i for k, i in order if k == c] == list(range(5))


def test_weights_1_2_4_8_exact_per_cycle():
    # strides 2^32, 2^31, 2^30, 2^29: after every 15 dispatches all passes
    # are equal again, so each cycle of 15 holds exactly 1, 2, 4, 8 programs
    order = sched.backlogged_order([1, 2, 4, 8], [[1] * 64] * 4)
    for cycles in (1, 2, 3, 4):
        got = counts(order, 15 * cycles)
        assert [got[c] for c in range(4)] == [cycles * w for w in (1, 2, 4, 8)]
    # the first cycle by hand, passes in units of 2^29 (strides 8, 4, 2, 1):
    # (0,0,0,0) -> 0,1,2,3 by the tie rule -> (8,4,2,1) -> 3 -> (8,4,2,2)
    # -> 2 -> (8,4,4,2) -> 3, 3 -> (8,4,4,4) -> 1 -> (8,8,4,4) -> 2 ->
    # (8,8,6,4) -> 3, 3 -> (8,8,6,6) -> 2 -> (8,8,8,6) -> 3, 3 -> all 8
    assert [c for c, _ in order[:15]] == [0, 1, 2, 3, 3, 2, 3, 3, 1, 2, 3, 3, 2, 3, 3]


def test_cost_scales_the_charge():
    # equal weights, client 1's programs cost 3: over 8 dispatches client 0
    # runs 6 programs and client 1 two (equal accelerator time)
    order = sched.backlogged_order([1, 1], [[1] * 20, [3] * 20])
    got = counts(order, 8)
    assert (got[0], got[1]) == (6, 2)
    # the same share by weight instead of cost: weight 3 vs 1, unit costs
    order = sched.backlogged_order([3, 1], [[1] * 20, [1] * 20])
    got = counts(order, 8)
    assert (got[0], got[1]) == (6, 2)


def test_idle_time_earns_no_credit():
    # client 0 alone for 10 dispatches (its pass reaches 10 * 2^32, the
    # virtual time 9 * 2^32); client 1 then arrives and resumes at 9 * 2^32,
    # so it leads by one program and the two alternate from there -- not ten
    # programs of client 1 in a row
    events = [("submit", 0, 1) for _ in range(20)] + [("dispatch", 10)]
    events += [("submit", 1, 1) for _ in range(10)] + [("dispatch", 8)]
    order = sched.simulate([1, 1], events)
    assert [c for c, _ in order[:10]] == [0] * 10
    assert [c for c, _ in order[10:18]] == [1, 0, 1, 0, 1, 0, 1, 0]


def test_empty_and_single_client():
    assert sched.backlogged_order([1, 5], [[], []]) == []
    assert sched.backlogged_order([7], [[2, 1, 4]]) == [(0, 0), (0, 1), (0, 2)]


def test_the_pages_share_ratios_hold_per_cycle():
    """The weights of Figure 9 (stored in tests/golden): with backlogged
    clients of equal program cost, every cycle of sum(weights) dispatches
    gives client c exactly weights[c] programs."""
    path = os.path.join(os.path.dirname(__file__), "golden", "pathways_fig9_share_ratios.txt")
    rows = [[int(v) for v in line.split("#", 1)[0].split()] for line in open(path)]
    rows = [r for r in rows if r]
    assert rows == [[1, 1, 1, 1], [1, 2, 4, 8]]
    for w in rows:
        order = sched.backlogged_order(w, [[1] * (16 * max(w))] * len(w))
        cyc = sum(w)
        for k in (1, 2, 3):
            got = counts(order, cyc * k)
            assert [got[c] for c in range(len(w))] == [k * x for x in w]
