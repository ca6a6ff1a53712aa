"""Oracle of the multi-tenant dispatch order (test infrastructure only).

Source: the PATHWAYS page ("PATHWAYS: Asynchronous Distributed Dataflow for
ML"), section 5.2 "Multi-tenancy" with Figures 8 and 9, and Appendix D with
Figure 11: programs of several independent clients are gang-scheduled onto
the same accelerators, interleaved in time, and the scheduler controls how
much accelerator time each client receives, for example in proportional
shares of 1:1:1:1 or 1:2:4:8.

Reading (the pages name no policy): stride scheduling (Waldspurger and
Weihl, "Stride scheduling: deterministic proportional-share resource
management", MIT/LCS/TM-528, 1995), in integer arithmetic:
  * client c has a weight w_c >= 1 and a stride s_c = floor(2^32 / w_c);
  * each program carries a cost (accelerator time in the caller's units);
  * among the clients with queued programs, the one with the smallest pass
    dispatches its oldest program (ties: the lowest client number); the
    virtual time becomes that pass, and the pass grows by cost * s_c;
  * a client whose queue was empty when a program arrives resumes at
    max(its pass, the virtual time): idle time earns no credit.
Pass values are plain Python integers (no overflow); the library rebases
its 64-bit passes by the virtual time when they grow large, which changes
no comparison.
"""
from __future__ import annotations

from collections import deque

STRIDE_ONE = 1 << 32


def stride(weight: int) -> int:
    assert weight >= 1
    return STRIDE_ONE // weight


def simulate(weights, events):
    """Run the dispatcher over a sequence of events and return the dispatch
    order as (client, program index within that client) pairs.

    events: ("submit", client, cost) appends a program to the client's queue;
    ("dispatch", n) dispatches up to n programs (fewer if every queue is
    empty); ("drain",) dispatches until every queue is empty.
    """
    n = len(weights)
    strides = [stride(w) for w in weights]
    passes = [0] * n
    queues = [deque() for _ in range(n)]
    submitted = [0] * n
    vtime = 0
    order = []

    def dispatch_one():
        nonlocal vtime
        ready = [c for c in range(n) if queues[c]]
        if not ready:
            return False
        c = min(ready, key=lambda k: (passes[k], k))
        idx, cost = queues[c].popleft()
        vtime = passes[c]
        passes[c] += cost * strides[c]
        order.append((c, idx))
        return True

    for ev in events:
        if ev[0] == "submit":
            _, c, cost = ev
            assert cost >= 1
            if not queues[c]:
                passes[c] = max(passes[c], vtime)
            queues[c].append((submitted[c], cost))
            submitted[c] += 1
        elif ev[0] == "dispatch":
            for _ in range(ev[1]):
                if not dispatch_one():
                    break
        elif ev[0] == "drain":
            while dispatch_one():
                pass
        else:
            raise ValueError(ev)
    return order


def backlogged_order(weights, costs):
    """Every program submitted before the first dispatch (costs[c] lists the
    costs of client c's programs in submission order), then drained."""
    events = [("submit", c, cost) for c in range(len(weights)) for cost in costs[c]]
    return simulate(weights, events + [("drain",)])
