"""CPU simulation of the persistent pipeline kernel's claim and publish
protocol (csrc/pipeline.hip) under random delays.

PATHWAYS page, section 5.3 and Table 2 (S stages over M microbatches, a
GPipe-like schedule) and sections 4.4-4.5 (a computation starts once the
futures of its inputs are ready): tile (s, m, r, c) of the pass may start only
once every column tile of row block (s - 1, m, r) was published, and the pass
must always finish. The kernel runs one persistent workgroup per CU; thread 0
of each claims tiles from the queue of its own XCD only (one claim in
flight), publishes each finished tile from inside the next tile's K loop,
and waits, bounded, when the next tile's input is not complete. Every stage
of a microbatch is in one queue, so producer and consumer of each
activation block share an XCD and its L2. This models thread 0 of every
workgroup as a coroutine over shared counters (each step between two yields
is atomic, as one atomic instruction is), with random tile, epilogue and
poll times, and checks:

  * no wait ever reaches the spin limit (the kernel would latch a timeout
    and publish a tile it never ran);
  * every tile starts exactly once, after its input row block was complete,
    and is published exactly once;
  * the order table is a bijection over the tiles, keeps every tile after
    its inputs and puts every tile in the queue of its inputs (the deal of
    the plan, re-derived here from its description).

The kernel's rules: a claim is always in flight a tile ahead; before waiting
for an input, the workgroup turns that claim into a held ticket and then
waits for whichever of its (at most three) held tickets becomes ready first.
"""
import heapq
import random

import pytest


def deal(S, M, RB, CT, nq, windows):
    """The plan's claim order: items in GPipe lock-step order (tick s + m,
    then stage) or, with stage windows, stage by stage within windows of 16
    microbatches, item (s, m) in queue m mod nq, each item's tiles together."""
    queues = [[] for _ in range(nq)]
    items = []
    if windows:
        for w0 in range(0, M, 16):
            for s in range(S):
                for m in range(w0, min(M, w0 + 16)):
                    items.append((s, m))
    else:
        for t in range(S + M - 1):
            for s in range(S):
                if 0 <= t - s < M:
                    items.append((s, t - s))
    for s, m in items:
        queues[m % nq].extend((s, m, r, c) for r in range(RB) for c in range(CT))
    order, head, length = [], [], []
    for q in queues:
        head.append(len(order))
        length.append(len(q))
        order.extend(q)
    return order, head, length, items


class Sim:
    def __init__(self, S, M, RB, CT, nwg, windows, seed, spin_limit=400.0, tile=(0.8, 1.2), start=(0.0, 0.3)):
        self.S, self.M, self.RB, self.CT = S, M, RB, CT
        self.nq = min(8, nwg)
        self.order, self.qstart, self.qlen, self.items = deal(S, M, RB, CT, self.nq, windows)
        self.qctr = [0] * self.nq
        self.rb = {}           # (s, m, r) -> published column tiles
        self.started = {}      # tile -> start time
        self.published = {}    # tile -> publish count
        self.expired = 0
        self.rng = random.Random(seed)
        self.nwg = nwg
        self.spin_limit = spin_limit
        self.now = 0.0
        self.tile_time, self.start_time = tile, start

    # --- shared state operations (each atomic) ---
    def ready(self, tile):
        s, m, r, _ = tile
        return s == 0 or self.rb.get((s - 1, m, r), 0) == self.CT

    def publish(self, tile):
        s, m, r, _ = tile
        self.rb[(s, m, r)] = self.rb.get((s, m, r), 0) + 1
        self.published[tile] = self.published.get(tile, 0) + 1

    def claim(self, q):
        k = self.qctr[q]
        self.qctr[q] += 1
        return k

    # --- one workgroup's thread 0 ---
    def workgroup(self, b):
        sim, rng = self, self.rng
        nq = self.nq
        # raw: the counter value of the claim in flight on queue q; held: a
        # claimed ticket not handed out yet
        st = {"q": b % nq, "raw": None, "held": None, "live": False, "done": False, "next": None}

        def issue():
            st["raw"] = sim.claim(st["q"])
            st["live"] = True

        def take():
            if st["held"] is not None:
                t, st["held"] = st["held"], None
                if not st["live"] and not st["done"]:
                    issue()
                return t
            if st["done"]:
                return None
            if not st["live"]:
                issue()
            t = sim.qstart[st["q"]] + st["raw"] if st["raw"] < sim.qlen[st["q"]] else None
            if t is None:
                st["done"], st["live"] = True, False
            else:
                issue()
            return t

        def resolve():
            if st["live"] and st["held"] is None and st["raw"] < sim.qlen[st["q"]]:
                st["held"] = sim.qstart[st["q"]] + st["raw"]
                st["live"] = False

        def start(t):
            tile = sim.order[t]
            assert sim.ready(tile), ("started before its input", tile)
            assert tile not in sim.started, ("started twice", tile)
            sim.started[tile] = sim.now

        def start_blocking(t):
            while t is not None:
                resolve()
                n, h = st["next"], st["held"]
                cands = [t, n, h]
                t0 = sim.now
                which = -1
                while sim.now - t0 <= sim.spin_limit:
                    for i, c in enumerate(cands):
                        if c is not None and sim.ready(sim.order[c]):
                            which = i
                            break
                    if which >= 0:
                        break
                    yield rng.uniform(0.005, 0.02)
                if which == 0:
                    start(t)
                    return t
                if which == 1:
                    st["next"] = t
                    start(n)
                    return n
                if which == 2:
                    st["held"], st["next"] = n, t
                    start(h)
                    return h
                sim.expired += 1
                sim.publish(sim.order[t])
                t = n
                st["next"] = take() if n is not None else None
            return None

        yield rng.uniform(*sim.start_time)  # workgroups start at different times
        issue()
        first = take()
        st["next"] = take() if first is not None else None
        cur = yield from start_blocking(first)
        nxt = st["next"]
        prev = None
        while cur is not None:
            k = rng.uniform(*sim.tile_time)  # the K loop; the previous tile is published at its hook
            yield 0.2 * k
            if prev is not None:
                sim.publish(sim.order[prev])
                prev = None
            yield 0.8 * k
            t2 = nxt
            ready = t2 is not None and sim.ready(sim.order[t2])
            if t2 is not None:
                st["next"] = take()
            if ready:
                start(t2)
                nxt = st["next"]
            yield rng.uniform(0.2, 0.4)  # epilogue
            prev = cur
            if ready:
                cur = t2
            else:
                sim.publish(sim.order[prev])
                prev = None
                cur = yield from start_blocking(t2)
                nxt = st["next"]
        if prev is not None:
            sim.publish(sim.order[prev])

    def run(self):
        heap = []
        gens = {}
        for b in range(self.nwg):
            gens[b] = self.workgroup(b)
            heapq.heappush(heap, (0.0, b))
        while heap:
            self.now, b = heapq.heappop(heap)
            try:
                d = next(gens[b])
            except StopIteration:
                continue
            heapq.heappush(heap, (self.now + d, b))
        return self


def check_complete(sim):
    tiles = set(sim.order)
    assert len(tiles) == len(sim.order) == sim.S * sim.M * sim.RB * sim.CT
    assert sim.expired == 0
    assert set(sim.started) == tiles
    assert all(sim.published.get(t) == 1 for t in tiles)


@pytest.mark.parametrize("windows", [False, True])
def test_order_table_keeps_inputs_first(windows):
    order, head, length, items = deal(16, 64, 8, 4, 8, windows)
    assert sorted(order) == sorted({(s, m, r, c) for s in range(16) for m in range(64) for r in range(8)
                                    for c in range(4)})
    pos = {it: i for i, it in enumerate(items)}
    for (s, m) in items:
        if s:
            assert pos[(s - 1, m)] < pos[(s, m)]
        if m:
            assert pos[(s, m - 1)] < pos[(s, m)]  # each stage takes its microbatches in order
    # every tile sits in the queue (the XCD) of the row blocks it reads, after them
    where = {}
    for q in range(8):
        for k, tile in enumerate(order[head[q]:head[q] + length[q]]):
            where[tile] = (q, k)
    for (s, m, r, c), (q, k) in where.items():
        for c2 in range(4):
            if s:
                assert where[(s - 1, m, r, c2)][0] == q and where[(s - 1, m, r, c2)][1] < k
    assert len(set(length)) == 1  # 64 microbatches over 8 XCDs: equal work per XCD


@pytest.mark.parametrize("S,M,RB,CT,nwg", [(3, 5, 2, 2, 4), (4, 9, 1, 4, 16), (5, 20, 3, 1, 12), (8, 16, 2, 2, 32)])
@pytest.mark.parametrize("windows", [False, True])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_claim_protocol_always_finishes(S, M, RB, CT, nwg, windows, seed):
    sim = Sim(S, M, RB, CT, nwg, windows, seed, tile=(0.3, 3.0), start=(0.0, 8.0)).run()
    check_complete(sim)


@pytest.mark.parametrize("windows", [False, True])
def test_claim_protocol_full_pass(windows):
    """The 16-stage, 64-microbatch pass of 2048 x 1024 microbatches on 256 workgroups."""
    check_complete(Sim(16, 64, 8, 4, 256, windows, 7, tile=(0.3, 3.0), start=(0.0, 8.0)).run())
