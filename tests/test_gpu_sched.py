"""GPU tests of the multi-tenant scheduler (PATHWAYS page, section 5.2 and
Figure 9: programs of several clients gang-scheduled in proportional shares;
Appendix D, Figure 11).

Parity: with every program queued before dispatch starts (hold), the order
the library dispatched (its records) equals the stride-scheduling oracle's
order exactly, and every client's chain state equals the chain oracle after
that client's programs, bit for bit. Concurrency: client threads in a closed
loop (submit, wait) get every program run once, in their own order."""
import threading

import numpy as np
import pytest
import torch

import pw_inputs
from oracle import chain as oc
from oracle import sched as osched

pytestmark = pytest.mark.gpu


def _client_ops(pw, c):
    # a different A per client, so that a program run on the wrong plan or
    # state shows in the results: A = x + (1 + c/8), B = x / 2
    return pw.op(pw.PW_OP_AFFINE, 1.0, 1.0 + c / 8.0), pw.op(pw.PW_OP_AFFINE, 0.5, 0.0)


@pytest.mark.parametrize("weights,max_inflight", [((1, 2, 4, 8), 2), ((1, 1, 1, 1), 1), ((3, 1, 2), 4)])
def test_backlogged_dispatch_order_matches_oracle(gpu, weights, max_inflight):
    pw = gpu
    print(f"sched order weights={weights} inflight={max_inflight}", flush=True)
    rng = np.random.default_rng(7)
    n_prog = 10
    steps = [[int(s) for s in rng.integers(1, 4, size=n_prog)] for _ in weights]
    sch = pw.Sched(max_inflight)
    chains, states, x0s = [], [], []
    for c, w in enumerate(weights):
        assert sch.add_client(w) == c
        a, b = _client_ops(pw, c)
        chains.append(pw.Chain(32 * (c + 1), 64, a_op=a, b_op=b))
        x0 = pw_inputs.chain_state(32 * (c + 1), 64, variant=c)
        x0s.append(x0)
        states.append(torch.from_numpy(x0).cuda())
    sch.hold(True)
    who = {}
    # submission order: round robin over clients (the order of queued
    # programs inside a client is what matters)
    for i in range(n_prog):
        for c in range(len(weights)):
            t = sch.submit_chain(c, chains[c], states[c], steps[c][i])
            who[t] = (c, i)
    sch.hold(False)
    for t in sorted(who):
        sch.wait(t, 30_000_000_000)
    recs = sch.records()
    assert len(recs) == len(who)
    assert [r[3] for r in recs] == list(range(len(who)))       # dispatch indices in order
    assert all(r[2] == pw.PW_OK for r in recs)
    got = [who[r[0]] for r in recs]
    assert all(r[1] == who[r[0]][0] for r in recs)
    want = osched.backlogged_order(list(weights), steps)   # cost = steps
    assert got == want
    # device times: programs run one after another on one stream
    starts = np.array([r[4] for r in recs])
    ends = np.array([r[5] for r in recs])
    assert np.all(ends >= starts) and np.all(starts[1:] >= ends[:-1] - 1e-3)
    for c in range(len(weights)):
        a, b = _client_ops(pw, c)
        ref = oc.chain(x0s[c], sum(steps[c]), a_op=_oracle_op(a), b_op=_oracle_op(b))
        assert np.array_equal(states[c].cpu().numpy().view(np.uint32), ref.state.view(np.uint32)), c
    sch.destroy()


def _oracle_op(o):
    from oracle import exchange as ox
    return ox.op_affine(o.a, o.b)


def test_closed_loop_client_threads(gpu):
    pw = gpu
    n_clients, per_client = 8, 12
    print(f"sched closed loop {n_clients} threads x {per_client}", flush=True)
    sch = pw.Sched(2)
    chains, states, x0s, steps = [], [], [], []
    for c in range(n_clients):
        sch.add_client(1 + c % 4)
        a, b = _client_ops(pw, c)
        chains.append(pw.Chain(64, 128, a_op=a, b_op=b))
        x0 = pw_inputs.chain_state(64, 128, variant=10 + c)
        x0s.append(x0)
        states.append(torch.from_numpy(x0).cuda())
        steps.append([1 + (c + i) % 2 for i in range(per_client)])
    errors = []

    def client(c):
        try:
            for i in range(per_client):
                t = sch.submit_chain(c, chains[c], states[c], steps[c][i])
                sch.wait(t, 30_000_000_000)
        except Exception as e:  # reported below
            errors.append((c, repr(e)))

    ths = [threading.Thread(target=client, args=(c,)) for c in range(n_clients)]
    for th in ths:
        th.start()
    for th in ths:
        th.join(60)
    assert not errors, errors
    assert not any(th.is_alive() for th in ths)
    recs = sch.records()
    assert len(recs) == n_clients * per_client
    assert sorted(r[3] for r in recs) == list(range(len(recs)))
    for c in range(n_clients):
        a, b = _client_ops(pw, c)
        ref = oc.chain(x0s[c], sum(steps[c]), a_op=_oracle_op(a), b_op=_oracle_op(b))
        assert np.array_equal(states[c].cpu().numpy().view(np.uint32), ref.state.view(np.uint32)), c
    sch.destroy()


def test_exchange_programs_and_errors(gpu):
    pw = gpu
    from oracle import exchange as ox
    print("sched exchange programs", flush=True)
    n, t, p = 8, 512, 16
    inp = pw_inputs.exchange_uniform(n, t, p)
    ex = pw.Exchange(n, t, p, a_op=pw.op(pw.PW_OP_AFFINE, 2.0, 1.0), b_op=pw.op(pw.PW_OP_ROWSUM))
    sch = pw.Sched(2)
    c = sch.add_client(1)
    x = torch.from_numpy(inp.x).cuda()
    dest = torch.from_numpy(inp.dest).cuda()
    tk = sch.submit_exchange(c, ex, x, dest)
    sch.wait(tk, 30_000_000_000)
    ref = ox.exchange_step(inp.x, inp.dest, n, n, a_op=ox.op_affine(2.0, 1.0), b_op=ox.op_rowsum())
    assert np.array_equal(ex.dst.cpu().numpy().view(np.uint32), ref.y.view(np.uint32))
    # a ticket is waited once
    with pytest.raises(pw.PwError) as e:
        sch.wait(tk, 0)
    assert e.value.code == pw.PW_ERR_STATE
    # a launch that fails reports its own error at wait: a destination out of range
    bad = dest.clone()
    bad[5] = n + 3
    tk = sch.submit_exchange(c, ex, x, bad)
    with pytest.raises(pw.PwError) as e:
        sch.wait(tk, 30_000_000_000)
    assert e.value.code == pw.PW_ERR_BAD_DEST
    # and the plan is usable again afterwards
    tk = sch.submit_exchange(c, ex, x, dest)
    sch.wait(tk, 30_000_000_000)
    # argument checks at submission
    prog = pw.pw_program()
    prog.kind, prog.cost, prog.plan = pw.PW_PROG_EXCHANGE, 0, ex.plan.handle.value
    import ctypes as C
    tt = C.c_uint64(0)
    assert pw.lib.pw_sched_submit(sch.handle, c, C.byref(prog), C.byref(tt)) == pw.PW_ERR_INVALID
    prog.cost = 1
    assert pw.lib.pw_sched_submit(sch.handle, 99, C.byref(prog), C.byref(tt)) == pw.PW_ERR_INVALID
    prog.plan = 0xdead0
    assert pw.lib.pw_sched_submit(sch.handle, c, C.byref(prog), C.byref(tt)) == pw.PW_ERR_STATE
    # a held scheduler times out a wait, then runs the program once released
    sch.hold(True)
    tk = sch.submit_exchange(c, ex, x, dest)
    with pytest.raises(pw.PwError) as e:
        sch.wait(tk, 2_000_000)
    assert e.value.code == pw.PW_ERR_TIMEOUT
    sch.hold(False)
    sch.wait(tk, 30_000_000_000)
    sch.destroy()
