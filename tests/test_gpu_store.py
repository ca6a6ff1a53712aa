"""GPU tests of the HBM object store (PATHWAYS page, section 4.6: buffers in
accelerator memory named by handle, ownership labels for garbage collection,
backpressure that stalls an allocation instead of failing it).

Parity: the placements (address - base) and the order in which waiting
requests are granted equal the oracle's (oracle/store.py) exactly. Stream
order: memory freed right after the launches that use it is not handed out
again before they finish, and their results are intact."""
import threading
import time

import numpy as np
import pytest
import torch

import pw_inputs
from oracle import chain as oc
from oracle import store as ostore

pytestmark = pytest.mark.gpu


def wait_until(pred, limit_s=10.0):
    t0 = time.time()
    while not pred():
        assert time.time() - t0 < limit_s, "condition not reached"
        time.sleep(0.001)


def test_placement_and_waiter_order_match_oracle(gpu):
    pw = gpu
    print("store placement", flush=True)
    unit = 1 << 20
    st = pw.Store(8 * unit)
    base = st.stats()["base"]
    ops = [("alloc", "A", unit, 1), ("alloc", "B", 3 * unit, 2), ("alloc", "C", unit + 5, 1),
           ("alloc", "D", 2 * unit, 3), ("free", "B"), ("alloc", "E", unit, 2), ("alloc", "F", 100, 2)]
    objs, offs = {}, {}
    for op in ops:
        if op[0] == "alloc":
            o, p = st.alloc(op[2], op[3], 0)
            objs[op[1]], offs[op[1]] = o, p - base
        else:
            st.free(objs.pop(op[1]))
            torch.cuda.synchronize()
            wait_until(lambda: st.stats()["pending_free"] == 0)  # the stream-ordered free has landed
    ref = ostore.run(8 * unit, ops)
    assert [(n, offs[n]) for n, _ in ref.grants] == ref.grants
    # waiters: two requests that do not fit, granted in arrival order once
    # the owner-1 objects are released
    results = {}

    def waiter(name, nbytes):
        o, p = st.alloc(nbytes, 4, 10_000_000_000)
        results[name] = (o, p - base)

    s0 = st.stats()["waiting"]
    t1 = threading.Thread(target=waiter, args=("G", 2 * unit))
    t1.start()
    wait_until(lambda: st.stats()["waiting"] == s0 + 1)
    t2 = threading.Thread(target=waiter, args=("H", unit))
    t2.start()
    wait_until(lambda: st.stats()["waiting"] == s0 + 2)
    assert st.release_owner(1) == 2          # A and C
    t1.join(10)
    t2.join(10)
    ref2 = ostore.run(8 * unit, ops + [("alloc", "G", 2 * unit, 4), ("alloc", "H", unit, 4), ("release", 1)])
    assert ref2.grants[-2:] == [("G", results["G"][1]), ("H", results["H"][1])]
    s = st.stats()
    assert s["stalls"] >= 2 and s["waiting"] == 0
    assert s["in_use"] == ref2.in_use()
    st.destroy()


def test_stream_ordered_free_and_reuse(gpu):
    """A long chained run writes its state in a store object that is freed
    right after the launch; a request for the whole store waits until the
    run has finished, and the run's result is intact in that memory."""
    pw = gpu
    n, e, steps = 2048, 128, 20000
    print("store stream-ordered free", flush=True)
    nbytes = n * e * 4
    st = pw.Store(nbytes)
    obj, ptr = st.alloc(nbytes)
    state = st.tensor(ptr, (n, e))
    x0 = pw_inputs.chain_state(n, e)
    state.copy_(torch.from_numpy(x0))
    ch = pw.Chain(n, e)
    f = ch.run(state, steps)
    st.free(obj)                                    # stream ordered: after the run
    t0 = time.perf_counter()
    obj2, ptr2 = st.alloc(nbytes, 0, 30_000_000_000)  # the whole store: waits for the run
    waited = time.perf_counter() - t0
    assert pw.future_query(f), "memory handed out before the work using it finished"
    assert ptr2 == ptr
    ref = oc.chain(x0, steps)
    got = st.tensor(ptr2, (n, e)).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.state.view(np.uint32))
    assert st.stats()["stalls"] == 1
    print(f"waited {waited * 1e3:.2f} ms for the run", flush=True)
    st.free(obj2)
    torch.cuda.synchronize()
    st.destroy()


def test_owner_release_timeout_and_errors(gpu):
    pw = gpu
    st = pw.Store(4 << 20)
    a1, _ = st.alloc(1 << 20, owner=7)
    a2, _ = st.alloc(1 << 20, owner=7)
    b1, _ = st.alloc(1 << 20, owner=9)
    # backpressure with a deadline: 2 MiB do not fit, the wait expires
    t0 = time.perf_counter()
    with pytest.raises(pw.PwError) as e:
        st.alloc(2 << 20, owner=9, timeout_ns=5_000_000)
    assert e.value.code == pw.PW_ERR_NOMEM and time.perf_counter() - t0 >= 0.004
    with pytest.raises(pw.PwError) as e:
        st.alloc(5 << 20)                            # larger than the store: at once
    assert e.value.code == pw.PW_ERR_NOMEM
    torch.cuda.synchronize()
    assert st.release_owner(7) == 2                  # the failed client's buffers
    s = st.stats()
    assert s["objects"] == 1 and s["in_use"] == 1 << 20
    with pytest.raises(pw.PwError) as e:
        st.free(a1)                                  # released with its owner
    assert e.value.code == pw.PW_ERR_STATE
    c1, _ = st.alloc(2 << 20, owner=9, timeout_ns=1_000_000_000)
    assert st.stats()["largest_free"] == 1 << 20
    st.free(b1)
    st.free(c1)
    torch.cuda.synchronize()
    s = st.stats()
    assert s["in_use"] == 0 and s["largest_free"] == 4 << 20 and s["pending_free"] == 0
    assert pw.lib.pw_store_free(st.handle, 12345, None) == pw.PW_ERR_STATE
    st.destroy()
