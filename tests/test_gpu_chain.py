"""GPU parity of the chained Arg -> A -> B -> Result executor (PATHWAYS page,
section 5.1, chained and fused submission; sections 4.4-4.5, futures) against
the CPU oracle, in all three modes. A = x + 1 and B = x / 2 are single fp32
roundings, so every step is bit-exact; the Result after 10,000 steps is 1.0
everywhere (the fp32 fixed point)."""
import numpy as np
import pytest
import torch

import pw_inputs
from oracle import chain as oc

pytestmark = pytest.mark.gpu

MODES = ["chained", "opbyop", "fused", "split"]


def _mode(pw, name):
    return {"chained": pw.PW_CHAIN_CHAINED, "opbyop": pw.PW_CHAIN_OPBYOP, "fused": pw.PW_CHAIN_FUSED,
            "split": pw.PW_CHAIN_SPLIT}[name]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("n,e", [(1, 128), (8, 128), (64, 1), (256, 100), (2048, 128), (300, 200)])
def test_chain_steps_bit_exact(gpu, mode, n, e):
    pw = gpu
    print(f"chain {mode} N={n} E={e}", flush=True)
    x0 = pw_inputs.chain_state(n, e)
    ref = oc.chain(x0, 40, record=40)
    ch = pw.Chain(n, e, mode=_mode(pw, mode))
    st = torch.from_numpy(x0).cuda()
    # one step per call for the first 8 steps, then 32 steps in one call
    for k in range(8):
        f = ch.run(st, 1)
        pw.future_wait(f, 10_000_000_000)
        assert np.array_equal(st.cpu().numpy().view(np.uint32), ref.history[k].view(np.uint32)), k
    f = ch.run(st, 32)
    pw.future_wait(f, 10_000_000_000)
    assert f.epoch == 40
    assert np.array_equal(st.cpu().numpy().view(np.uint32), ref.state.view(np.uint32))
    ep, fi, _ = ch.plan.read_futures()
    assert np.all(ep[pw.PW_NODE_A, :n] == 40) and np.all(ep[pw.PW_NODE_B, :n] == 40)
    calls = 9
    want = calls if mode == "fused" else 40
    assert np.all(fi[pw.PW_NODE_A, :n] == want) and np.all(fi[pw.PW_NODE_B, :n] == want)
    assert ep[pw.PW_NODE_RESULT, 0] == 40 and fi[pw.PW_NODE_RESULT, 0] == calls


@pytest.mark.parametrize("mode", MODES)
def test_chain_full_size_10000_steps(gpu, mode):
    """2048 shards x 128 fp32, 10,000 steps: bit-exact with the oracle (all 1.0)."""
    pw = gpu
    x0 = pw_inputs.chain_state(2048, 128)
    ref = oc.chain(x0, 10000)
    ch = pw.Chain(2048, 128, mode=_mode(pw, mode), flags=pw.PW_FLAG_TRACE)
    st = torch.from_numpy(x0).cuda()
    f = ch.run(st, 10000)
    pw.future_wait(f, 60_000_000_000)
    out = st.cpu().numpy()
    assert np.array_equal(out.view(np.uint32), ref.state.view(np.uint32))
    assert np.all(out == np.float32(1.0))
    ep, fi, stamps = ch.plan.read_futures(trace=True)
    assert np.all(ep[pw.PW_NODE_B, :2048] == 10000)
    if mode != "fused":
        assert np.all(fi[pw.PW_NODE_A, :2048] == 10000) and np.all(fi[pw.PW_NODE_B, :2048] == 10000)
        # the last A of each shard fired before its last B, both before Result
        assert np.all(stamps[pw.PW_NODE_A, :2048] <= stamps[pw.PW_NODE_B, :2048])
        assert np.all(stamps[pw.PW_NODE_B, :2048] <= stamps[pw.PW_NODE_RESULT, 0])


def test_chain_aux_receives_last_a(gpu):
    pw = gpu
    x0 = pw_inputs.chain_state(16, 64)
    ref = oc.chain(x0, 3, record=3)
    ch = pw.Chain(16, 64)
    st = torch.from_numpy(x0).cuda()
    aux = torch.empty_like(st)
    pw.future_wait(ch.run(st, 3, aux=aux), 10_000_000_000)
    last_a = (ref.history[1] + np.float32(1))           # A of step 3 reads the Result of step 2
    assert np.array_equal(aux.cpu().numpy().view(np.uint32), last_a.view(np.uint32))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("depth", [1, 3, 20])
def test_chain_split_into_calls_matches_one_program(gpu, mode, depth):
    """20 steps run as calls of `depth` steps each (each call's Result is the
    next call's Arg, the epochs continue) equal the oracle's 20 steps bit for
    bit: the program length per call changes dispatch, not values."""
    pw = gpu
    n, e, k = 64, 128, 20
    x0 = pw_inputs.chain_state(n, e)
    ref = oc.chain(x0, k)
    ch = pw.Chain(n, e, mode=_mode(pw, mode))
    st = torch.from_numpy(x0).cuda()
    done = 0
    while done < k:
        d = min(depth, k - done)
        f = ch.run(st, d)
        done += d
    pw.future_wait(f, 10_000_000_000)
    assert np.array_equal(st.cpu().numpy().view(np.uint32), ref.state.view(np.uint32))
    assert not np.all(ref.state == np.float32(1.0))  # still short of the fp32 fixed point


def test_chain_rejects_bad_state(gpu):
    pw = gpu
    ch = pw.Chain(8, 128)
    st = torch.zeros((8, 64), device="cuda")
    with pytest.raises(pw.PwError) as e:
        ch.run(st, 1)
    assert e.value.code == pw.PW_ERR_INVALID


@pytest.mark.parametrize("n", [1537, 2049, 4099])
def test_chain_packed_shards_bit_exact(gpu, n):
    """Shard counts where a wave serves two shards of 128 elements, with a
    ragged last wave: 40 steps and the fire counts equal the oracle's."""
    pw = gpu
    print(f"chain packed N={n}", flush=True)
    x0 = pw_inputs.chain_state(n, 128)
    ref = oc.chain(x0, 40, record=40)
    ch = pw.Chain(n, 128, mode=pw.PW_CHAIN_CHAINED)
    st = torch.from_numpy(x0).cuda()
    f = ch.run(st, 3)
    pw.future_wait(f, 10_000_000_000)
    assert np.array_equal(st.cpu().numpy().view(np.uint32), ref.history[2].view(np.uint32))
    aux = torch.empty_like(st)
    f = ch.run(st, 37, aux=aux)
    pw.future_wait(f, 10_000_000_000)
    assert f.epoch == 40
    assert np.array_equal(st.cpu().numpy().view(np.uint32), ref.state.view(np.uint32))
    last_a = ref.history[38] + np.float32(1)          # A of step 40 reads the Result of step 39
    assert np.array_equal(aux.cpu().numpy().view(np.uint32), last_a.view(np.uint32))
    ep, fi, _ = ch.plan.read_futures()
    assert np.all(ep[pw.PW_NODE_A, :n] == 40) and np.all(ep[pw.PW_NODE_B, :n] == 40)
    assert np.all(fi[pw.PW_NODE_A, :n] == 40) and np.all(fi[pw.PW_NODE_B, :n] == 40)
    assert ep[pw.PW_NODE_RESULT, 0] == 40 and fi[pw.PW_NODE_RESULT, 0] == 2


def test_chain_rejects_misaligned_state(gpu):
    pw = gpu
    ch = pw.Chain(8, 128)
    flat = torch.zeros(8 * 128 + 1, device="cuda")
    with pytest.raises(pw.PwError) as e:
        ch.run(flat[1:].view(8, 128), 1)
    assert e.value.code == pw.PW_ERR_INVALID


@pytest.mark.parametrize("n", [8, 256, 2048])
def test_chain_split_placement_crosses_xcds(gpu, n):
    """PW_CHAIN_SPLIT: A[i] and B[i] run on different waves of different
    workgroups, A preferably on the first half of the XCDs and B on the
    second, so each gate is a cross-workgroup release/acquire. 200 steps are
    bit-exact with the oracle; the placement table shows where each node ran;
    and the last step's fire stamps, taken when each node fired, put A[i]
    before B[i] before the Result for every shard (B waits on A across
    workgroups, so this order is the gate's, not program order's)."""
    pw = gpu
    x0 = pw_inputs.chain_state(n, 128)
    ref = oc.chain(x0, 200)
    ch = pw.Chain(n, 128, mode=pw.PW_CHAIN_SPLIT, flags=pw.PW_FLAG_TRACE)
    st = torch.from_numpy(x0).cuda()
    pw.future_wait(ch.run(st, 200), 30_000_000_000)
    assert np.array_equal(st.cpu().numpy().view(np.uint32), ref.state.view(np.uint32))
    pl = ch.placement()
    cross = float((pl[:, 0] != pl[:, 1]).mean())
    print(f"split placement N={n}: {cross:.1%} of shards have A and B on different XCDs", flush=True)
    if torch.cuda.get_device_properties(0).multi_processor_count >= 64:
        assert cross > 0.5
    ep, fi, stamps = ch.plan.read_futures(trace=True)
    assert np.all(fi[pw.PW_NODE_A, :n] == 200) and np.all(fi[pw.PW_NODE_B, :n] == 200)
    sa, sb = stamps[pw.PW_NODE_A, :n].astype(np.int64), stamps[pw.PW_NODE_B, :n].astype(np.int64)
    assert np.all(sa < sb) and np.all(sb <= stamps[pw.PW_NODE_RESULT, 0])
