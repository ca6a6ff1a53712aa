"""GPU parity of the one-launch exchange step (csrc/exchange_small.hip,
PW_FLAG_ONE_LAUNCH) for small steps, against the same step run as separate
launches (the default) and against the CPU oracle.

PATHWAYS page, section 4.3 (progress tracking decides when a shard has all
its messages) and sections 4.4-4.5 (B consumes the exchange's futures and
starts as soon as they are ready): in one launch, B of a segment is gated
on that segment's EXCHANGE future inside the launch. Bars: every output bit
for bit equal to the separate launches' (routing, indices, payload, the fp32
row sums, which use the same summation order); routing and payload equal to
the oracle's; every future fires once per call; with tracing, each B[d]
fires after its EXCHANGE[d] and before the Result.
"""
import numpy as np
import pytest
import torch

import pw_inputs
from oracle import exchange as ox

pytestmark = pytest.mark.gpu


def _dest(kind, n, t, seed=0):
    rng = np.random.default_rng(seed + n * 7 + t)
    g = n * t
    if kind == "uniform":
        return rng.integers(0, n, size=g).astype(np.int32)
    if kind == "identity":
        return np.repeat(np.arange(n, dtype=np.int32), t)
    if kind == "reversed":
        return np.repeat(np.arange(n - 1, -1, -1, dtype=np.int32), t)
    if kind == "zipf4":
        return pw_inputs.exchange_zipf(n, t, 1, with_payload=False).dest
    if kind == "half_empty":
        return (rng.integers(0, max(n // 2, 1), size=g) * 2 % n).astype(np.int32)
    raise ValueError(kind)


def _pair(pw, n, t, p, a_op, b_op, flags=0):
    one = pw.Exchange(n, t, p, a_op=a_op, b_op=b_op, flags=flags | pw.PW_FLAG_ONE_LAUNCH, want_counts=True)
    split = pw.Exchange(n, t, p, a_op=a_op, b_op=b_op, flags=flags, want_counts=True)
    return one, split


def _same(a, b):
    if a is None:
        return b is None
    return torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                       b.view(torch.int32) if b.dtype == torch.float32 else b)


SHAPES = [
    # (N, T, P, dest kind): all fit one launch (<= 64 destinations, <= 256 slabs)
    (8, 4096, 64, "uniform"),      # the 8-shard step: 256 slabs of 128 tuples
    (8, 4095, 64, "half_empty"),   # ragged last slab, empty destinations
    (1, 1000, 4, "uniform"),
    (3, 300, 8, "uniform"),
    (16, 2000, 16, "zipf4"),
    (32, 1024, 64, "identity"),    # 256 slabs x 32 destinations: the largest slab table
    (64, 100, 128, "reversed"),
    (5, 7, 4, "uniform"),
]


@pytest.mark.parametrize("n,t,p,kind", SHAPES)
def test_one_launch_equals_split_launches_and_oracle(gpu, n, t, p, kind):
    pw = gpu
    print(f"one-launch exchange N={n} T={t} P={p} {kind}", flush=True)
    aff, rs = pw.op(pw.PW_OP_AFFINE, 2.0, 1.0), pw.op(pw.PW_OP_ROWSUM)
    x = torch.from_numpy(pw_inputs.exchange_uniform(n, t, p).x).cuda()
    dest = _dest(kind, n, t)
    dd = torch.from_numpy(dest).cuda()
    probe = pw.Exchange(n, t, p, flags=pw.PW_FLAG_TIMING | pw.PW_FLAG_ONE_LAUNCH)
    pw.future_wait(probe.step(x, dd), 30_000_000_000)
    assert set(probe.plan.kernel_times()) == {"exchange_small"}  # the step is one launch
    for a_op, b_op in ((aff, rs), (None, None), (aff, pw.op(pw.PW_OP_AFFINE, 0.5, 0.0))):
        one, split = _pair(pw, n, t, p, a_op, b_op, flags=pw.PW_FLAG_TRACE)
        for _ in range(3):  # repeated calls: the call-tagged slab table and the counter sets by call parity
            f1 = one.step(x, dd)
            f2 = split.step(x, dd)
        pw.future_wait(f1, 30_000_000_000)
        pw.future_wait(f2, 30_000_000_000)
        for name in ("dst", "src_index", "counts", "offsets", "b_out"):
            assert _same(getattr(one, name), getattr(split, name)), name
        ref = ox.exchange_step(x.cpu().numpy(), dest, n, n,
                               a_op=ox.op_affine(2.0, 1.0) if a_op is not None else ox.op_identity())
        assert np.array_equal(one.src_index.cpu().numpy(), ref.src_index.astype(np.int32))
        assert np.array_equal(one.dst.cpu().numpy().view(np.uint32), ref.y.view(np.uint32))
        ep, fi, st = one.plan.read_futures(trace=True)
        assert np.all(ep[pw.PW_NODE_EXCHANGE, :n] == 3) and np.all(fi[pw.PW_NODE_EXCHANGE, :n] == 3)
        assert np.all(ep[pw.PW_NODE_B, :n] == 3) and np.all(fi[pw.PW_NODE_B, :n] == 3)
        assert fi[pw.PW_NODE_RESULT, 0] == 3
        # gating, from the last call's stamps: EXCHANGE[d] <= B[d] <= Result
        assert np.all(st[pw.PW_NODE_EXCHANGE, :n] <= st[pw.PW_NODE_B, :n])
        assert np.all(st[pw.PW_NODE_B, :n] <= st[pw.PW_NODE_RESULT, 0])


def test_one_launch_new_inputs_every_call(gpu):
    """Back-to-back calls with different payloads and routings into the same
    output buffers: every call's rows, indices and row sums must be its own
    (the slab table is reused across calls, told apart by the call tag, and B
    reads rows written by other workgroups of the same launch; a stale read
    from an earlier call would show here, not with repeated inputs)."""
    pw = gpu
    n, t, p = 8, 4096, 64
    aff, rs = pw.op(pw.PW_OP_AFFINE, 2.0, 1.0), pw.op(pw.PW_OP_ROWSUM)
    one, split = _pair(pw, n, t, p, aff, rs)
    for k, kind in enumerate(("uniform", "zipf4", "reversed", "half_empty", "uniform")):
        print(f"one-launch call {k}: {kind}", flush=True)
        x = torch.from_numpy(pw_inputs.exchange_uniform(n, t, p, variant=100 + k).x).cuda()
        dest = _dest(kind, n, t, seed=k)
        dd = torch.from_numpy(dest).cuda()
        pw.future_wait(one.step(x, dd), 30_000_000_000)
        pw.future_wait(split.step(x, dd), 30_000_000_000)
        for name in ("dst", "src_index", "counts", "offsets", "b_out"):
            assert _same(getattr(one, name), getattr(split, name)), (k, name)
        ref = ox.exchange_step(x.cpu().numpy(), dest, n, n, a_op=ox.op_affine(2.0, 1.0))
        rows = int(ref.offsets[-1])
        assert np.array_equal(one.src_index.cpu().numpy()[:rows], ref.src_index.astype(np.int32))
        assert np.array_equal(one.dst.cpu().numpy().view(np.uint32)[:rows], ref.y.view(np.uint32))


def test_plan_calls_refuse_graph_capture(gpu):
    """A plan's call fixes its epoch (and the one-launch table tag) on the
    host, so a graph replay would reuse them: a call on a capturing stream
    returns PW_ERR_UNSUPPORTED and enqueues nothing; the plan then works as
    before."""
    pw = gpu
    n, t, p = 8, 512, 16
    x = torch.from_numpy(pw_inputs.exchange_uniform(n, t, p).x).cuda()
    dd = torch.from_numpy(_dest("uniform", n, t)).cuda()
    for flags in (0, pw.PW_FLAG_ONE_LAUNCH):
        ex = pw.Exchange(n, t, p, b_op=pw.op(pw.PW_OP_ROWSUM), flags=flags)
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with pytest.raises(pw.PwError) as err:
            with torch.cuda.graph(g, stream=s):
                ex.step(x, dd, stream=s)
        assert err.value.code == pw.PW_ERR_UNSUPPORTED and "graph" in str(err.value)
        pw.future_wait(ex.step(x, dd), 30_000_000_000)
        ref = ox.exchange_step(x.cpu().numpy(), _dest("uniform", n, t), n, n)
        assert np.array_equal(ex.dst.cpu().numpy().view(np.uint32), ref.y.view(np.uint32))


def test_one_launch_b_overlaps_the_exchange(gpu):
    """32 destinations fed by disjoint source shards (identity routing): each
    segment completes when its own 8 slabs have arrived, and B of a segment
    may fire while other segments are still arriving. Over 20 traced steps,
    count the steps where some B[d] fired before the last EXCHANGE[d']; the
    per-destination order holds in every step."""
    pw = gpu
    n, t, p = 32, 1024, 64
    x = torch.from_numpy(pw_inputs.exchange_uniform(n, t, p).x).cuda()
    dd = torch.from_numpy(_dest("identity", n, t)).cuda()
    ex = pw.Exchange(n, t, p, a_op=pw.op(pw.PW_OP_AFFINE, 2.0, 1.0), b_op=pw.op(pw.PW_OP_ROWSUM),
                     flags=pw.PW_FLAG_TRACE | pw.PW_FLAG_ONE_LAUNCH)
    overlapped = 0
    for _ in range(20):
        pw.future_wait(ex.step(x, dd), 30_000_000_000)
        _, _, st = ex.plan.read_futures(trace=True)
        xs, bs = st[pw.PW_NODE_EXCHANGE, :n].astype(np.int64), st[pw.PW_NODE_B, :n].astype(np.int64)
        assert np.all(xs <= bs)
        overlapped += int(bs.min() < xs.max())
    print(f"steps where some B[d] fired before the last EXCHANGE[d']: {overlapped} of 20", flush=True)


def test_one_launch_bad_destination(gpu):
    pw = gpu
    n, t = 8, 512
    x = torch.from_numpy(pw_inputs.exchange_uniform(n, t, 64).x).cuda()
    dest = _dest("uniform", n, t)
    dest[5] = n
    dest[600] = -1
    ex = pw.Exchange(n, t, 64, b_op=pw.op(pw.PW_OP_ROWSUM), flags=pw.PW_FLAG_ONE_LAUNCH)
    f = ex.step(x, torch.from_numpy(dest).cuda())
    with pytest.raises(pw.PwError) as e:
        pw.future_wait(f, 10_000_000_000)
    assert e.value.code == pw.PW_ERR_BAD_DEST
    ok = (dest >= 0) & (dest < n)
    offs = ex.offsets.cpu().numpy()
    assert offs[-1] == ok.sum()
    si = ex.src_index.cpu().numpy()[: offs[-1]]
    assert np.array_equal(si, np.flatnonzero(ok)[np.argsort(dest[ok], kind="stable")])
    dest[5], dest[600] = 1, 2
    pw.future_wait(ex.step(x, torch.from_numpy(dest).cuda()), 10_000_000_000)
