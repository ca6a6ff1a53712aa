"""GPU parity of the exchange (PATHWAYS page, section 4.3) against the CPU
oracle, through the C ABI.

Bar: routing, indices, offsets, counts and payload bits are bit-exact; the
fp32 A = 2x + 1 is bit-exact (one rounding, 2x exact); B = per-tuple sum is
within 1e-6 relative of the oracle's fp64 sum: the GPU sums 64 fp32 terms in
a tree of depth 6, whose error is at most 6 * 2^-24 * sum|x| (plus one final
rounding), and on these inputs sum|x| / |sum x| <= 2.1, so the error stays
below 7.6e-7 |sum x|. Rows whose sum nearly cancels (|sum x| < 1e-3 sum|x|)
would need the absolute form of that bound; none occur on the workload and
the test counts them. Every future fires exactly once per call and only
after its inputs.
"""
import numpy as np
import pytest
import torch

import pw_inputs
from oracle import exchange as ox
from oracle import invariants as inv

pytestmark = pytest.mark.gpu


def _dest_case(kind, n, t):
    g = n * t
    rng = np.random.default_rng(n * 1000 + t)
    if kind == "uniform":
        return rng.integers(0, n, size=g).astype(np.int32)
    if kind == "zipf4":
        return pw_inputs.exchange_zipf(n, t, 1, with_payload=False).dest
    if kind == "all_to_one":
        return np.full(g, n // 2, np.int32)
    if kind == "identity":
        return np.repeat(np.arange(n, dtype=np.int32), t)
    if kind == "reversed":
        return np.repeat(np.arange(n - 1, -1, -1, dtype=np.int32), t)
    if kind == "half_empty":
        return (rng.integers(0, max(n // 2, 1), size=g) * 2 % n).astype(np.int32)
    raise ValueError(kind)


def run(pw, x, dest, n, t, a_op=None, b_op=None, dtype=None, flags=0, counts=True, repeats=1):
    dtype = pw.PW_F32 if dtype is None else dtype
    p = x.shape[1]
    ex = pw.Exchange(n, t, p, dtype=dtype, a_op=a_op, b_op=b_op, flags=flags, want_counts=counts)
    xd = x.cuda()
    dd = torch.from_numpy(dest).cuda()
    futs = []
    for _ in range(repeats):
        futs.append(ex.step(xd, dd))
    pw.future_wait(futs[-1], 30_000_000_000)
    torch.cuda.synchronize()
    return ex, futs


def check_rowsum(got, y, ref_sum):
    """B = per-tuple sum against the oracle's fp64 sum: within 1e-6 relative;
    a row whose sum nearly cancels is held to the fp32 tree bound instead."""
    got = got.astype(np.float64)
    ref = np.asarray(ref_sum, dtype=np.float64)
    mag = np.abs(y.astype(np.float64)).sum(axis=1)
    err = np.abs(got - ref)
    cancel = np.abs(ref) < 1e-3 * mag
    assert np.all(err[~cancel] <= 1e-6 * np.abs(ref[~cancel])), float((err[~cancel] / np.abs(ref[~cancel])).max())
    assert np.all(err[cancel] <= 7 * 2.0 ** -24 * mag[cancel])
    print(f"row sums: max relative error {float((err[~cancel] / np.abs(ref[~cancel])).max()):.2e}, "
          f"{int(cancel.sum())} near-cancelling rows", flush=True)
    return int(cancel.sum())


def _bits(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    return t.numpy().view(np.uint32)


CASES = [
    # (N, T, P, dest kind)
    (1, 1000, 4, "uniform"),
    (2, 37, 64, "uniform"),
    (3, 300, 8, "uniform"),
    (8, 4096, 64, "uniform"),
    (8, 4095, 64, "half_empty"),
    (64, 1001, 16, "zipf4"),
    (255, 333, 4, "uniform"),
    (256, 700, 64, "zipf4"),
    (256, 513, 64, "all_to_one"),
    (64, 300, 64, "identity"),
    (64, 300, 64, "reversed"),
    (2048, 50, 4, "uniform"),
    (2048, 33, 4, "zipf4"),
    (8192, 3, 4, "uniform"),      # the most shards a plan takes: the ranking kernel's LDS is then 128 KiB
    (8192, 2, 64, "half_empty"),
    (4, 10, 8192, "uniform"),     # 32 KiB rows: one tuple per scatter workgroup, two copy batches each
    (1024, 4, 16, "zipf4"),       # <= 16 ranking tiles: the last ranking workgroup runs the scan
    (16, 8192, 16, "uniform"),    # 16 scan blocks x 16 destinations: the most the fused one-column-per-thread scan takes
    (32, 2048, 16, "zipf4"),      # 8 blocks x 32 destinations, fused; (64, 1001) above: 8 x 64, a scan launch
    (2048, 2, 4, "uniform"),
]


@pytest.mark.parametrize("n,t,p,kind", CASES)
def test_exchange_parity(gpu, n, t, p, kind):
    pw = gpu
    print(f"exchange parity N={n} T={t} P={p} {kind}", flush=True)
    x = torch.from_numpy(pw_inputs.exchange_uniform(n, t, p).x)
    dest = _dest_case(kind, n, t)
    ex, futs = run(pw, x, dest, n, t)
    ref = ox.exchange_step(x.numpy(), dest, n, n)
    assert np.array_equal(ex.offsets.cpu().numpy(), ref.offsets)
    assert np.array_equal(ex.src_index.cpu().numpy(), ref.src_index.astype(np.int32))
    assert np.array_equal(ex.counts.cpu().numpy(), ref.counts.astype(np.int32))
    assert np.array_equal(_bits(ex.dst), ref.y.view(np.uint32))
    inv.check_exchange(dest, n, ex.src_index.cpu().numpy(), ex.offsets.cpu().numpy(), ex.counts.cpu().numpy(),
                       ex.dst.cpu().numpy(), x.numpy())
    ep, fi, _ = ex.plan.read_futures()
    assert np.all(ep[pw.PW_NODE_EXCHANGE, :n] == 1) and np.all(fi[pw.PW_NODE_EXCHANGE, :n] == 1)
    assert np.all(ep[pw.PW_NODE_B, :n] == 1) and np.all(fi[pw.PW_NODE_B, :n] == 1)
    assert ep[pw.PW_NODE_RESULT, 0] == 1 and fi[pw.PW_NODE_RESULT, 0] == 1


def test_more_than_4096_tiles(gpu):
    """18 M tuples over 3 destinations: 4395 ranking tiles, so the scan's
    blocks hold 32 tiles (two rounds per column) and its second level runs
    as its own launch with a partial group of destinations."""
    pw = gpu
    n, t = 3, 6_000_000
    print(f"exchange N={n} T={t} P=1 (more than 4096 tiles)", flush=True)
    x = torch.from_numpy(pw_inputs.exchange_uniform(n, t, 1).x)
    dest = _dest_case("uniform", n, t)
    ex, _ = run(pw, x, dest, n, t)
    ref = ox.exchange_step(x.numpy(), dest, n, n)
    assert np.array_equal(ex.offsets.cpu().numpy(), ref.offsets)
    assert np.array_equal(ex.counts.cpu().numpy(), ref.counts.astype(np.int32))
    assert np.array_equal(ex.src_index.cpu().numpy(), ref.src_index.astype(np.int32))
    assert np.array_equal(_bits(ex.dst), ref.y.view(np.uint32))
    ep, fi, _ = ex.plan.read_futures()
    assert np.all(fi[pw.PW_NODE_EXCHANGE, :n] == 1) and fi[pw.PW_NODE_RESULT, 0] == 1


def test_tiny_rows_full_size_chunks(gpu):
    """16.7 M tuples of one fp32: 4096-tuple tiles and the largest scatter
    chunk (1024 tuples per workgroup, 4 per tile)."""
    pw = gpu
    n, t = 64, 262144
    print(f"exchange tiny rows N={n} T={t} P=1", flush=True)
    x = torch.from_numpy(pw_inputs.exchange_uniform(n, t, 1).x)
    dest = _dest_case("zipf4", n, t)
    ex, _ = run(pw, x, dest, n, t)
    ref = ox.exchange_step(x.numpy(), dest, n, n)
    assert np.array_equal(ex.offsets.cpu().numpy(), ref.offsets)
    assert np.array_equal(ex.src_index.cpu().numpy(), ref.src_index.astype(np.int32))
    assert np.array_equal(_bits(ex.dst), ref.y.view(np.uint32))
    ep, fi, _ = ex.plan.read_futures()
    assert np.all(fi[pw.PW_NODE_EXCHANGE, :n] == 1) and fi[pw.PW_NODE_RESULT, 0] == 1


def test_small_workload_a_and_b(gpu):
    """8 shards x 4096 tuples, A = 2x + 1, B = per-tuple sum: the full step."""
    pw = gpu
    inp = pw_inputs.exchange_uniform(8, 4096, 64)
    x = torch.from_numpy(inp.x)
    ex, _ = run(pw, x, inp.dest, 8, 4096, a_op=pw.op(pw.PW_OP_AFFINE, 2.0, 1.0), b_op=pw.op(pw.PW_OP_ROWSUM),
                flags=pw.PW_FLAG_TRACE)
    ref = ox.exchange_step(inp.x, inp.dest, 8, 8, a_op=ox.op_affine(2.0, 1.0), b_op=ox.op_rowsum())
    assert np.array_equal(ex.src_index.cpu().numpy(), ref.src_index.astype(np.int32))
    assert np.array_equal(_bits(ex.dst), ref.y.view(np.uint32))          # A bit-exact
    check_rowsum(ex.b_out.cpu().numpy(), ref.y, ref.b_out)
    ep, fi, st = ex.plan.read_futures(trace=True)
    assert np.all(fi[pw.PW_NODE_EXCHANGE, :8] == 1) and np.all(fi[pw.PW_NODE_B, :8] == 1)
    # fire order respects the graph: exchange[d] before B[d] before Result
    for d in range(8):
        assert st[pw.PW_NODE_EXCHANGE, d] <= st[pw.PW_NODE_B, d] <= st[pw.PW_NODE_RESULT, 0]


def test_bf16_payloads_and_odd_rows(gpu):
    pw = gpu
    for n, t, p in [(64, 257, 1024), (5, 300, 6), (7, 99, 2)]:
        print(f"bf16 exchange N={n} T={t} P={p}", flush=True)
        xf = pw_inputs.exchange_uniform(n, t, p).x
        x = torch.from_numpy(xf).to(torch.bfloat16)
        dest = _dest_case("uniform", n, t)
        ex, _ = run(pw, x, dest, n, t, dtype=pw.PW_BF16)
        ref = ox.exchange_step(x.float().numpy(), dest, n, n)
        assert np.array_equal(ex.src_index.cpu().numpy(), ref.src_index.astype(np.int32))
        assert np.array_equal(ex.dst.float().cpu().numpy().view(np.uint32), ref.y.view(np.uint32))


def test_repeated_calls_are_deterministic_and_fire_once_each(gpu):
    pw = gpu
    n, t = 64, 999
    x = torch.from_numpy(pw_inputs.exchange_uniform(n, t, 16).x)
    dest = _dest_case("zipf4", n, t)
    ex = pw.Exchange(n, t, 16, want_counts=True)
    xd, dd = x.cuda(), torch.from_numpy(dest).cuda()
    first = None
    for i in range(20):
        ex.dst.fill_(float("nan"))
        ex.src_index.fill_(-1)
        f = ex.step(xd, dd)
        pw.future_wait(f, 30_000_000_000)
        assert f.epoch == i + 1
        cur = (_bits(ex.dst).copy(), ex.src_index.cpu().numpy().copy())
        if first is None:
            first = cur
        else:
            assert np.array_equal(cur[0], first[0]) and np.array_equal(cur[1], first[1])
    ep, fi, _ = ex.plan.read_futures()
    assert np.all(ep[pw.PW_NODE_EXCHANGE, :n] == 20) and np.all(fi[pw.PW_NODE_EXCHANGE, :n] == 20)
    assert fi[pw.PW_NODE_RESULT, 0] == 20
    assert pw.future_query(f)


def test_empty_exchange(gpu):
    pw = gpu
    ex = pw.Exchange(5, 0, 4, want_index=False)
    x = torch.empty((0, 4), device="cuda")
    dest = torch.empty(0, dtype=torch.int32, device="cuda")
    f = ex.step(x, dest)
    pw.future_wait(f, 10_000_000_000)
    assert ex.offsets.cpu().tolist() == [0] * 6
    ep, fi, _ = ex.plan.read_futures()
    assert np.all(fi[pw.PW_NODE_EXCHANGE, :5] == 1) and fi[pw.PW_NODE_RESULT, 0] == 1


def test_bad_destination_is_reported(gpu):
    pw = gpu
    n, t = 4, 100
    x = torch.from_numpy(pw_inputs.exchange_uniform(n, t, 4).x)
    dest = _dest_case("uniform", n, t)
    dest[17] = 9
    dest[50] = -3
    ex = pw.Exchange(n, t, 4)
    f = ex.step(x.cuda(), torch.from_numpy(dest).cuda())
    with pytest.raises(pw.PwError) as e:
        pw.future_wait(f, 10_000_000_000)
    assert e.value.code == pw.PW_ERR_BAD_DEST
    # the valid tuples were still exchanged stably
    ok = (dest >= 0) & (dest < n)
    offs = ex.offsets.cpu().numpy()
    assert offs[-1] == ok.sum()
    si = ex.src_index.cpu().numpy()[: offs[-1]]
    assert np.array_equal(si, np.flatnonzero(ok)[np.argsort(dest[ok], kind="stable")])
    # the status was reported once; a clean call afterwards succeeds
    dest[17], dest[50] = 1, 2
    f = ex.step(x.cuda(), torch.from_numpy(dest).cuda())
    pw.future_wait(f, 10_000_000_000)


def test_large_zipf_exchange_full_size(gpu):
    """256 shards x 65536 tuples x 64 fp32, Zipf(1.1) choice of 4 destinations,
    the configuration the bench times: offsets, counts and source indices in
    full against the oracle, and every one of the 16,777,216 payload rows bit
    for bit against the source row its index names (compared in 1 Mi-row
    chunks on the host)."""
    pw = gpu
    inp = pw_inputs.exchange_zipf(256, 65536, 64)
    print("full-size zipf exchange: inputs ready", flush=True)
    ex, _ = run(pw, torch.from_numpy(inp.x), inp.dest, 256, 65536, counts=True)
    counts = ox.histogram(inp.dest, 256, 256, 65536)
    offsets = ox.exclusive_scan(counts.sum(axis=0))
    src_index = ox.stable_place(inp.dest, offsets)
    assert np.array_equal(ex.offsets.cpu().numpy(), offsets)
    assert np.array_equal(ex.counts.cpu().numpy(), counts.astype(np.int32))
    si = ex.src_index.cpu().numpy()
    assert np.array_equal(si, src_index.astype(np.int32))
    g = si.size
    xb = inp.x.view(np.uint32)
    step = 1 << 20
    for i in range(0, g, step):
        got = ex.dst[i:i + step].cpu().numpy().view(np.uint32)
        assert np.array_equal(got, xb[src_index[i:i + step]]), i
    print(f"full-size zipf exchange: all {g} payload rows bit-exact", flush=True)


def test_every_shard_future_waited_individually(gpu):
    """PATHWAYS page, sections 4.4-4.5: computations consume buffer futures.
    Each EXCHANGE[d] and B[d] future of a step is waited on by itself (the wait
    polls that future's own word in the device table) and queried, for two
    calls in a row: each returns with its call's epoch and no error."""
    pw = gpu
    n, t = 16, 2000
    x = torch.from_numpy(pw_inputs.exchange_uniform(n, t, 16).x).cuda()
    dest = torch.from_numpy(_dest_case("zipf4", n, t)).cuda()
    ex = pw.Exchange(n, t, 16, b_op=pw.op(pw.PW_OP_ROWSUM))
    for call in (1, 2):
        f = ex.step(x, dest)
        assert f.epoch == call
        for node in (pw.PW_NODE_EXCHANGE, pw.PW_NODE_B):
            for d in range(n):
                fd = pw.pw_future_t(f.plan_id, node, d, f.epoch)
                pw.future_wait(fd, 10_000_000_000)
                assert pw.future_query(fd)
        pw.future_wait(f, 10_000_000_000)
    ep, fi, _ = ex.plan.read_futures()
    assert np.all(ep[pw.PW_NODE_EXCHANGE, :n] == 2) and np.all(fi[pw.PW_NODE_B, :n] == 2)
    later = pw.pw_future_t(f.plan_id, pw.PW_NODE_B, 0, 3)  # an epoch never launched
    with pytest.raises(pw.PwError) as e:
        pw.future_wait(later, 1_000_000)
    assert e.value.code == pw.PW_ERR_STATE


def test_device_error_is_reported_to_its_own_call(gpu):
    """A destination out of range in the second of three calls is latched
    with that call's epoch: waits on the first call return OK, the second
    reports PW_ERR_BAD_DEST, the third OK."""
    pw = gpu
    n, t = 4, 100
    x = torch.from_numpy(pw_inputs.exchange_uniform(n, t, 4).x).cuda()
    good = _dest_case("uniform", n, t)
    bad = good.copy()
    bad[17] = 9
    ex = pw.Exchange(n, t, 4)
    g, b = torch.from_numpy(good).cuda(), torch.from_numpy(bad).cuda()
    f1 = ex.step(x, g)
    f2 = ex.step(x, b)
    f3 = ex.step(x, g)
    torch.cuda.synchronize()
    pw.future_wait(pw.pw_future_t(f1.plan_id, pw.PW_NODE_EXCHANGE, 0, f1.epoch), 10_000_000_000)
    pw.future_wait(f1, 10_000_000_000)
    with pytest.raises(pw.PwError) as e:
        pw.future_wait(f2, 10_000_000_000)
    assert e.value.code == pw.PW_ERR_BAD_DEST
    pw.future_wait(f3, 10_000_000_000)
