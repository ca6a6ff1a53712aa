"""GPU parity of the exchange (PATHWAYS page, section 4.3) against the CPU
oracle, through the C ABI.

Bar: routing, indices, offsets, counts and payload bits are bit-exact; the
fp32 A = 2x + 1 is bit-exact (one rounding, 2x exact); B = per-tuple sum is
within 1e-6 of the sum of magnitudes of its terms (fp32 summation bound, a
depth-6 tree: 6 * 2^-24 * sum|x| < 1e-6 * sum|x|); every future fires
exactly once per call and only after its inputs.
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
    got = ex.b_out.cpu().numpy().astype(np.float64)
    mag = np.abs(ref.y.astype(np.float64)).sum(axis=1)
    assert np.all(np.abs(got - ref.b_out.astype(np.float64)) <= 1e-6 * mag)
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
    """256 shards x 65536 tuples x 64 fp32, Zipf(1.1) choice of 4 destinations:
    indices and offsets checked in full, payload rows on a sample."""
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
    rng = np.random.default_rng(0)
    sample = np.sort(rng.choice(si.size, size=200_000, replace=False))
    got = ex.dst[torch.from_numpy(sample).cuda()].cpu().numpy()
    assert np.array_equal(got.view(np.uint32), inp.x[src_index[sample]].view(np.uint32))
