"""pw_exchange_scratch, the allocation-free form of the EXCHANGE step (its
tables in the library's static 8 MiB device array), against pw_exchange on
the same inputs: every output bit for bit, on consecutive calls of different
shapes (the second smaller, so it runs over the first call's leftovers)."""
import numpy as np
import pytest
import torch

import pw_inputs

pytestmark = pytest.mark.gpu


def _dest(n, t, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "zipf4":
        return pw_inputs.exchange_zipf(n, t, 1, with_payload=False).dest
    return rng.integers(0, n, size=n * t).astype(np.int32)


def _compare(pw, n, t, p, kind, a_op, b_op, seed):
    print(f"scratch exchange N={n} T={t} P={p} {kind}", flush=True)
    x = torch.from_numpy(pw_inputs.exchange_uniform(n, t, p).x).cuda()
    d = torch.from_numpy(_dest(n, t, kind, seed)).cuda()
    ex = pw.Exchange(n, t, p, a_op=a_op, b_op=b_op, want_counts=True)
    pw.future_wait(ex.step(x, d), 30_000_000_000)
    dst = torch.full_like(ex.dst, float("nan"))
    offs = torch.full_like(ex.offsets, -1)
    si = torch.full_like(ex.src_index, -1)
    cnt = torch.full_like(ex.counts, -1)
    bo = torch.full_like(ex.b_out, float("nan")) if ex.b_out is not None else None
    io = pw.exchange_io(x, d, dst, n, n, p, src_index=si, counts=cnt, offsets=offs, b_out=bo)
    pw.exchange_scratch(ex.desc, io)
    torch.cuda.synchronize()
    assert torch.equal(offs, ex.offsets)
    assert torch.equal(si, ex.src_index)
    assert torch.equal(cnt, ex.counts)
    assert torch.equal(dst.view(torch.int32), ex.dst.view(torch.int32))
    if bo is not None:
        assert torch.equal(bo.view(torch.int32), ex.b_out.view(torch.int32))
    assert int(offs[-1]) == n * t


def test_scratch_exchange_matches_the_planned_one(gpu):
    pw = gpu
    aff, rs = pw.op(pw.PW_OP_AFFINE, 2.0, 1.0), pw.op(pw.PW_OP_ROWSUM)
    _compare(pw, 64, 999, 16, "zipf4", aff, rs, 1)      # ~1 MB of tables
    _compare(pw, 8, 100, 64, "uniform", aff, rs, 2)     # smaller: over the first call's leftovers
    _compare(pw, 8, 4096, 64, "uniform", aff, rs, 3)    # the 8-shard step with A and B
    _compare(pw, 3, 7, 4, "uniform", None, None, 4)     # identity A and B, tiny


def test_scratch_exchange_rejects_what_does_not_fit(gpu):
    pw = gpu
    d = pw.desc(pw.PW_GRAPH_EXCHANGE, 256, 65536, 64)
    x = torch.empty((1, 64), device="cuda")
    io = pw.exchange_io(x, None, x, 256, 256, 64)
    with pytest.raises(pw.PwError) as e:
        pw.exchange_scratch(d, io)
    assert e.value.code == pw.PW_ERR_INVALID and "8388608" in str(e.value)
