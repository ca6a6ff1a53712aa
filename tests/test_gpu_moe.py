"""GPU parity of the mixture-of-experts step (PATHWAYS page, section 6.3:
data-dependent routing of sub-examples to experts; section 4.3: the
exchange) against the CPU oracle, through the C ABI.

Bars:
  * router logits: |g - o| <= gamma_K (|x| . |W_r|) + 1e-30, gamma_K = K 2^-24
    (fp32 summation of exact bf16 products in any order, K = d);
  * routing, conditionally: the oracle's top-2, gates, exchange (counts,
    offsets, source index) recomputed from the GPU's own fp32 logits must
    match: experts and indices bit-exact, gates within 1e-6 relative, the
    dispatched rows bit-exact copies of the token rows;
  * expert outputs Y: within 1e-2 + 2e-2 |o| of the oracle's FFN on the same
    rows, and within one bf16 ulp + the fp32 summation bounds of both GEMMs
    (2^-7 |Y| + (2^-7 + gamma_H) (|H| . |W2|) + gamma_d 1.13 (|x| . |W1|) . |W2|);
  * combine, conditionally on the GPU's Y and gates: one bf16 ulp of the
    value + 2^-23 (|g0 y0| + |g1 y1|) (the fp32 product rounded before the
    fused add; it matters when the two terms cancel);
  * end to end from the tokens, on tokens the oracle routes the same way:
    within 1e-2 + 2e-2 |o|. Tokens whose 2nd and 3rd logits nearly tie may
    route differently; they are counted and must be near ties.
"""
import numpy as np
import pytest
import torch

import pw_inputs
from oracle import invariants as inv
from oracle import moe as om
from oracle import numerics as nm

pytestmark = pytest.mark.gpu


def run(pw, tokens, d, experts, hidden, shards, flags=0):
    inp = pw_inputs.moe(tokens, d, experts, hidden)
    wr, w1, w2 = inp.w_router.cuda(), inp.w1.cuda(), inp.w2.cuda()
    m = pw.MoE(wr, w1, w2, tokens, num_src_shards=shards, flags=flags, want_counts=True)
    f = m.step(inp.x.cuda())
    pw.future_wait(f, 120_000_000_000)
    return inp, m


def check_logits(x, wr, lg_gpu, rows=None):
    ref = om.router_logits(x, wr).astype(np.float64)
    summ = np.abs(x.astype(np.float64)) @ np.abs(wr.astype(np.float64))
    bound = x.shape[1] * 2.0 ** -24 * summ + 1e-30
    err = np.abs(lg_gpu.astype(np.float64) - ref)
    assert np.all(err <= bound), float((err / bound).max())
    return ref


def check_expert_rows(xrows, w1e, w2e, y_gpu):
    """Y rows of one expert against the oracle's FFN on the same input rows."""
    ref = om.expert_ffn(xrows, w1e, w2e).astype(np.float64)
    a1 = np.abs(xrows.astype(np.float64)) @ np.abs(w1e.astype(np.float64))
    h = nm.to_bf16(nm.to_f32(nm.gelu(nm.to_f32(xrows.astype(np.float64) @ w1e.astype(np.float64))))).astype(np.float64)
    w2a = np.abs(w2e.astype(np.float64))
    K1, K2 = w1e.shape[0], w2e.shape[0]
    bound = (2.0 ** -7 * np.maximum(np.abs(ref), np.abs(y_gpu)) + (2.0 ** -7 + K2 * 2.0 ** -24) * (np.abs(h) @ w2a)
             + K1 * 2.0 ** -24 * 1.13 * (a1 @ w2a))
    g = y_gpu.astype(np.float64)
    assert np.all(np.abs(g - ref) <= 1e-2 + 2e-2 * np.abs(ref)), float(np.abs(g - ref).max())
    assert np.all(np.abs(g - ref) <= bound), float((np.abs(g - ref) / (bound + 1e-30)).max())


@pytest.mark.parametrize("tokens,d,experts,hidden,shards", [
    (512, 256, 8, 512, 4), (300, 512, 64, 256, 3), (1000, 256, 2, 256, 8), (64, 256, 5, 768, 1),
    (1, 256, 4, 256, 1),   # one token: two expert rows, every other expert empty
    (400, 768, 8, 256, 2),  # the router's 6-block instance (one per d / 128)
    (700, 1280, 16, 256, 2),  # the largest d: the router's W_r^T fills a CU's whole LDS
    (4096, 256, 8, 256, 4)])  # 32 ranking tiles in 2 scan blocks: the one-workgroup scan launch
def test_moe_small(gpu, tokens, d, experts, hidden, shards):
    pw = gpu
    print(f"moe T={tokens} d={d} E={experts} H={hidden} S={shards}", flush=True)
    inp, m = run(pw, tokens, d, experts, hidden, shards, flags=pw.PW_FLAG_TRACE)
    x = inp.x.float().numpy()
    wr = inp.w_router.float().numpy()
    w1 = inp.w1.float().numpy()
    w2 = inp.w2.float().numpy()
    lg = m.logits.cpu().numpy()
    check_logits(x, wr, lg)
    # routing recomputed by the oracle from the GPU's logits
    cond = om.moe_step(x, wr, w1, w2, num_src=shards, logits=lg, with_ffn=False)
    assert np.array_equal(m.experts.cpu().numpy(), cond.experts.astype(np.int32))
    g = m.gates.cpu().numpy()
    assert np.all(np.abs(g - cond.gates) <= 1e-6 * np.abs(cond.gates))
    assert np.array_equal(m.offsets.cpu().numpy(), cond.offsets)
    assert np.array_equal(m.counts.cpu().numpy(), cond.counts.astype(np.int32))
    si = m.src_index.cpu().numpy()
    assert np.array_equal(si, cond.src_index.astype(np.int32))
    inv.check_exchange(cond.dest, experts, si, cond.offsets, cond.counts)
    xd = m.xd.float().cpu().numpy()
    assert np.array_equal(xd.view(np.uint32), x[si // 2].view(np.uint32))
    # expert outputs, per expert segment
    y = m.y.float().cpu().numpy()
    offs = cond.offsets
    for e in range(experts):
        if offs[e + 1] > offs[e]:
            check_expert_rows(xd[offs[e]:offs[e + 1]], w1[e], w2[e], y[offs[e]:offs[e + 1]])
    # combine, conditionally on the GPU's Y and gates
    pos = np.empty(2 * tokens, np.int64)
    pos[si] = np.arange(2 * tokens)
    y0, y1 = y[pos[0::2]].astype(np.float64), y[pos[1::2]].astype(np.float64)
    comb = om.combine_rows(g, y[pos[0::2]], y[pos[1::2]]).astype(np.float64)
    out = m.out.float().cpu().numpy().astype(np.float64)
    terms = np.abs(g[:, :1] * y0) + np.abs(g[:, 1:] * y1)
    assert np.all(np.abs(out - comb) <= 2.0 ** -7 * np.maximum(np.abs(comb), np.abs(out)) + 2.0 ** -23 * terms + 1e-30)
    # end to end from the tokens
    full = om.moe_step(x, wr, w1, w2, num_src=shards)
    same = np.all(full.experts == cond.experts, axis=1)
    o = full.out.astype(np.float64)
    assert np.all(np.abs(out[same] - o[same]) <= 1e-2 + 2e-2 * np.abs(o[same]))
    if not same.all():
        srt = np.sort(full.logits.astype(np.float64), axis=1)[:, ::-1]
        gaps = np.minimum(srt[:, 0] - srt[:, 1], srt[:, 1] - srt[:, 2])
        assert np.all(gaps[~same] < 1e-4), gaps[~same]
    # futures: every expert's exchange and FFN fired once, Result once
    ep, fi, st = m.plan.read_futures(trace=True)
    assert np.all(fi[pw.PW_NODE_EXCHANGE, :experts] == 1) and np.all(fi[pw.PW_NODE_B, :experts] == 1)
    assert fi[pw.PW_NODE_RESULT, 0] == 1
    assert np.all(st[pw.PW_NODE_EXCHANGE, :experts] <= st[pw.PW_NODE_B, :experts])
    assert np.all(st[pw.PW_NODE_B, :experts] <= st[pw.PW_NODE_RESULT, 0])


def test_moe_full_size(gpu):
    """131072 tokens x 1024, 64 experts, FFN 1024 -> 4096 -> 1024, the
    configuration the bench times. In full: every router logit against fp64,
    routing and the exchange (conditionally on the GPU's logits), every
    dispatched row bit for bit, the expert outputs of two whole experts (the
    largest and the smallest segment), and the combine of every token
    (conditionally on the GPU's expert outputs and gates). End to end from the
    tokens on a sample (the full oracle FFN is 4.4 TFLOP of fp64)."""
    pw = gpu
    tokens, d, experts, hidden = 131072, 1024, 64, 4096
    inp, m = run(pw, tokens, d, experts, hidden, 64)
    print("full-size moe: step done", flush=True)
    lg = m.logits.cpu().numpy()
    x = inp.x.float().numpy()
    wr = inp.w_router.float().numpy()
    for i in range(0, tokens, 16384):
        check_logits(x[i:i + 16384], wr, lg[i:i + 16384])
    experts_c, gates_c, dest_c, counts_c, offsets_c, si_c = om.route(lg, experts, 64)
    assert np.array_equal(m.experts.cpu().numpy(), experts_c.astype(np.int32))
    g = m.gates.cpu().numpy()
    assert np.all(np.abs(g - gates_c) <= 1e-6 * np.abs(gates_c))
    assert np.array_equal(m.offsets.cpu().numpy(), offsets_c)
    assert np.array_equal(m.counts.cpu().numpy(), counts_c.astype(np.int32))
    si = m.src_index.cpu().numpy()
    assert np.array_equal(si, si_c.astype(np.int32))
    print("full-size moe: logits within bounds, routing and exchange exact", flush=True)
    xbits = inp.x.view(torch.int16).numpy()
    xd = m.xd.view(torch.int16).cpu().numpy()
    assert np.array_equal(xd, xbits[si // 2])
    print(f"full-size moe: all {si.size} dispatched rows bit-exact", flush=True)
    y = m.y.float().cpu().numpy()
    sizes = np.diff(offsets_c)
    for e in (int(np.argmax(sizes)), int(np.argmin(sizes))):
        lo, hi = int(offsets_c[e]), int(offsets_c[e + 1])
        xr = x[si[lo:hi] // 2]  # the dispatched rows (equal to xd bit for bit, checked above)
        check_expert_rows(xr, inp.w1[e].float().numpy(), inp.w2[e].float().numpy(), y[lo:hi])
        print(f"full-size moe: expert {e}, all {hi - lo} rows within bounds", flush=True)
    pos = np.empty(2 * tokens, np.int64)
    pos[si] = np.arange(2 * tokens)
    out_all = m.out.float().cpu().numpy()
    for i in range(0, tokens, 16384):
        sl = slice(i, i + 16384)
        y0, y1 = y[pos[0::2][sl]], y[pos[1::2][sl]]
        comb = om.combine_rows(g[sl], y0, y1).astype(np.float64)
        out = out_all[sl].astype(np.float64)
        terms = np.abs(g[sl, :1] * y0.astype(np.float64)) + np.abs(g[sl, 1:] * y1.astype(np.float64))
        assert np.all(np.abs(out - comb) <= 2.0 ** -7 * np.maximum(np.abs(comb), np.abs(out)) + 2.0 ** -23 * terms
                      + 1e-30), i
    print(f"full-size moe: combine of all {tokens} tokens within bounds", flush=True)
    # end to end from the tokens on a sample (both slots through the oracle's FFN)
    rng = np.random.default_rng(9)
    sample = np.sort(rng.choice(tokens, size=48, replace=False))
    xs = x[sample]
    ref = []
    for i, t in enumerate(sample):
        ys = []
        for j in range(2):
            e = int(experts_c[t, j])
            ys.append(om.expert_ffn(xs[i:i + 1], inp.w1[e].float().numpy(), inp.w2[e].float().numpy())[0])
        ref.append(om.combine_rows(gates_c[t:t + 1], ys[0][None], ys[1][None])[0])
    ref = np.array(ref, dtype=np.float64)
    out = out_all[sample].astype(np.float64)
    assert np.all(np.abs(out - ref) <= 1e-2 + 2e-2 * np.abs(ref)), float(np.abs(out - ref).max())


# ---------------------------------------------------------------- capacity
# PATHWAYS page, section 4.5: a node whose resource needs depend on its
# predecessor's results is scheduled sequentially. With a capacity C each
# expert keeps its first C tuples in tuple order; the static path (one call)
# uses buffers of the bound min(2T, E C), the split path (begin, host reads
# the offsets, allocates exactly, end) buffers of the routed size. Both must
# match the oracle, and each other bit for bit.

def check_capacity_step(pw, m, inp, shards, cap):
    """Routing, dispatch, expert rows and combine of a capacity step against
    the oracle, conditionally on the GPU's logits; returns the kept rows."""
    x = inp.x.float().numpy()
    wr = inp.w_router.float().numpy()
    w1 = inp.w1.float().numpy()
    w2 = inp.w2.float().numpy()
    tokens, experts = x.shape[0], wr.shape[1]
    lg = m.logits.cpu().numpy()
    check_logits(x, wr, lg)
    cond = om.moe_step(x, wr, w1, w2, num_src=shards, logits=lg, with_ffn=False, capacity=cap)
    assert np.array_equal(m.experts.cpu().numpy(), cond.experts.astype(np.int32))
    g = m.gates.cpu().numpy()
    assert np.all(np.abs(g - cond.gates) <= 1e-6 * np.abs(cond.gates))
    offs = cond.offsets
    rows = int(offs[-1])
    assert np.array_equal(m.offsets.cpu().numpy(), offs)
    assert np.array_equal(m.counts.cpu().numpy(), cond.counts.astype(np.int32))   # routed, before the limit
    si = m.src_index.cpu().numpy()[:rows]
    assert np.array_equal(si, cond.src_index.astype(np.int32))
    xd = m.xd[:rows].float().cpu().numpy()
    assert np.array_equal(xd.view(np.uint32), x[si // 2].view(np.uint32))
    y = m.y[:rows].float().cpu().numpy()
    for e in range(experts):
        if offs[e + 1] > offs[e]:
            check_expert_rows(xd[offs[e]:offs[e + 1]], w1[e], w2[e], y[offs[e]:offs[e + 1]])
    pos = np.full(2 * tokens, -1, np.int64)
    pos[si] = np.arange(rows)
    yz = np.concatenate([y, np.zeros((1, y.shape[1]), np.float32)])  # row -1: a dropped tuple
    y0, y1 = yz[pos[0::2]], yz[pos[1::2]]
    comb = om.combine_rows(g, y0, y1).astype(np.float64)
    out = m.out.float().cpu().numpy().astype(np.float64)
    terms = np.abs(g[:, :1] * y0.astype(np.float64)) + np.abs(g[:, 1:] * y1.astype(np.float64))
    assert np.all(np.abs(out - comb) <= 2.0 ** -7 * np.maximum(np.abs(comb), np.abs(out)) + 2.0 ** -23 * terms + 1e-30)
    both = (pos[0::2] < 0) & (pos[1::2] < 0)
    assert np.all(out[both] == 0)
    return rows


@pytest.mark.parametrize("tokens,d,experts,hidden,shards,factor", [
    (512, 256, 8, 512, 4, 1.0), (300, 512, 64, 256, 3, 0.5), (1000, 256, 2, 256, 8, 0.75),
    (64, 256, 5, 768, 1, 0.25), (512, 256, 8, 256, 4, 4.0)])
def test_moe_capacity_static_and_split(gpu, tokens, d, experts, hidden, shards, factor):
    pw = gpu
    cap = max(1, int(factor * 2 * tokens / experts))
    print(f"moe capacity T={tokens} E={experts} C={cap}", flush=True)
    inp = pw_inputs.moe(tokens, d, experts, hidden)
    wr, w1, w2 = inp.w_router.cuda(), inp.w1.cuda(), inp.w2.cuda()
    x = inp.x.cuda()
    m = pw.MoE(wr, w1, w2, tokens, num_src_shards=shards, capacity=cap, want_counts=True)
    pw.future_wait(m.step(x), 120_000_000_000)
    rows = check_capacity_step(pw, m, inp, shards, cap)
    assert rows == int(np.minimum(m.counts.cpu().numpy().sum(axis=0), cap).sum())
    if factor < 1.0:
        assert rows < 2 * tokens  # something was dropped
    # the split step: same results, buffers of exactly `rows` rows
    m2 = pw.MoE(wr, w1, w2, tokens, num_src_shards=shards, capacity=cap, want_counts=True, static_buffers=False)
    pw.future_wait(m2.split_step(x), 120_000_000_000)
    assert m2.xd.shape[0] == rows and m2.y.shape[0] == rows
    assert np.array_equal(m2.offsets.cpu().numpy(), m.offsets.cpu().numpy())
    for a, b in ((m2.xd, m.xd[:rows]), (m2.y, m.y[:rows]), (m2.out, m.out), (m2.src_index[:rows], m.src_index[:rows])):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    # a second split step on the same plan (the open step closed properly)
    pw.future_wait(m2.split_step(x), 120_000_000_000)
    assert torch.equal(m2.out.view(torch.int16), m.out.view(torch.int16))


def test_moe_split_call_order_errors(gpu):
    pw = gpu
    import ctypes as C
    inp = pw_inputs.moe(256, 256, 4, 256)
    m = pw.MoE(inp.w_router.cuda(), inp.w1.cuda(), inp.w2.cuda(), 256, num_src_shards=1, capacity=100,
               static_buffers=False)
    x = inp.x.cuda()
    io = m._io(x)
    f = pw.pw_future_t()
    with pytest.raises(pw.PwError) as e:
        m.plan.exchange_end(io)
    assert e.value.code == pw.PW_ERR_STATE
    offs = m.plan.exchange_begin(io, 4)
    assert offs[0] == 0 and offs[-1] <= 400
    assert pw.lib.pw_exchange(m.plan.handle, C.byref(io), None, C.byref(f)) == pw.PW_ERR_STATE
    o2 = np.zeros(5, np.int64)
    assert pw.lib.pw_exchange_begin(m.plan.handle, C.byref(io), None, C.c_void_p(o2.ctypes.data)) == pw.PW_ERR_STATE
    other = x.clone()
    bad = m._io(other)
    assert pw.lib.pw_exchange_end(m.plan.handle, C.byref(bad), None, C.byref(f)) == pw.PW_ERR_INVALID
    # too small an output for what begin reported
    rows = int(offs[-1])
    xd = torch.empty((rows, 256), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((rows, 256), dtype=torch.bfloat16, device="cuda")
    io.dst = pw.sharded(xd, 4, 256, pw.PW_BF16, m.offsets)
    io.dst.num_tuples = rows - 1
    io.b_out = y.data_ptr()
    assert pw.lib.pw_exchange_end(m.plan.handle, C.byref(io), None, C.byref(f)) == pw.PW_ERR_INVALID
    io.dst.num_tuples = rows
    fut = m.plan.exchange_end(io)
    pw.future_wait(fut, 60_000_000_000)
    assert fut.epoch == 1


def test_moe_capacity_full_size(gpu):
    """131072 tokens x 1024, 64 experts, FFN 1024 -> 4096 -> 1024, capacity
    factor 1.0 (C = 4096 tuples per expert): the kept routing and exchange in
    full against the oracle (conditionally on the GPU's logits), the split
    step bit-identical to the static one, sampled tokens' outputs end to end."""
    pw = gpu
    tokens, d, experts, hidden = 131072, 1024, 64, 4096
    cap = 2 * tokens // experts
    inp = pw_inputs.moe(tokens, d, experts, hidden)
    wr, w1, w2 = inp.w_router.cuda(), inp.w1.cuda(), inp.w2.cuda()
    x = inp.x.cuda()
    m = pw.MoE(wr, w1, w2, tokens, num_src_shards=64, capacity=cap, want_counts=True)
    pw.future_wait(m.step(x), 120_000_000_000)
    print("full-size moe capacity: static step done", flush=True)
    lg = m.logits.cpu().numpy()
    experts_c, gates_c, dest_c, counts_c, offsets_c, si_c = om.route(lg, experts, 64, capacity=cap)
    assert np.array_equal(m.experts.cpu().numpy(), experts_c.astype(np.int32))
    assert np.array_equal(m.offsets.cpu().numpy(), offsets_c)
    assert np.array_equal(m.counts.cpu().numpy(), counts_c.astype(np.int32))
    rows = int(offsets_c[-1])
    assert rows < 2 * tokens
    si = m.src_index[:rows].cpu().numpy()
    assert np.array_equal(si, si_c.astype(np.int32))
    m2 = pw.MoE(wr, w1, w2, tokens, num_src_shards=64, capacity=cap, static_buffers=False)
    pw.future_wait(m2.split_step(x), 120_000_000_000)
    print("full-size moe capacity: split step done", flush=True)
    assert torch.equal(m2.y.view(torch.int16), m.y[:rows].view(torch.int16))
    assert torch.equal(m2.out.view(torch.int16), m.out.view(torch.int16))
    # sampled tokens end to end (oracle FFN on the token's kept tuples)
    rng = np.random.default_rng(19)
    pos = np.full(2 * tokens, -1, np.int64)
    pos[si] = np.arange(rows)
    dropped = np.flatnonzero((pos[0::2] < 0) | (pos[1::2] < 0))
    kept = np.flatnonzero((pos[0::2] >= 0) & (pos[1::2] >= 0))
    sample = np.sort(np.concatenate([rng.choice(kept, 16, replace=False), rng.choice(dropped, 16, replace=False)]))
    xs = inp.x[torch.from_numpy(sample)].float().numpy()
    out = m.out[torch.from_numpy(sample).cuda()].float().cpu().numpy().astype(np.float64)
    for i, t in enumerate(sample):
        ys = []
        for j in range(2):
            e = int(experts_c[t, j])
            ys.append(om.expert_ffn(xs[i:i + 1], inp.w1[e].float().numpy(), inp.w2[e].float().numpy())[0]
                      if pos[2 * t + j] >= 0 else np.zeros(d, np.float32))
        ref = om.combine_rows(gates_c[t:t + 1], ys[0][None], ys[1][None])[0].astype(np.float64)
        assert np.all(np.abs(out[i] - ref) <= 1e-2 + 2e-2 * np.abs(ref)), (t, float(np.abs(out[i] - ref).max()))
