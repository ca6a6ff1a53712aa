"""Benchmark of the sharded-dataflow hot path on one MI355X.

A step is one pass of Arg -> A -> sparse exchange (ranking, scan, stable
scatter, progress futures) -> B -> Result over the large exchange workload:
256 shards x 65536 tuples, 64 fp32 payload ~ N(0, 1), each source sending to
4 destinations drawn with Zipf(1.1) weights (A and B are identities). Inputs
are resident in HBM before the timed region. One JSON line goes to stdout.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

`value` = exchanged tuples per second (whole step, K steps between two
synchronisations). `roofline` prices the dominant kernel (the scatter) at its
algorithmic bytes (520 B per tuple: 256 B payload read + 256 B written, 4 B
destination read, 4 B source index written) over its mean HIP-event duration
in a second timed region of K steps on a plan that records events around
every kernel (kept out of the first, whose `value` they would lower by
~1.5%), against the 8 TB/s HBM peak. `cpu_baseline` times the
CPU oracle (single-threaded NumPy) on the same workload. Further sections:
`inputs` (versions, SHA-256 of the inputs), `small_step` (the 8-shard step
with A and B, warm and cold), `pipeline`, `moe`, the chain sweep, the vendor
references, and the optional studies.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "exchanged tuples/s & % HBM peak; chained sharded A->B steps/s vs N"
BYTES_PER_TUPLE = 520


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_info():
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model or platform.processor(), "os_cpu_count": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0))}


def traffic_for(kernel_src: str, kernel: str, launches_g: int):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current source of the kernel (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(kernel)
    if not rec:
        return None
    with open(kernel_src, "rb") as f:
        h = hashlib.sha256(f.read()).hexdigest()
    if rec.get("source_sha256") != h:
        return None
    return rec.get("bytes_per_launch")


def chain_sweep(pw, torch, pw_inputs, steps):
    """Chained Arg -> A -> B -> Result steps (A = x + 1, B = x / 2, 128 fp32 per
    shard) per second against N, for the three submission modes."""
    modes = {"chained": pw.PW_CHAIN_CHAINED, "split": pw.PW_CHAIN_SPLIT, "opbyop": pw.PW_CHAIN_OPBYOP,
             "fused": pw.PW_CHAIN_FUSED}
    out = {"steps": steps, "elems_per_shard": 128, "steps_per_s": {}, "ns_per_node": {},
           "placement": "chained: A[i] and B[i] on the same lanes (gate ordered by program order); split: A[i] "
                        "and B[i] on different workgroups, normally different XCDs (cross-CU handoff: coherent stores, epoch, coherent loads)",
           "split_cross_xcd_fraction": {}}
    for name, mode in modes.items():
        out["steps_per_s"][name] = {}
        out["ns_per_node"][name] = {}
        for n in (8, 64, 256, 2048):
            ch = pw.Chain(n, 128, mode=mode)
            st = torch.from_numpy(pw_inputs.chain_state(n, 128)).cuda()
            pw.future_wait(ch.run(st, min(steps, 1000)), 60_000_000_000)
            torch.cuda.synchronize()
            s = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            t0 = time.perf_counter()
            f = ch.run(st, steps)
            e1.record(s)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            pw.future_wait(f, 60_000_000_000)
            sec = max(e0.elapsed_time(e1) * 1e-3, wall)
            out["steps_per_s"][name][n] = steps / sec
            out["ns_per_node"][name][n] = sec / (2 * steps) * 1e9
            if name == "split":
                pl = ch.placement()
                out["split_cross_xcd_fraction"][n] = float((pl[:, 0] != pl[:, 1]).mean())
            ch.plan.destroy()
    return out


def dispatch_study(pw, torch, pw_inputs, total=4096):
    """Per-node cost of the chained A -> B program against program length D
    (steps per call) for five ways of dispatching it: the persistent executor
    (one launch per call, device-side futures gate every node) with A[i] and
    B[i] on the same wave ("chained") or on different workgroups, normally on
    different XCDs ("split": every gate a cross-workgroup release and
    acquire), parallel asynchronous dispatch (one launch per node, all
    enqueued without waiting), a fused kernel loop (no futures), and
    sequential dispatch (one step per call, the host waiting for it before the
    next)."""
    modes = {"chained": pw.PW_CHAIN_CHAINED, "split": pw.PW_CHAIN_SPLIT, "opbyop": pw.PW_CHAIN_OPBYOP,
             "fused": pw.PW_CHAIN_FUSED}
    depths = (1, 4, 16, 64, 256, 1024, 4096)
    out = {"total_steps_per_point": total, "elems_per_shard": 128, "unit": "ns per gated node (2 nodes per step)",
           "by_n": {}}
    for n in (256, 2048):
        row = {}
        st0 = torch.from_numpy(pw_inputs.chain_state(n, 128)).cuda()
        for name, mode in modes.items():
            ch = pw.Chain(n, 128, mode=mode)
            row[name] = {}
            for depth in depths:
                st = st0.clone()
                pw.future_wait(ch.run(st, depth), 60_000_000_000)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(total // depth):
                    f = ch.run(st, depth)
                pw.future_wait(f, 60_000_000_000)
                torch.cuda.synchronize()
                row[name][depth] = (time.perf_counter() - t0) / (2 * total) * 1e9
            ch.plan.destroy()
        ch = pw.Chain(n, 128, mode=pw.PW_CHAIN_OPBYOP)
        st = st0.clone()
        steps = 512
        t0 = time.perf_counter()
        for _ in range(steps):
            pw.future_wait(ch.run(st, 1), 60_000_000_000)
        row["sequential"] = {1: (time.perf_counter() - t0) / (2 * steps) * 1e9}
        ch.plan.destroy()
        out["by_n"][n] = row
    return out


def multi_tenant(pw, torch, pw_inputs, point_s=1.5, target_ms=0.33):
    """Programs of concurrent clients through the multi-tenant scheduler
    (PATHWAYS page, section 5.2, Figures 8 and 9; Appendix D, Figure 11).
    A program is a chained run of D steps over 256 shards x 128 fp32, D sized
    to ~0.33 ms of device time. Throughput: each client a host thread in a
    closed loop (submit, wait), per client count, against one client calling
    the plan directly (no scheduler); busy = summed device time of the
    programs over the span from the first start to the last end. Shares: four
    clients with every program queued up front, device time per client over
    the dispatches before the first client runs dry."""
    import threading
    n, e = 256, 128
    x0 = torch.from_numpy(pw_inputs.chain_state(n, e)).cuda()
    cal = pw.Chain(n, e)
    st = x0.clone()
    pw.future_wait(cal.run(st, 256), 60_000_000_000)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    pw.future_wait(cal.run(st, 4096), 60_000_000_000)
    step_s = (time.perf_counter() - t0) / 4096
    d = max(1, int(round(target_ms * 1e-3 / step_s)))
    cal.plan.destroy()
    out = {"program": f"chained run of {d} steps, {n} shards x {e} fp32", "steps_per_program": d}

    # one client calling the plan directly, no scheduler
    ch = pw.Chain(n, e)
    st = x0.clone()
    pw.future_wait(ch.run(st, d), 60_000_000_000)
    k = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < point_s:
        pw.future_wait(ch.run(st, d), 60_000_000_000)
        k += 1
    wall = time.perf_counter() - t0
    out["direct_one_client"] = {"programs_per_s": k / wall, "program_ms_wall": wall / k * 1e3}
    ch.plan.destroy()

    def closed_loop(clients, weights=None):
        sch = pw.Sched(2)
        chains = [pw.Chain(n, e) for _ in range(clients)]
        states = [x0.clone() for _ in range(clients)]
        for c in range(clients):
            sch.add_client(weights[c] if weights else 1)
        for c in range(clients):  # warm the plans
            sch.wait(sch.submit_chain(c, chains[c], states[c], d), 60_000_000_000)
        sch.records()
        stop = [False]
        done = [0] * clients

        def client(c):
            while not stop[0]:
                sch.wait(sch.submit_chain(c, chains[c], states[c], d), 60_000_000_000)
                done[c] += 1

        ths = [threading.Thread(target=client, args=(c,)) for c in range(clients)]
        t0 = time.perf_counter()
        for th in ths:
            th.start()
        time.sleep(point_s)
        stop[0] = True
        for th in ths:
            th.join()
        wall = time.perf_counter() - t0
        recs = sch.records()
        sch.destroy()
        for ch in chains:
            ch.plan.destroy()
        busy = sum(r[5] - r[4] for r in recs)
        span = max(r[5] for r in recs) - min(r[4] for r in recs)
        return {"programs_per_s": sum(done) / wall, "device_busy": busy / span,
                "program_ms_device": busy / len(recs), "programs": sum(done)}

    out["scheduler_clients"] = {}
    for c in (1, 2, 4, 8, 16):
        out["scheduler_clients"][c] = closed_loop(c)

    def shares(weights, per_client=240):
        sch = pw.Sched(2)
        chains = [pw.Chain(n, e) for _ in weights]
        states = [x0.clone() for _ in weights]
        for w in weights:
            sch.add_client(w)
        sch.hold(True)
        tickets = [sch.submit_chain(c, chains[c], states[c], d) for c in range(len(weights)) for _ in range(per_client)]
        sch.hold(False)
        for t in tickets:
            sch.wait(t, 60_000_000_000)
        recs = sch.records()
        sch.destroy()
        for ch in chains:
            ch.plan.destroy()
        # the window where every client still had queued programs
        seen = [0] * len(weights)
        end = len(recs)
        for i, r in enumerate(recs):
            seen[r[1]] += 1
            if seen[r[1]] == per_client:
                end = i + 1
                break
        dev = [0.0] * len(weights)
        for r in recs[:end]:
            dev[r[1]] += r[5] - r[4]
        tot = sum(dev)
        return {"weights": list(weights), "device_time_share": [x / tot for x in dev],
                "target_share": [w / sum(weights) for w in weights], "window_programs": end}

    out["shares"] = [shares((1, 1, 1, 1)), shares((1, 2, 4, 8))]
    return out


MFMA_BF16_PEAK_TFLOPS = 2500.0


def small_step_bench(pw, torch, pw_inputs, iters=50, cold_iters=20):
    """The 8-shard step (8 x 4096 tuples x 64 fp32, A = 2x + 1, exchange,
    B = per-tuple sum): 25.6 MB per step, cache-resident and launch-latency
    bound. Timed warm (steps back to back) and cold (a 512 MiB write before
    each step evicts the 256 MB last-level cache), as the default separate
    launches and as one launch in which B waits on the exchange futures inside
    the launch (PW_FLAG_ONE_LAUNCH). With tracing, the one-launch steps where
    some B[d] fired before the last EXCHANGE[d'] are counted."""
    n, t, p = 8, 4096, 64
    inp = pw_inputs.exchange_uniform(n, t, p)
    x = torch.from_numpy(inp.x).cuda()
    dest = torch.from_numpy(inp.dest).cuda()
    st = torch.cuda.current_stream()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    g = n * t

    def timed(flags):
        ex = pw.Exchange(n, t, p, a_op=pw.op(pw.PW_OP_AFFINE, 2.0, 1.0), b_op=pw.op(pw.PW_OP_ROWSUM), flags=flags)
        for _ in range(5):
            f = ex.step(x, dest)
        pw.future_wait(f, 60_000_000_000)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(iters):
            f = ex.step(x, dest)
        e1.record(st)
        torch.cuda.synchronize()
        pw.future_wait(f, 60_000_000_000)
        warm_us = e0.elapsed_time(e1) / iters * 1e3
        cold = []
        for _ in range(cold_iters):
            flush.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            f = ex.step(x, dest)
            b.record(st)
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b) * 1e3)
        pw.future_wait(f, 60_000_000_000)
        cold.sort()
        return {"us_per_step_warm": warm_us, "us_per_step_cold_median": cold[len(cold) // 2],
                "tuples_per_s_warm": g / (warm_us * 1e-6), "gbs_warm_algorithmic": 780 * g / (warm_us * 1e-6) / 1e9}

    out = {"workload": "8 shards x 4096 tuples x 64 fp32 ~U(-1,1), dest uniform, A = 2x+1, B = per-tuple sum",
           "bytes_per_tuple_step": 780, "path": "separate launches (rank with the scan in its last workgroup, scatter, B)"}
    out.update(timed(0))
    out["one_launch"] = timed(pw.PW_FLAG_ONE_LAUNCH)
    tr = pw.Exchange(n, t, p, a_op=pw.op(pw.PW_OP_AFFINE, 2.0, 1.0), b_op=pw.op(pw.PW_OP_ROWSUM),
                     flags=pw.PW_FLAG_TRACE | pw.PW_FLAG_ONE_LAUNCH)
    overlap = 0
    for _ in range(20):
        pw.future_wait(tr.step(x, dest), 60_000_000_000)
        _, _, stamps = tr.plan.read_futures(trace=True)
        xs = stamps[pw.PW_NODE_EXCHANGE, :n].astype("int64")
        bs = stamps[pw.PW_NODE_B, :n].astype("int64")
        overlap += int(bs.min() < xs.max())
    out["one_launch"]["traced_steps_with_b_before_last_exchange"] = f"{overlap} of 20"
    return out


def input_record(np, torch, arrays):
    """numpy / torch versions and the SHA-256 of each generated input array."""
    rec = {"numpy": np.__version__, "torch": torch.__version__}
    for name, a in arrays.items():
        a = np.ascontiguousarray(a)
        rec[name] = {"shape": list(a.shape), "dtype": str(a.dtype),
                     "sha256": hashlib.sha256(memoryview(a).cast("B")).hexdigest()}
    return rec


def pipeline_bench(pw, torch, pw_inputs, passes=3):
    """16-stage GPipe pipeline, 64 microbatches of 2048 x 1024 bf16, each stage a
    1024 x 1024 GEMM + GELU: 4.398 TFLOP per pass, one launch per pass. Timed in
    both claim orders: GPipe lock-step ticks, and stage by stage within windows
    of 16 microbatches (PW_FLAG_STAGE_WINDOWS; same dependencies and results)."""
    s, m, rows, d = 16, 64, 2048, 1024
    inp = pw_inputs.pipeline(s, m, rows, d)
    w = inp.w.cuda()
    x = inp.x.cuda()
    acts = torch.empty((s, m, rows, d), dtype=torch.bfloat16, device="cuda")
    flops = 2.0 * s * m * rows * d * d

    def timed(extra_flags):
        pipe = pw.Pipeline(w, m, rows, flags=pw.PW_FLAG_TIMING | extra_flags)
        pw.future_wait(pipe.run(x, acts), 60_000_000_000)
        pipe.plan.reset_times()
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(passes):
            f = pipe.run(x, acts)
        e1.record(st)
        torch.cuda.synchronize()
        pw.future_wait(f, 60_000_000_000)
        ms = e0.elapsed_time(e1) / passes
        kt = pipe.plan.kernel_times()
        kms = kt["pipeline"][1] / kt["pipeline"][0]
        tf = flops / (kms * 1e-3) / 1e12
        return {"ms_per_pass": ms, "kernel_ms": kms, "tflops": tf, "frac_bf16_peak": tf / MFMA_BF16_PEAK_TFLOPS}

    out = {"workload": "GPipe 16 stages x 64 microbatches of 2048x1024 bf16, stage = 1024x1024 GEMM + GELU",
           "order": "lock-step ticks"}
    out.update(timed(0))
    out["stage_windows"] = timed(pw.PW_FLAG_STAGE_WINDOWS)
    out.update({"flop_per_pass": flops, "gpipe_bubble_lockstep": (s - 1) / (m + s - 1)})
    # the same GEMM + GELU as one stage over the 64 microbatches (no GPipe
    # dependencies): the shape of the vendor reference's pipeline_stage_gemm_gelu
    one = pw.Pipeline(w[:1].contiguous(), m, rows, flags=pw.PW_FLAG_TIMING)
    acts1 = torch.empty((1, m, rows, d), dtype=torch.bfloat16, device="cuda")
    pw.future_wait(one.run(x, acts1), 60_000_000_000)
    one.plan.reset_times()
    for _ in range(5):
        f = one.run(x, acts1)
    pw.future_wait(f, 60_000_000_000)
    kt = one.plan.kernel_times()
    kms = kt["pipeline"][1] / kt["pipeline"][0]
    out["single_stage"] = {"shape": f"{m} x [{rows}x{d}] @ [{d}x{d}] with GELU, one launch", "kernel_ms": kms,
                           "tflops": flops / s / (kms * 1e-3) / 1e12}
    return out


def moe_bench(pw, torch, pw_inputs, steps=3):
    """MoE step: 131072 tokens x 1024 bf16, router 1024 x 64 + top-2, dispatch
    exchange to 64 experts, FFN 1024 -> 4096 -> 1024 GELU, gated combine."""
    tokens, d, experts, hidden = 131072, 1024, 64, 4096
    inp = pw_inputs.moe(tokens, d, experts, hidden)
    wr, w1, w2 = inp.w_router.cuda(), inp.w1.cuda(), inp.w2.cuda()
    x = inp.x.cuda()
    m = pw.MoE(wr, w1, w2, tokens, num_src_shards=64, flags=pw.PW_FLAG_TIMING, want_logits=False)
    pw.future_wait(m.step(x), 60_000_000_000)
    m.plan.reset_times()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(steps):
        f = m.step(x)
    e1.record(st)
    torch.cuda.synchronize()
    pw.future_wait(f, 60_000_000_000)
    ms = e0.elapsed_time(e1) / steps
    kt = {k: v[1] / v[0] for k, v in m.plan.kernel_times().items()}
    ffn_ms = kt["ffn1"] + kt["ffn2"]
    flops = 2.0 * 2 * tokens * (d * hidden + hidden * d)
    tf = flops / (ffn_ms * 1e-3) / 1e12
    return {"workload": "MoE: 131072 tokens x 1024 bf16, 64 experts, top-2, FFN 1024->4096->1024 GELU",
            "ms_per_step": ms, "kernel_ms": kt, "expert_tflops": tf, "expert_frac_bf16_peak": tf / MFMA_BF16_PEAK_TFLOPS,
            "expert_flop": flops}


def moe_capacity_bench(pw, torch, pw_inputs, steps=5):
    """Data-dependent output sizes (PATHWAYS page, section 4.5: a node whose
    resource needs depend on its predecessor falls back to sequential
    scheduling). MoE steps with an expert capacity C (kept: the first C tuples
    of each expert): the static path (one call, buffers of the bound
    min(2T, E C)) against the sequential one (route, the host waits for the
    segment offsets, allocates exactly, then the rest), wall clock per step
    including the wait, at the full workload and at a 16x smaller one where
    the host round trip weighs more."""
    out = []
    for tokens, factor in ((131072, 1.0), (131072, 1.25), (8192, 1.0)):
        d, experts, hidden = 1024, 64, 4096
        cap = int(factor * 2 * tokens / experts)
        inp = pw_inputs.moe(tokens, d, experts, hidden)
        wr, w1, w2 = inp.w_router.cuda(), inp.w1.cuda(), inp.w2.cuda()
        x = inp.x.cuda()
        ms = {}
        rows = None
        for mode in ("static", "sequential"):
            m = pw.MoE(wr, w1, w2, tokens, num_src_shards=64, capacity=cap, want_logits=False,
                       static_buffers=(mode == "static"))
            run = m.step if mode == "static" else m.split_step
            pw.future_wait(run(x), 60_000_000_000)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                f = run(x)
            pw.future_wait(f, 60_000_000_000)
            torch.cuda.synchronize()
            ms[mode] = (time.perf_counter() - t0) / steps * 1e3
            if mode == "sequential":
                rows = int(m.xd.shape[0])
            m.plan.destroy()
        bound = min(2 * tokens, experts * cap)
        out.append({"tokens": tokens, "capacity_factor": factor, "capacity": cap,
                    "ms_per_step_static": ms["static"], "ms_per_step_sequential": ms["sequential"],
                    "rows_static_bound": bound, "rows_routed": rows,
                    "dropped_tuple_share": 1.0 - rows / (2 * tokens)})
    return out


def store_bench(pw, torch, pw_inputs, point_s=1.0, clients=8):
    """Backpressure of the HBM object store (PATHWAYS page, section 4.6).
    Each client thread loops: take its program's state buffer from the store
    (waiting if the store is full), copy its input in, run a chained program
    of ~0.3 ms on it, free the buffer stream-ordered right after the launch,
    wait for the result. The store holds `slots` such buffers; with fewer
    slots than clients, allocations stall instead of failing. Programs/s and
    the store's stall counters per slot count."""
    import threading
    n, e, d = 256, 128, 503
    nbytes = n * e * 4
    x0 = torch.from_numpy(pw_inputs.chain_state(n, e)).cuda()
    out = {"program": f"chained run of {d} steps on {n} shards x {e} fp32; state ({nbytes} B) from the store",
           "clients": clients, "by_slots": {}}
    chains = [pw.Chain(n, e) for _ in range(clients)]
    for slots in (1, 2, 4, 8):
        st = pw.Store(slots * nbytes)
        stop = [False]
        done = [0] * clients
        errors = []

        def client(c):
            try:
                while not stop[0]:
                    obj, ptr = st.alloc(nbytes, owner=c, timeout_ns=10_000_000_000)
                    state = st.tensor(ptr, (n, e))
                    state.copy_(x0)
                    f = chains[c].run(state, d)
                    st.free(obj)
                    pw.future_wait(f, 10_000_000_000)
                    done[c] += 1
            except Exception as ex:  # reported in the result
                errors.append(repr(ex))

        ths = [threading.Thread(target=client, args=(c,)) for c in range(clients)]
        t0 = time.perf_counter()
        for th in ths:
            th.start()
        time.sleep(point_s)
        stop[0] = True
        for th in ths:
            th.join()
        wall = time.perf_counter() - t0
        torch.cuda.synchronize()
        s = st.stats()
        out["by_slots"][slots] = {"programs_per_s": sum(done) / wall, "programs": sum(done), "stalls": s["stalls"],
                                  "stalled_ms_total": s["stalled_ms"], "errors": errors[:3]}
        st.destroy()
    for ch in chains:
        ch.plan.destroy()
    return out


def reference_bench(torch, iters=10):
    """Context, not the product path: the vendor BLAS (hipBLASLt through
    torch.matmul) on the shapes of the two GEMM rows, and torch's elementwise
    copy, on the same device. Inputs random bf16 like the workloads."""
    def gemm(batch, m, k, n, gelu):
        a = torch.randn(batch, m, k, device="cuda").to(torch.bfloat16)
        b = (torch.randn(batch, k, n, device="cuda") * 0.02).to(torch.bfloat16)
        f = (lambda: torch.nn.functional.gelu(torch.matmul(a, b))) if gelu else (lambda: torch.matmul(a, b))
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        return {"shape": f"{batch} x [{m}x{k}] @ [{k}x{n}]" + (" then GELU" if gelu else ""), "ms": ms,
                "tflops": 2.0 * batch * m * n * k / (ms * 1e-3) / 1e12}
    out = {"note": "vendor BLAS via torch on the same device, for context only",
           "pipeline_stage_gemm_gelu": gemm(64, 2048, 1024, 1024, True),
           "pipeline_stage_gemm": gemm(64, 2048, 1024, 1024, False),
           "ffn2_like_gemm": gemm(64, 4096, 4096, 1024, False),
           # the measured dense-GEMM rate beside the published 2.5 PFLOP/s
           "square_8192_gemm": gemm(1, 8192, 8192, 8192, False)}
    x = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        torch.neg(x, out=y)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    out["copy_gbs"] = 2.0 * x.numel() * 4 / (ms * 1e-3) / 1e9
    return out


def cpu_other_rows(pw_inputs, pipeline=True, moe=True):
    """The oracle on bounded samples of the other rows, scaled to the full
    workload (reported beside the GPU numbers, never a target)."""
    import numpy as np
    from oracle import chain as oc
    from oracle import exchange as ox
    out = {}
    small = pw_inputs.exchange_uniform(8, 4096, 64)
    reps = 20
    t0 = time.perf_counter()
    for _ in range(reps):
        ox.exchange_step(small.x, small.dest, 8, 8, a_op=ox.op_affine(2.0, 1.0), b_op=ox.op_rowsum())
    dt = (time.perf_counter() - t0) / reps
    out["small_step"] = {"value": 8 * 4096 / dt, "unit": "tuples/s", "cores": 1,
                         "sample": f"the whole 8 x 4096 x 64 step with A = 2x+1 and B = row sum "
                                   f"(oracle.exchange.exchange_step, NumPy), mean of {reps}: {dt * 1e3:.2f} ms"}
    x0 = pw_inputs.chain_state(2048, 128)
    steps = 1000
    t0 = time.perf_counter()
    oc.chain(x0, steps)
    dt = time.perf_counter() - t0
    out["chain"] = {"value": steps / dt, "unit": "steps/s", "cores": 1,
                    "sample": f"N=2048 shards x 128 fp32, {steps} of the 10,000 steps (oracle.chain.chain, NumPy)"}
    if pipeline:
        from oracle import pipeline as op
        inp = pw_inputs.pipeline(16, 1, 2048, 1024)
        x = inp.x[0].float().numpy()
        w = inp.w.float().numpy()
        t0 = time.perf_counter()
        op.forward(x, w)
        dt = time.perf_counter() - t0
        out["pipeline"] = {"value": dt * 64 * 1e3, "unit": "ms per pass (estimated)", "cores": _blas_threads(),
                           "sample": f"1 of 64 microbatches through all 16 stages (oracle.pipeline.forward, NumPy fp64 GEMMs) "
                                     f"in {dt:.2f} s, times 64"}
    if moe:
        from oracle import moe as om
        tokens = 2048
        inp = pw_inputs.moe(tokens, 1024, 64, 4096)
        t0 = time.perf_counter()
        om.moe_step(inp.x.float().numpy(), inp.w_router.float().numpy(), inp.w1.float().numpy(),
                    inp.w2.float().numpy())
        dt = time.perf_counter() - t0
        out["moe"] = {"value": dt * (131072 / tokens) * 1e3, "unit": "ms per step (estimated)", "cores": _blas_threads(),
                      "sample": f"{tokens} of 131072 tokens through oracle.moe.moe_step (NumPy fp64 GEMMs) in {dt:.2f} s, "
                                f"scaled by token count"}
    return out


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-chain", action="store_true", help="skip the chained-steps sweep")
    ap.add_argument("--no-pipeline", action="store_true", help="skip the pipeline measurement")
    ap.add_argument("--no-moe", action="store_true", help="skip the mixture-of-experts measurement")
    ap.add_argument("--chain-steps", type=int, default=10000)
    ap.add_argument("--no-reference", action="store_true", help="skip the vendor-BLAS and copy reference timings")
    ap.add_argument("--no-cpu-extra", action="store_true", help="skip the oracle samples of the chain and pipeline rows")
    ap.add_argument("--cpu-moe", action="store_true", help="also time the oracle on a 2048-token MoE sample (~45 s)")
    ap.add_argument("--dispatch-study", action="store_true",
                    help="also measure per-node cost against program length for the four dispatch modes")
    ap.add_argument("--moe-capacity", action="store_true",
                    help="MoE with an expert capacity: one static call vs route, host wait, exact allocation, rest")
    ap.add_argument("--store", action="store_true", help="object-store backpressure: client programs vs store slots")
    ap.add_argument("--multi-tenant", action="store_true",
                    help="throughput of concurrent clients and proportional shares through the scheduler")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 3 plain elementwise copies of 1 GiB (torch.neg) to scale HBM counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library runs every shard on a single MI355X "
              "(no inter-GPU path is built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import pw_inputs
    import sparse_shard_exchange_amd as pw

    n, t, p = 256, 65536, 64
    log("generating inputs")
    inp = pw_inputs.exchange_zipf(n, t, p)
    g = n * t
    x = torch.from_numpy(inp.x).cuda()
    dest = torch.from_numpy(inp.dest).cuda()
    counts = np.bincount(inp.dest, minlength=n)
    # Two plans of the same step: `ex` runs the timed steps behind `value`;
    # `ex_k` records HIP events around every kernel (PW_FLAG_TIMING) for the
    # per-kernel durations and the roofline, in a second timed region of the
    # same length (the events cost ~25 us per step, so they stay out of the
    # first).
    ex = pw.Exchange(n, t, p)
    ex_k = pw.Exchange(n, t, p, flags=pw.PW_FLAG_TIMING)
    torch.cuda.synchronize()

    log("warmup")
    for plan in (ex, ex_k):
        for _ in range(args.warmup):
            f = plan.step(x, dest)
        pw.future_wait(f, 60_000_000_000)
    ex_k.plan.reset_times()
    torch.cuda.synchronize()

    log("timed steps")
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    e0.record(stream)
    t0 = time.perf_counter()
    marks[0].record(stream)
    for i in range(args.steps):
        f = ex.step(x, dest)
        marks[i + 1].record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    pw.future_wait(f, 60_000_000_000)
    ms_events = e0.elapsed_time(e1) / args.steps
    ms_wall = (t1 - t0) * 1e3 / args.steps
    ms = max(ms_events, ms_wall)
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    pct = lambda q: per_step[min(len(per_step) - 1, int(q * (len(per_step) - 1) + 0.5))]

    log("timed steps with kernel events")
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for _ in range(args.steps):
        f = ex_k.step(x, dest)
    k1.record(stream)
    torch.cuda.synchronize()
    pw.future_wait(f, 60_000_000_000)
    ms_with_events = k0.elapsed_time(k1) / args.steps
    kt = ex_k.plan.kernel_times()
    per_kernel = {k: v[1] / max(v[0], 1) for k, v in kt.items()}
    scat_ms = per_kernel["scatter"]
    achieved = BYTES_PER_TUPLE * g / (scat_ms * 1e-3) / 1e9
    traffic = traffic_for(os.path.join(ROOT, "sparse_shard_exchange_amd", "csrc", "exchange.hip"), "scatter", g)

    result = {
        "metric": METRIC,
        "value": g / (ms * 1e-3),
        "unit": "tuples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "zipf exchange: N=256 shards x T=65536 tuples, 64 fp32 payload ~N(0,1), "
                        "k=4 destinations per source drawn Zipf(1.1), A=B=identity",
            "tuples": g,
            "algorithmic_bytes_per_tuple": BYTES_PER_TUPLE,
            "hottest_destination_share": float(counts.max() / g),
            "empty_destinations": int((counts == 0).sum()),
        },
        "ms_per_step_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
        "step_gbs_algorithmic": BYTES_PER_TUPLE * g / (ms * 1e-3) / 1e9,
        "step_frac_hbm_peak": BYTES_PER_TUPLE * g / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "kernel_ms": per_kernel,
        "ms_per_step_with_kernel_events": ms_with_events,
        "roofline": {
            "kernel": "scatter",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
        },
    }

    del ex, ex_k, x, dest
    torch.cuda.empty_cache()
    result["inputs"] = input_record(np, torch, {"x": inp.x, "dest": inp.dest})
    log("small step")
    result["small_step"] = small_step_bench(pw, torch, pw_inputs)
    if not args.no_pipeline:
        log("pipeline")
        result["pipeline"] = pipeline_bench(pw, torch, pw_inputs)

    if not args.no_moe:
        log("moe")
        result["moe"] = moe_bench(pw, torch, pw_inputs)

    if args.moe_capacity:
        log("moe capacity: static vs sequential")
        result["moe_capacity"] = moe_capacity_bench(pw, torch, pw_inputs)

    if not args.no_chain:
        log("chain sweep")
        result["chain"] = chain_sweep(pw, torch, pw_inputs, args.chain_steps)

    if args.dispatch_study:
        log("dispatch study")
        result["dispatch_study"] = dispatch_study(pw, torch, pw_inputs)

    if args.store:
        log("object store backpressure")
        result["store"] = store_bench(pw, torch, pw_inputs)

    if args.multi_tenant:
        log("multi-tenant scheduler")
        result["multi_tenant"] = multi_tenant(pw, torch, pw_inputs)

    if not args.no_reference:
        log("reference (vendor BLAS, copy)")
        result["reference"] = reference_bench(torch)

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        result["copy_calibration"] = {"kernel": "torch.neg", "bytes_read": a.numel() * 4, "bytes_written": b.numel() * 4}
        del a, b

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        from oracle import exchange as ox
        xs, ds = inp.x, inp.dest
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            ox.exchange_step(xs, ds, n, n)
            times.append(time.perf_counter() - t0)
        dt = sorted(times)[1]
        result["cpu_baseline"] = {
            "value": g / dt, "unit": "tuples/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole workload ({g} tuples, {n} sources) through oracle.exchange.exchange_step, "
                      f"median of 3 runs {dt:.2f} s, single-threaded NumPy",
            **cpu_info(),
        }
        if not args.no_cpu_extra:
            log("cpu baseline, other rows (oracle samples)")
            result["cpu_baseline_other_rows"] = cpu_other_rows(pw_inputs, not args.no_pipeline, args.cpu_moe)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
