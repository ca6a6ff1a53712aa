"""Python binding of libpw.so, the C ABI of the sharded-dataflow hot path.

Argument marshalling only: every step of the path runs in the library's HIP
kernels. PyTorch supplies device memory (tensors, the plan workspace) and the
stream (``torch.cuda.current_stream()``). The names mirror ``include/pw.h``.

Importing this package loads ``libpw.so`` from this directory and fails
loudly if it is missing: there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes as C
import os

# torch first: libpw.so links libamdhip64.so.7, and torch ships its own copy
# of that runtime under the same soname. Loaded after torch, our dependency
# resolves to torch's copy; loaded before, the process would end up with two
# HIP runtimes, and ours would find no device once torch's had claimed it.
import torch  # noqa: F401  (load order only)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpw.so")

# ---- constants (include/pw.h) ------------------------------------------------
PW_ABI_VERSION = 1
PW_OK, PW_ERR_INVALID, PW_ERR_NOMEM, PW_ERR_DEVICE = 0, -1, -2, -3
PW_ERR_TIMEOUT, PW_ERR_BAD_DEST, PW_ERR_STATE, PW_ERR_UNSUPPORTED = -4, -5, -6, -7
PW_F32, PW_BF16 = 0, 1
PW_GRAPH_EXCHANGE, PW_GRAPH_CHAIN, PW_GRAPH_MOE, PW_GRAPH_PIPELINE = 0, 1, 2, 3
PW_OP_IDENTITY, PW_OP_AFFINE, PW_OP_ROWSUM = 0, 1, 2
PW_CHAIN_CHAINED, PW_CHAIN_OPBYOP, PW_CHAIN_FUSED, PW_CHAIN_SPLIT = 0, 1, 2, 3
PW_FLAG_TRACE, PW_FLAG_TIMING, PW_FLAG_STAGE_WINDOWS, PW_FLAG_ONE_LAUNCH = 0x1, 0x2, 0x4, 0x8
PW_NODE_ARG, PW_NODE_A, PW_NODE_EXCHANGE, PW_NODE_B, PW_NODE_RESULT, PW_NODE_STAGE = 0, 1, 2, 3, 4, 5


class pw_op(C.Structure):
    _fields_ = [("kind", C.c_uint32), ("a", C.c_float), ("b", C.c_float)]


class pw_plan_desc(C.Structure):
    _fields_ = [
        ("abi_version", C.c_uint32), ("kind", C.c_uint32), ("num_shards", C.c_uint32),
        ("num_src_shards", C.c_uint32), ("tuples_per_shard", C.c_uint64), ("payload_elems", C.c_uint32),
        ("dtype", C.c_uint32), ("a_op", pw_op), ("b_op", pw_op), ("top_k", C.c_uint32),
        ("hidden", C.c_uint32), ("microbatches", C.c_uint32), ("chain_mode", C.c_uint32),
        ("flags", C.c_uint32), ("capacity", C.c_uint32), ("spin_limit_ns", C.c_uint64),
        ("w_router", C.c_void_p), ("w1", C.c_void_p), ("w2", C.c_void_p),
    ]


class pw_sharded_buf(C.Structure):
    _fields_ = [
        ("base", C.c_void_p), ("num_tuples", C.c_uint64), ("num_shards", C.c_uint32),
        ("elems_per_tuple", C.c_uint32), ("dtype", C.c_uint32), ("reserved0", C.c_uint32),
        ("shard_offsets", C.c_void_p),
    ]


class pw_future_t(C.Structure):
    _fields_ = [("plan_id", C.c_uint64), ("node", C.c_uint32), ("shard", C.c_int32), ("epoch", C.c_uint64)]

    def __repr__(self):
        return f"pw_future_t(plan={self.plan_id}, node={self.node}, shard={self.shard}, epoch={self.epoch})"


class pw_exchange_io(C.Structure):
    _fields_ = [
        ("src", pw_sharded_buf), ("dest", C.c_void_p), ("dst", pw_sharded_buf), ("src_index", C.c_void_p),
        ("counts", C.c_void_p), ("b_out", C.c_void_p), ("result", C.c_void_p), ("logits", C.c_void_p),
        ("experts", C.c_void_p), ("gates", C.c_void_p),
    ]


class pw_kernel_time(C.Structure):
    _fields_ = [("name", C.c_char * 32), ("launches", C.c_uint64), ("total_ms", C.c_double)]


PW_PROG_CHAIN, PW_PROG_EXCHANGE = 0, 1


class pw_store_stats(C.Structure):
    _fields_ = [
        ("base", C.c_uint64), ("capacity", C.c_uint64), ("in_use", C.c_uint64), ("pending_free", C.c_uint64),
        ("largest_free", C.c_uint64), ("objects", C.c_uint64), ("waiting", C.c_uint64), ("stalls", C.c_uint64),
        ("stalled_ms", C.c_double),
    ]


class pw_program(C.Structure):
    _fields_ = [
        ("kind", C.c_uint32), ("cost", C.c_uint32), ("plan", C.c_void_p), ("steps", C.c_uint64),
        ("state", pw_sharded_buf), ("aux", C.c_void_p), ("io", pw_exchange_io),
    ]


class pw_sched_record(C.Structure):
    _fields_ = [
        ("ticket", C.c_uint64), ("client", C.c_uint32), ("status", C.c_int32), ("dispatch", C.c_uint64),
        ("start_ms", C.c_double), ("end_ms", C.c_double),
    ]


# Every function the header declares, with its C signature.
_SIGNATURES = {
    "pw_abi_version": (C.c_uint32, []),
    "pw_strerror": (C.c_char_p, [C.c_int]),
    "pw_last_error": (C.c_char_p, []),
    "pw_plan": (C.c_int, [C.POINTER(pw_plan_desc), C.c_void_p, C.c_size_t, C.POINTER(C.c_size_t), C.POINTER(C.c_void_p)]),
    "pw_plan_destroy": (C.c_int, [C.c_void_p]),
    "pw_exchange": (C.c_int, [C.c_void_p, C.POINTER(pw_exchange_io), C.c_void_p, C.POINTER(pw_future_t)]),
    "pw_exchange_begin": (C.c_int, [C.c_void_p, C.POINTER(pw_exchange_io), C.c_void_p, C.c_void_p]),
    "pw_exchange_end": (C.c_int, [C.c_void_p, C.POINTER(pw_exchange_io), C.c_void_p, C.POINTER(pw_future_t)]),
    "pw_exchange_scratch": (C.c_int, [C.POINTER(pw_plan_desc), C.POINTER(pw_exchange_io), C.c_void_p]),
    "pw_chain_run": (C.c_int, [C.c_void_p, C.c_uint64, C.POINTER(pw_sharded_buf), C.c_void_p, C.c_void_p,
                               C.POINTER(pw_future_t)]),
    "pw_future_wait": (C.c_int, [pw_future_t, C.c_int64]),
    "pw_future_query": (C.c_int, [pw_future_t, C.POINTER(C.c_int)]),
    "pw_plan_read_futures": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                       C.POINTER(C.c_uint32), C.POINTER(C.c_uint32)]),
    "pw_plan_chain_placement": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t]),
    "pw_plan_kernel_times": (C.c_int, [C.c_void_p, C.POINTER(pw_kernel_time), C.c_int, C.POINTER(C.c_int)]),
    "pw_plan_reset_times": (C.c_int, [C.c_void_p]),
    "pw_sched_create": (C.c_int, [C.c_uint32, C.POINTER(C.c_void_p)]),
    "pw_sched_add_client": (C.c_int, [C.c_void_p, C.c_uint32, C.POINTER(C.c_uint32)]),
    "pw_sched_submit": (C.c_int, [C.c_void_p, C.c_uint32, C.POINTER(pw_program), C.POINTER(C.c_uint64)]),
    "pw_sched_wait": (C.c_int, [C.c_void_p, C.c_uint64, C.c_int64]),
    "pw_sched_hold": (C.c_int, [C.c_void_p, C.c_int]),
    "pw_sched_records": (C.c_int, [C.c_void_p, C.POINTER(pw_sched_record), C.c_size_t, C.POINTER(C.c_size_t)]),
    "pw_sched_destroy": (C.c_int, [C.c_void_p]),
    "pw_store_create": (C.c_int, [C.c_size_t, C.POINTER(C.c_void_p)]),
    "pw_store_alloc": (C.c_int, [C.c_void_p, C.c_size_t, C.c_uint32, C.c_int64, C.POINTER(C.c_uint64),
                                 C.POINTER(C.c_void_p)]),
    "pw_store_free": (C.c_int, [C.c_void_p, C.c_uint64, C.c_void_p]),
    "pw_store_release_owner": (C.c_int, [C.c_void_p, C.c_uint32, C.c_void_p, C.POINTER(C.c_uint64)]),
    "pw_store_get_stats": (C.c_int, [C.c_void_p, C.POINTER(pw_store_stats)]),
    "pw_store_destroy": (C.c_int, [C.c_void_p]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_shard_exchange_amd.build` "
                          "(the HIP library is the only implementation; there is no fallback)")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.pw_abi_version() != PW_ABI_VERSION:
        raise ImportError(f"libpw ABI {lib.pw_abi_version()} != {PW_ABI_VERSION}")
    return lib


lib = _load()


class PwError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{lib.pw_strerror(code).decode()} ({code}): {msg}")
        self.code = code


def check(rc: int) -> int:
    if rc != PW_OK:
        raise PwError(rc, lib.pw_last_error().decode())
    return rc


def op(kind=PW_OP_IDENTITY, a=0.0, b=0.0) -> pw_op:
    return pw_op(kind, a, b)


def desc(kind, num_shards, tuples_per_shard, payload_elems=0, dtype=PW_F32, num_src_shards=0,
         a_op=None, b_op=None, top_k=0, hidden=0, microbatches=0, chain_mode=PW_CHAIN_CHAINED,
         flags=0, spin_limit_ns=0, w_router=None, w1=None, w2=None, capacity=0) -> pw_plan_desc:
    d = pw_plan_desc()
    d.abi_version = PW_ABI_VERSION
    d.kind = kind
    d.num_shards = num_shards
    d.num_src_shards = num_src_shards
    d.tuples_per_shard = tuples_per_shard
    d.payload_elems = payload_elems
    d.dtype = dtype
    d.a_op = a_op or op()
    d.b_op = b_op or op()
    d.top_k = top_k
    d.hidden = hidden
    d.microbatches = microbatches
    d.chain_mode = chain_mode
    d.flags = flags
    d.capacity = capacity
    d.spin_limit_ns = spin_limit_ns
    d.w_router = _ptr(w_router)
    d.w1 = _ptr(w1)
    d.w2 = _ptr(w2)
    return d


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def workspace_size(d: pw_plan_desc) -> int:
    """Host-only sizing call (no HIP)."""
    need = C.c_size_t(0)
    check(lib.pw_plan(C.byref(d), None, 0, C.byref(need), None))
    return need.value


def sharded(t, num_shards, elems_per_tuple, dtype, shard_offsets=None) -> pw_sharded_buf:
    b = pw_sharded_buf()
    b.base = _ptr(t)
    b.num_tuples = (t.numel() // elems_per_tuple) if (t is not None and elems_per_tuple) else 0
    b.num_shards = num_shards
    b.elems_per_tuple = elems_per_tuple
    b.dtype = dtype
    b.shard_offsets = _ptr(shard_offsets)
    return b


class Plan:
    """A built plan: the opaque handle plus the torch-allocated workspace it lives in."""

    def __init__(self, d: pw_plan_desc, device="cuda"):
        import torch
        self.desc = d
        self.ws_bytes = workspace_size(d)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        h = C.c_void_p()
        need = C.c_size_t(0)
        check(lib.pw_plan(C.byref(d), C.c_void_p(self.ws.data_ptr()), self.ws.numel(), C.byref(need), C.byref(h)))
        self.handle = h

    def destroy(self):
        if self.handle:
            check(lib.pw_plan_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                lib.pw_plan_destroy(self.handle)
        except Exception:
            pass

    def exchange(self, io: pw_exchange_io, stream=None) -> pw_future_t:
        f = pw_future_t()
        check(lib.pw_exchange(self.handle, C.byref(io), _stream(stream), C.byref(f)))
        return f

    def exchange_begin(self, io: pw_exchange_io, num_dest: int, stream=None):
        """First half of a split step; blocks, returns the segment offsets
        (numpy int64 [num_dest + 1])."""
        import numpy as np
        offs = np.zeros(num_dest + 1, dtype=np.int64)
        check(lib.pw_exchange_begin(self.handle, C.byref(io), _stream(stream), C.c_void_p(offs.ctypes.data)))
        return offs

    def exchange_end(self, io: pw_exchange_io, stream=None) -> pw_future_t:
        f = pw_future_t()
        check(lib.pw_exchange_end(self.handle, C.byref(io), _stream(stream), C.byref(f)))
        return f

    def chain_run(self, steps: int, state: pw_sharded_buf, aux=None, stream=None) -> pw_future_t:
        f = pw_future_t()
        check(lib.pw_chain_run(self.handle, steps, C.byref(state), _ptr(aux), _stream(stream), C.byref(f)))
        return f

    def read_futures(self, trace=False):
        """(epochs, fires, stamps) as numpy arrays [nodes, width]."""
        import numpy as np
        nodes, width = C.c_uint32(0), C.c_uint32(0)
        check(lib.pw_plan_read_futures(self.handle, None, None, None, 0, C.byref(nodes), C.byref(width)))
        n = nodes.value * width.value
        ep = np.zeros(n, np.uint32)
        fi = np.zeros(n, np.uint32)
        st = np.zeros(n, np.uint64) if trace else None
        check(lib.pw_plan_read_futures(self.handle, ep.ctypes.data, fi.ctypes.data,
                                       st.ctypes.data if trace else None, n, C.byref(nodes), C.byref(width)))
        shape = (nodes.value, width.value)
        return ep.reshape(shape), fi.reshape(shape), (st.reshape(shape) if trace else None)

    def kernel_times(self) -> dict:
        n = C.c_int(0)
        check(lib.pw_plan_kernel_times(self.handle, None, 0, C.byref(n)))
        arr = (pw_kernel_time * max(n.value, 1))()
        check(lib.pw_plan_kernel_times(self.handle, arr, n.value, C.byref(n)))
        return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n.value)}

    def reset_times(self):
        check(lib.pw_plan_reset_times(self.handle))


def exchange_scratch(d: pw_plan_desc, io: pw_exchange_io, stream=None) -> None:
    """One EXCHANGE step with the library's static scratch tables (no plan,
    no workspace, nothing allocated); stream ordered, no future."""
    check(lib.pw_exchange_scratch(C.byref(d), C.byref(io), _stream(stream)))


def future_wait(f: pw_future_t, timeout_ns: int = -1) -> None:
    check(lib.pw_future_wait(f, timeout_ns))


def future_query(f: pw_future_t) -> bool:
    fired = C.c_int(0)
    check(lib.pw_future_query(f, C.byref(fired)))
    return bool(fired.value)


def exchange_io(src, dest, dst, num_src, num_dest, elems, dtype=PW_F32, src_index=None, counts=None,
                offsets=None, b_out=None, result=None, logits=None, experts=None, gates=None) -> pw_exchange_io:
    io = pw_exchange_io()
    io.src = sharded(src, num_src, elems, dtype)
    io.dest = _ptr(dest)
    io.dst = sharded(dst, num_dest, elems, dtype, offsets)
    io.src_index = _ptr(src_index)
    io.counts = _ptr(counts)
    io.b_out = _ptr(b_out)
    io.result = _ptr(result)
    io.logits = _ptr(logits)
    io.experts = _ptr(experts)
    io.gates = _ptr(gates)
    return io


class Exchange:
    """One EXCHANGE plan with its output buffers, for repeated steps on
    inputs of one shape. Allocation happens here, once; ``step`` only
    enqueues the library's kernels."""

    def __init__(self, num_shards, tuples_per_shard, payload_elems, dtype=PW_F32, num_src_shards=0,
                 a_op=None, b_op=None, flags=0, spin_limit_ns=0, want_index=True, want_counts=False,
                 device="cuda"):
        import torch
        self.N = num_shards
        self.S = num_src_shards or num_shards
        self.P = payload_elems
        self.dtype = dtype
        self.G = self.S * tuples_per_shard
        self.desc = desc(PW_GRAPH_EXCHANGE, num_shards, tuples_per_shard, payload_elems, dtype, num_src_shards,
                         a_op=a_op, b_op=b_op, flags=flags, spin_limit_ns=spin_limit_ns)
        self.plan = Plan(self.desc, device)
        tdt = torch.float32 if dtype == PW_F32 else torch.bfloat16
        self.dst = torch.empty((self.G, payload_elems), dtype=tdt, device=device)
        self.offsets = torch.empty(self.N + 1, dtype=torch.int64, device=device)
        self.src_index = torch.empty(self.G, dtype=torch.int32, device=device) if want_index else None
        self.counts = torch.empty((self.S, self.N), dtype=torch.int32, device=device) if want_counts else None
        bk = self.desc.b_op.kind
        if bk == PW_OP_ROWSUM:
            self.b_out = torch.empty(self.G, dtype=torch.float32, device=device)
        elif bk == PW_OP_AFFINE:
            self.b_out = torch.empty((self.G, payload_elems), dtype=torch.float32, device=device)
        else:
            self.b_out = None

    def io(self, x, dest) -> pw_exchange_io:
        return exchange_io(x, dest, self.dst, self.S, self.N, self.P, self.dtype, src_index=self.src_index,
                           counts=self.counts, offsets=self.offsets, b_out=self.b_out)

    def step(self, x, dest, stream=None) -> pw_future_t:
        return self.plan.exchange(self.io(x, dest), stream)


class Chain:
    """One CHAIN plan: N shards of E fp32, A and B elementwise, run in
    Chained, OpByOp or Fused mode."""

    def __init__(self, num_shards, elems, a_op=None, b_op=None, mode=PW_CHAIN_CHAINED, flags=0,
                 spin_limit_ns=0, device="cuda"):
        self.N, self.E = num_shards, elems
        self.desc = desc(PW_GRAPH_CHAIN, num_shards, elems, 0, PW_F32,
                         a_op=a_op or op(PW_OP_AFFINE, 1.0, 1.0), b_op=b_op or op(PW_OP_AFFINE, 0.5, 0.0),
                         chain_mode=mode, flags=flags, spin_limit_ns=spin_limit_ns)
        self.plan = Plan(self.desc, device)

    def run(self, state, steps, aux=None, stream=None) -> pw_future_t:
        return self.plan.chain_run(steps, sharded(state, self.N, self.E, PW_F32), aux, stream)

    def placement(self):
        """PW_CHAIN_SPLIT plans: numpy [N, 2] XCD of the waves that ran A[i], B[i]
        in the last call."""
        import numpy as np
        out = np.zeros(2 * self.N, np.uint32)
        check(lib.pw_plan_chain_placement(self.plan.handle, out.ctypes.data, out.size))
        return out.reshape(self.N, 2)


class Pipeline:
    """One PIPELINE plan: S stages of h = bf16(GELU(h . W_s)) over M microbatches
    of rows x d bf16, GPipe fill/drain, one launch per pass. W is [S][d][d]
    bf16, stored [in][out] (borrowed: keep it alive while the plan lives)."""

    def __init__(self, w, microbatches, rows, flags=0, spin_limit_ns=0, device="cuda"):
        import torch
        assert w.dtype == torch.bfloat16 and w.dim() == 3 and w.shape[1] == w.shape[2]
        self.w = w
        self.S, self.d = w.shape[0], w.shape[1]
        self.M, self.R = microbatches, rows
        self.desc = desc(PW_GRAPH_PIPELINE, self.S, rows, self.d, PW_BF16, microbatches=microbatches,
                         flags=flags, spin_limit_ns=spin_limit_ns, w1=w)
        self.plan = Plan(self.desc, device)

    def run(self, x, acts, stream=None) -> pw_future_t:
        """x: [M][rows][d] bf16; acts: [S][M][rows][d] bf16 receives every stage output."""
        return self.plan.chain_run(1, sharded(x, self.M, self.d, PW_BF16), acts, stream)


class MoE:
    """One MOE plan: router d x E + top-2 softmax gate, dispatch exchange to E
    expert shards, expert FFN d -> hidden -> d with GELU, gated combine.
    Weights (bf16, stored [in][out]) are borrowed: keep them alive."""

    def __init__(self, w_router, w1, w2, tokens, num_src_shards=64, flags=0, spin_limit_ns=0,
                 want_logits=True, want_counts=False, capacity=0, static_buffers=True, device="cuda"):
        import torch
        self.d, self.E = w_router.shape
        self.hidden = w1.shape[2]
        assert tokens % num_src_shards == 0
        self.T, self.S = tokens, num_src_shards
        self.w = (w_router, w1, w2)
        self.capacity = capacity
        self.device = device
        self.desc = desc(PW_GRAPH_MOE, self.E, tokens // num_src_shards, self.d, PW_BF16,
                         num_src_shards=num_src_shards, top_k=2, hidden=self.hidden, flags=flags,
                         spin_limit_ns=spin_limit_ns, w_router=w_router, w1=w1, w2=w2, capacity=capacity)
        self.plan = Plan(self.desc, device)
        bf = torch.bfloat16
        # dispatched rows at most: every tuple, or E * capacity if fewer
        self.static_rows = min(2 * tokens, self.E * capacity) if capacity else 2 * tokens
        rows = self.static_rows if static_buffers else 0  # split_step allocates them per step
        self.xd = torch.empty((rows, self.d), dtype=bf, device=device)
        self.y = torch.empty((rows, self.d), dtype=bf, device=device)
        self.out = torch.empty((tokens, self.d), dtype=bf, device=device)
        self.offsets = torch.empty(self.E + 1, dtype=torch.int64, device=device)
        self.src_index = torch.empty(2 * tokens, dtype=torch.int32, device=device)
        self.experts = torch.empty((tokens, 2), dtype=torch.int32, device=device)
        self.gates = torch.empty((tokens, 2), dtype=torch.float32, device=device)
        self.logits = torch.empty((tokens, self.E), dtype=torch.float32, device=device) if want_logits else None
        self.counts = torch.empty((num_src_shards, self.E), dtype=torch.int32, device=device) if want_counts else None

    def _io(self, x) -> pw_exchange_io:
        io = pw_exchange_io()
        io.src = sharded(x, self.S, self.d, PW_BF16)
        io.dest = None
        io.dst = sharded(self.xd, self.E, self.d, PW_BF16, self.offsets)
        io.src_index = _ptr(self.src_index)
        io.counts = _ptr(self.counts)
        io.b_out = _ptr(self.y)
        io.result = _ptr(self.out)
        io.logits = _ptr(self.logits)
        io.experts = _ptr(self.experts)
        io.gates = _ptr(self.gates)
        return io

    def step(self, x, stream=None) -> pw_future_t:
        """One step with buffers of the static bound (one call)."""
        return self.plan.exchange(self._io(x), stream)

    def split_step(self, x, stream=None) -> pw_future_t:
        """One step in two calls: route (the host waits for the segment
        offsets), allocate the dispatched rows and expert outputs at exactly
        the routed size, then run the rest."""
        import torch
        io = self._io(x)
        offs = self.plan.exchange_begin(io, self.E, stream)
        rows = int(offs[-1])
        self.xd = torch.empty((rows, self.d), dtype=torch.bfloat16, device=self.device)
        self.y = torch.empty((rows, self.d), dtype=torch.bfloat16, device=self.device)
        io.dst = sharded(self.xd, self.E, self.d, PW_BF16, self.offsets)
        io.dst.num_tuples = rows
        io.b_out = _ptr(self.y)
        return self.plan.exchange_end(io, stream)


class Sched:
    """Multi-tenant scheduler: clients with weights submit programs (chain
    runs, exchange steps) that run one after another on the scheduler's own
    stream in proportional shares. Tensors handed to a program are kept
    referenced here until its ticket is waited."""

    def __init__(self, max_inflight=2):
        h = C.c_void_p()
        check(lib.pw_sched_create(max_inflight, C.byref(h)))
        self.handle = h
        self._keep = {}

    def add_client(self, weight=1) -> int:
        c = C.c_uint32(0)
        check(lib.pw_sched_add_client(self.handle, weight, C.byref(c)))
        return c.value

    def _submit(self, client, prog, keep) -> int:
        t = C.c_uint64(0)
        check(lib.pw_sched_submit(self.handle, client, C.byref(prog), C.byref(t)))
        self._keep[t.value] = keep
        return t.value

    def submit_chain(self, client, chain, state, steps, cost=None, aux=None) -> int:
        """A chain run of `steps` steps of `chain` (a Chain) over `state`;
        cost defaults to the step count."""
        prog = pw_program()
        prog.kind = PW_PROG_CHAIN
        prog.cost = steps if cost is None else cost
        prog.plan = chain.plan.handle.value
        prog.steps = steps
        prog.state = sharded(state, chain.N, chain.E, PW_F32)
        prog.aux = _ptr(aux)
        return self._submit(client, prog, (chain, state, aux))

    def submit_exchange(self, client, ex, x, dest, cost=1) -> int:
        """One step of `ex` (an Exchange) on x, dest."""
        prog = pw_program()
        prog.kind = PW_PROG_EXCHANGE
        prog.cost = cost
        prog.plan = ex.plan.handle.value
        prog.io = ex.io(x, dest)
        return self._submit(client, prog, (ex, x, dest))

    def wait(self, ticket, timeout_ns=-1) -> None:
        rc = lib.pw_sched_wait(self.handle, ticket, timeout_ns)
        if rc != PW_ERR_TIMEOUT:  # the ticket is consumed; on a timeout it stays waitable
            self._keep.pop(ticket, None)
        check(rc)

    def hold(self, on=True) -> None:
        check(lib.pw_sched_hold(self.handle, 1 if on else 0))

    def records(self, capacity=1 << 16) -> list:
        """Records of finished programs in dispatch order (each read once):
        (ticket, client, status, dispatch, start_ms, end_ms) tuples."""
        out = []
        buf = (pw_sched_record * capacity)()
        while True:
            n = C.c_size_t(0)
            check(lib.pw_sched_records(self.handle, buf, capacity, C.byref(n)))
            out += [(r.ticket, r.client, r.status, r.dispatch, r.start_ms, r.end_ms) for r in buf[:n.value]]
            if n.value < capacity:
                return out

    def destroy(self) -> None:
        if self.handle:
            check(lib.pw_sched_destroy(self.handle))
            self.handle = None
            self._keep.clear()

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                lib.pw_sched_destroy(self.handle)
        except Exception:
            pass


class _DeviceArray:
    """A borrowed view of device memory for torch.as_tensor (array interface
    of version 2); the memory stays the store's."""

    def __init__(self, ptr, shape, typestr):
        self.__cuda_array_interface__ = {"shape": tuple(shape), "typestr": typestr, "data": (ptr, False),
                                         "version": 2, "strides": None}


class Store:
    """HBM object store: owner-labelled device buffers with backpressure."""

    _TYPESTR = {"float32": "<f4", "int32": "<i4", "int64": "<i8", "uint8": "|u1"}

    def __init__(self, nbytes):
        h = C.c_void_p()
        check(lib.pw_store_create(nbytes, C.byref(h)))
        self.handle = h

    def alloc(self, nbytes, owner=0, timeout_ns=-1):
        """(object handle, device address)."""
        obj, ptr = C.c_uint64(0), C.c_void_p()
        check(lib.pw_store_alloc(self.handle, nbytes, owner, timeout_ns, C.byref(obj), C.byref(ptr)))
        return obj.value, ptr.value

    def tensor(self, ptr, shape, dtype="float32"):
        """A torch tensor over store memory (borrowed: valid until freed)."""
        import torch
        return torch.as_tensor(_DeviceArray(ptr, shape, self._TYPESTR[dtype]), device="cuda")

    def free(self, obj, stream=None):
        check(lib.pw_store_free(self.handle, obj, _stream(stream)))

    def release_owner(self, owner, stream=None) -> int:
        n = C.c_uint64(0)
        check(lib.pw_store_release_owner(self.handle, owner, _stream(stream), C.byref(n)))
        return n.value

    def stats(self) -> dict:
        st = pw_store_stats()
        check(lib.pw_store_get_stats(self.handle, C.byref(st)))
        return {name: getattr(st, name) for name, _ in st._fields_}

    def destroy(self):
        if self.handle:
            check(lib.pw_store_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                lib.pw_store_destroy(self.handle)
        except Exception:
            pass
