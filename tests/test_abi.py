"""The C-ABI library loads, exports every symbol include/pw.h declares, and
its host-only paths (sizing, validation, error codes, futures of unknown
plans) work without a GPU. No compute call is made here."""
import ctypes as C
import os
import re

import pytest

import sparse_shard_exchange_amd as pw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "pw.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(pw_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) >= 12, names
    lib = C.CDLL(pw.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(pw._SIGNATURES), set(names) ^ set(pw._SIGNATURES)


def test_abi_version_and_strerror():
    assert pw.lib.pw_abi_version() == pw.PW_ABI_VERSION
    for code in range(0, -8, -1):
        s = pw.lib.pw_strerror(code)
        assert s and s != b"unknown status"
    assert pw.lib.pw_strerror(-99) == b"unknown status"


def test_struct_sizes_match_the_header_layout():
    # field order and padding follow the C declarations on x86-64
    assert C.sizeof(pw.pw_op) == 12
    assert C.sizeof(pw.pw_future_t) == 24
    assert C.sizeof(pw.pw_sharded_buf) == 40
    assert C.sizeof(pw.pw_plan_desc) == 112
    assert C.sizeof(pw.pw_exchange_io) == 144
    assert C.sizeof(pw.pw_program) == 216
    assert C.sizeof(pw.pw_sched_record) == 40
    assert C.sizeof(pw.pw_store_stats) == 72


def test_store_argument_errors_need_no_device():
    h = C.c_void_p(0)
    assert pw.lib.pw_store_create(100, C.byref(h)) == pw.PW_ERR_INVALID   # below 256 bytes
    assert pw.lib.pw_store_create(1 << 20, None) == pw.PW_ERR_INVALID
    obj, ptr = C.c_uint64(0), C.c_void_p()
    assert pw.lib.pw_store_alloc(None, 256, 0, 0, C.byref(obj), C.byref(ptr)) == pw.PW_ERR_INVALID
    assert pw.lib.pw_store_free(None, 1, None) == pw.PW_ERR_INVALID
    assert pw.lib.pw_store_release_owner(None, 1, None, None) == pw.PW_ERR_INVALID
    st = pw.pw_store_stats()
    assert pw.lib.pw_store_get_stats(None, C.byref(st)) == pw.PW_ERR_INVALID
    assert pw.lib.pw_store_destroy(None) == pw.PW_ERR_INVALID


def test_scheduler_argument_errors_need_no_device():
    h = C.c_void_p(0)
    assert pw.lib.pw_sched_create(0, C.byref(h)) == pw.PW_ERR_INVALID
    assert pw.lib.pw_sched_create(65, C.byref(h)) == pw.PW_ERR_INVALID
    assert pw.lib.pw_sched_create(1, None) == pw.PW_ERR_INVALID
    c = C.c_uint32(0)
    assert pw.lib.pw_sched_add_client(None, 1, C.byref(c)) == pw.PW_ERR_INVALID
    t = C.c_uint64(0)
    prog = pw.pw_program()
    assert pw.lib.pw_sched_submit(None, 0, C.byref(prog), C.byref(t)) == pw.PW_ERR_INVALID
    assert pw.lib.pw_sched_wait(None, 1, 0) == pw.PW_ERR_INVALID
    assert pw.lib.pw_sched_hold(None, 1) == pw.PW_ERR_INVALID
    n = C.c_size_t(0)
    assert pw.lib.pw_sched_records(None, None, 0, C.byref(n)) == pw.PW_ERR_INVALID
    assert pw.lib.pw_sched_destroy(None) == pw.PW_ERR_INVALID


def _ex(**kw):
    base = dict(kind=pw.PW_GRAPH_EXCHANGE, num_shards=256, tuples_per_shard=65536, payload_elems=64)
    base.update(kw)
    return pw.desc(**base)


def test_sizing_is_host_only_and_scales_with_tiles():
    small = pw.workspace_size(_ex(num_shards=8, tuples_per_shard=4096))
    big = pw.workspace_size(_ex())
    assert 0 < small < big
    assert big >= 256 * 4096 * 4        # the destination x tile table of the large exchange


@pytest.mark.parametrize("bad,code", [
    (dict(num_shards=0), pw.PW_ERR_INVALID),
    (dict(kind=9), pw.PW_ERR_INVALID),
    (dict(dtype=7), pw.PW_ERR_INVALID),
    (dict(payload_elems=0), pw.PW_ERR_INVALID),
    (dict(dtype=pw.PW_BF16, payload_elems=3), pw.PW_ERR_INVALID),
    (dict(a_op=pw.op(pw.PW_OP_ROWSUM)), pw.PW_ERR_INVALID),
    (dict(b_op=pw.op(11)), pw.PW_ERR_INVALID),
    (dict(dtype=pw.PW_BF16, a_op=pw.op(pw.PW_OP_AFFINE, 2, 1)), pw.PW_ERR_INVALID),
    (dict(tuples_per_shard=1 << 24), pw.PW_ERR_INVALID),
    (dict(flags=0x80), pw.PW_ERR_INVALID),
    (dict(flags=pw.PW_FLAG_STAGE_WINDOWS), pw.PW_ERR_INVALID),   # a pipeline claim order on an exchange
])
def test_validation_errors(bad, code):
    d = _ex(**bad)
    need = C.c_size_t(0)
    rc = pw.lib.pw_plan(C.byref(d), None, 0, C.byref(need), None)
    assert rc == code
    assert pw.lib.pw_last_error()


def test_bad_abi_version():
    d = _ex()
    d.abi_version = 99
    with pytest.raises(pw.PwError) as e:
        pw.workspace_size(d)
    assert e.value.code == pw.PW_ERR_INVALID and b"abi_version" in pw.lib.pw_last_error()


def test_workspace_too_small_is_nomem_before_any_device_call():
    d = _ex(num_shards=8, tuples_per_shard=4096)
    need = pw.workspace_size(d)
    h = C.c_void_p()
    # a fake 256-aligned pointer: the size check fails before the pointer is used
    rc = pw.lib.pw_plan(C.byref(d), C.c_void_p(1 << 20), need - 256, None, C.byref(h))
    assert rc == pw.PW_ERR_NOMEM
    rc = pw.lib.pw_plan(C.byref(d), C.c_void_p((1 << 20) + 8), need, None, C.byref(h))
    assert rc == pw.PW_ERR_INVALID     # misaligned workspace


def test_calls_on_dead_plans_and_futures():
    assert pw.lib.pw_plan_destroy(None) == pw.PW_ERR_STATE
    assert pw.lib.pw_plan_destroy(C.c_void_p(0xdead0)) == pw.PW_ERR_STATE
    f = pw.pw_future_t(12345, pw.PW_NODE_RESULT, -1, 1)
    assert pw.lib.pw_future_wait(f, 0) == pw.PW_ERR_STATE
    fired = C.c_int(7)
    assert pw.lib.pw_future_query(f, C.byref(fired)) == pw.PW_ERR_STATE and fired.value == 0
    io = pw.pw_exchange_io()
    fut = pw.pw_future_t()
    assert pw.lib.pw_exchange(None, C.byref(io), None, C.byref(fut)) == pw.PW_ERR_STATE
    st = pw.pw_sharded_buf()
    assert pw.lib.pw_chain_run(None, 1, C.byref(st), None, None, C.byref(fut)) == pw.PW_ERR_STATE


@pytest.mark.parametrize("bad", [
    dict(num_shards=0), dict(tuples_per_shard=0), dict(dtype=pw.PW_BF16),
    dict(a_op=pw.op(pw.PW_OP_ROWSUM)), dict(chain_mode=7),
])
def test_chain_validation(bad):
    base = dict(kind=pw.PW_GRAPH_CHAIN, num_shards=2048, tuples_per_shard=128,
                a_op=pw.op(pw.PW_OP_AFFINE, 1, 1), b_op=pw.op(pw.PW_OP_AFFINE, 0.5, 0))
    base.update(bad)
    with pytest.raises(pw.PwError) as e:
        pw.workspace_size(pw.desc(**base))
    assert e.value.code == pw.PW_ERR_INVALID


@pytest.mark.parametrize("bad, code", [
    (dict(payload_elems=1536), pw.PW_ERR_INVALID),   # the router's W_r^T must fit one CU's LDS
    (dict(payload_elems=1000), pw.PW_ERR_INVALID),
    (dict(hidden=4000), pw.PW_ERR_INVALID),
    (dict(top_k=1), pw.PW_ERR_UNSUPPORTED),
    (dict(num_shards=65), pw.PW_ERR_INVALID),
    (dict(w1=None), pw.PW_ERR_INVALID),
    (dict(dtype=pw.PW_F32), pw.PW_ERR_INVALID),
])
def test_moe_validation(bad, code):
    fake = 1 << 40  # never dereferenced: sizing is host-only
    base = dict(kind=pw.PW_GRAPH_MOE, num_shards=64, tuples_per_shard=2048, num_src_shards=64, payload_elems=1024,
                dtype=pw.PW_BF16, top_k=2, hidden=4096, w_router=fake, w1=fake, w2=fake)
    assert pw.workspace_size(pw.desc(**base)) > 0
    base.update(bad)
    with pytest.raises(pw.PwError) as e:
        pw.workspace_size(pw.desc(**base))
    assert e.value.code == code


def test_chain_sizing():
    d = pw.desc(pw.PW_GRAPH_CHAIN, 2048, 128, a_op=pw.op(pw.PW_OP_AFFINE, 1, 1))
    assert pw.workspace_size(d) >= 2048 * 128 * 4


def test_scratch_exchange_size_limit_needs_no_device():
    """The allocation-free step rejects a descriptor whose tables outgrow its
    8 MiB static array before any device call, naming both sizes."""
    d = pw.desc(pw.PW_GRAPH_EXCHANGE, 256, 65536, 64)
    io = pw.pw_exchange_io()
    rc = pw.lib.pw_exchange_scratch(C.byref(d), C.byref(io), None)
    assert rc == pw.PW_ERR_INVALID
    msg = pw.lib.pw_last_error().decode()
    assert "8388608" in msg, msg
    d2 = pw.desc(pw.PW_GRAPH_CHAIN, 8, 128, 0)
    assert pw.lib.pw_exchange_scratch(C.byref(d2), C.byref(io), None) == pw.PW_ERR_INVALID
