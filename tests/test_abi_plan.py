"""Host-side checks of the C ABI library: it loads, exports every entry point
that include/rar.h declares, and its host planner agrees with the oracle and
with the pages' tables.  No GPU needed (no compute call is made)."""
import ctypes
import itertools
import json
import os
import re

import numpy as np
import pytest

import oracle
import ring_all_reduce_channelmask_amd as rar
from ring_all_reduce_channelmask_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "rar.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:rar_result_t|const char\*)\s+(\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(n for n, _, _ in _lib.SIGNATURES) == names


def test_error_strings():
    lib = _lib.load()
    for code in range(6):
        assert lib.rar_get_error_string(code)


def test_cache_release_with_nothing_cached_touches_no_device():
    # no communicator is cached in this process: the call returns at once,
    # making no HIP call (on a host without a GPU any HIP call would fail)
    assert _lib.load().ring_allreduce_cache_release() == _lib.SUCCESS
    rar.ring_allreduce_cache_release()


def test_ring_info_matches_pages_and_oracle():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "ring_tables.json")))
    for key in ("0-1-2-3", "0-2-3-1"):
        t = g["ring_index_tables"][key]
        idx, prv, nxt = rar.ring_info(t["order"])
        for rank, ix, p, n in t["rows"]:
            assert (idx[rank], prv[rank], nxt[rank]) == (ix, p, n)
    rng = np.random.default_rng(1)
    for N in (2, 3, 5, 8, 13, 64):
        for _ in range(5):
            order = [int(x) for x in rng.permutation(N)]
            assert [list(v) for v in rar.ring_info(order)] == \
                [list(v) for v in oracle.ring_setup(order)]


@pytest.mark.parametrize("order", [[0, 1, 1, 2], [0, 1, 2, 4], [0], [-1, 0]])
def test_ring_info_rejects(order):
    with pytest.raises(rar.RarError) as e:
        rar.ring_info(order)
    assert e.value.code == _lib.INVALID_ARGUMENT


PLAN_CASES = [
    (4, 0x1, "SIMPLE", 65536, 4, "float32", [1024]),
    (4, 0xF, "LL", 512 * 1024, 4, "float32", [131072]),
    (4, 0xFFF, "SIMPLE", 4 << 20, 4, "float32", [16 << 20]),
    (4, 0xFFF, "LL128", 4915200, 4, "float32", [16 << 20]),
    (8, 0xFFFF, "SIMPLE", 4 << 20, 4, "bfloat16", [32 << 20]),
    (8, 0xFFFF, "SIMPLE", 4 << 20, 2, "int32", [32 << 20]),
    (4, 0b101101010011, "LL", 512 * 1024, 4, "bfloat16", [7168] * 104),
    (3, 0x5, "LL128", 8 * 2048, 4, "int32", [1, 0, 77, 4099, 3]),
    (2, 1 << 63, "SIMPLE", 8 * 512, 2, "float32", [0, 5]),
    # element, channel and byte offsets beyond 2^31 and 2^32
    (4, (1 << 64) - 1, "SIMPLE", 4 << 20, 4, "int32", [(1 << 31) + 5, 3, (1 << 33) + 17]),
    (3, 0xF0F, "LL128", 4915200, 4, "bfloat16", [(1 << 32) + 9, 0, 1 << 31]),
]


@pytest.mark.parametrize("case", PLAN_CASES, ids=[f"{c[2]}-{c[5]}-{len(c[6])}" for c in PLAN_CASES])
def test_planner_matches_oracle_split(case):
    N, mask, proto, buff, cs, dt, counts = case
    ours, cmax = rar.plan_pieces(N, mask, proto, buff, cs, dt, counts)
    theirs, ocmax = oracle.geometry(N, mask, proto, buff, cs, dt, counts)
    assert cmax == ocmax
    assert ours == theirs


def test_planner_pages_geometry():
    """Course 23 "Buffer 到 Chunk 的实测公式" and the LL/LL128 default chunks."""
    for buff, chunk_bytes in [(65536, 32768), (1 << 20, 512 << 10), (4 << 20, 2 << 20)]:
        _, cmax = rar.plan_pieces(4, 0xF, "SIMPLE", buff, 4, "float32", [16 << 20])
        assert cmax * 4 == chunk_bytes
    _, cmax = rar.plan_pieces(4, 0xF, "LL", 0, 0, "float32", [1])
    assert cmax * 4 == 32768
    _, cmax = rar.plan_pieces(4, 0xF, "LL128", 0, 0, "float32", [1])
    assert cmax * 4 == 576000


@pytest.mark.parametrize("args,why", [
    ((4, 0, "SIMPLE", 65536, 4), "empty mask"),
    ((4, 1, "SIMPLE", 65536, 8), "chunk of 8 steps deadlocks"),
    ((4, 1, "SIMPLE", 65536, 3), "odd chunkSteps"),
    ((4, 1, "SIMPLE", 65536 + 128, 4), "Simple buffer not a multiple of 512"),
    ((4, 1, "LL", 65536 + 128, 4), "LL buffer not a multiple of 256"),
    ((4, 1, "LL128", 4915200 + 1024, 4), "LL128 buffer not a multiple of 2048"),
    ((1, 1, "SIMPLE", 65536, 4), "one rank"),
    ((65, 1, "SIMPLE", 65536, 4), "too many ranks"),
])
def test_planner_rejects(args, why):
    with pytest.raises(rar.RarError) as e:
        rar.plan_pieces(*args, "float32", [100])
    assert e.value.code == _lib.INVALID_ARGUMENT, why


def test_comm_create_validates_before_touching_a_device():
    """Invalid arguments are rejected on the host, before any HIP call."""
    for kwargs in [dict(nranks=4, ring_order=[0, 1, 2, 2], mask=1),
                   dict(nranks=4, ring_order=[0, 1, 2, 3], mask=0),
                   dict(nranks=4, ring_order=[0, 1, 2, 3], mask=1, chunk_steps=8),
                   dict(nranks=4, ring_order=[0, 1, 2, 3], mask=1, lanes=99),
                   dict(nranks=4, ring_order=[0, 1, 2, 3], mask=1, waves=9),
                   dict(nranks=4, ring_order=[0, 1, 2, 3], mask=1, deal_works=2),
                   dict(nranks=4, ring_order=[[0, 1, 2, 3], [0, 1, 3, 3]], mask=3),
                   dict(nranks=3, ring_order=[[0, 1, 2]] * 65, mask=1)]:
        with pytest.raises(rar.RarError) as e:
            rar.Comm(**kwargs)
        assert e.value.code == _lib.INVALID_ARGUMENT, kwargs


def test_package_fails_loudly_without_library(tmp_path, monkeypatch):
    """The product path has no fallback: a missing librar.so is an error."""
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "librar.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()


def _oneshot_raw(send, recv, count, dtype="float32", op=0, tune=None, nranks=None):
    lib = _lib.load()
    n = len(send) if nranks is None else nranks
    s = (ctypes.c_void_p * len(send))(*send)
    r = (ctypes.c_void_p * len(recv))(*recv)
    t = _lib.OneshotTuning(*(tune or (0, 0, 0, 0)))
    return lib.rar_oneshot_allreduce(s, r, n, count, _lib.DTYPE[dtype], op, ctypes.byref(t), None)


def test_oneshot_validates_on_the_host():
    """Bad arguments are rejected before any HIP call; nothing here is ever
    dereferenced (the addresses are made up and no launch happens)."""
    A = 1 << 40
    ok_s, ok_r = [A, A + 4096], [A + 8192, A + 12288]
    assert _oneshot_raw(ok_s, ok_r, 0) == _lib.SUCCESS                  # count 0: no launch
    assert _oneshot_raw([0, 0], [0, 0], 0) == _lib.SUCCESS              # pointers not looked at
    bad = [
        (dict(send=ok_s, recv=ok_r, count=16, nranks=1), "one rank"),
        (dict(send=ok_s, recv=ok_r, count=16, nranks=65), "65 ranks"),
        (dict(send=[A, A + 4098], recv=ok_r, count=16), "not element-aligned (fp32 at 2 mod 4)"),
        (dict(send=[A, 0], recv=ok_r, count=16), "NULL"),
        (dict(send=[A, A + 64], recv=ok_r, count=17), "send buffers overlap (17 fp32 > 64 B)"),
        (dict(send=ok_s, recv=[A + 8192, A + 8192], count=16), "two ranks share a receive buffer"),
        (dict(send=ok_s, recv=[A + 4096, A + 12288], count=16), "rank 0 receives into rank 1's input"),
        (dict(send=ok_s, recv=ok_r, count=16, tune=(0, 9, 0, 0)), "waves"),
        (dict(send=ok_s, recv=ok_r, count=16, tune=(0, 0, 3, 0)), "unroll"),
        (dict(send=ok_s, recv=ok_r, count=16, tune=(-1, 0, 0, 0)), "workgroups"),
    ]
    for kw, why in bad:
        assert _oneshot_raw(**kw) == _lib.INVALID_ARGUMENT, why
    assert _oneshot_raw(ok_s, ok_r, 16, op=7) == _lib.INVALID_ARGUMENT  # unknown operator
    # PreMulSum only through the entry point that takes scalars
    assert _oneshot_raw(ok_s, ok_r, 16, op=5) == _lib.INVALID_ARGUMENT
    lib = _lib.load()
    s = (ctypes.c_void_p * 2)(*ok_s)
    r = (ctypes.c_void_p * 2)(*ok_r)
    t = _lib.OneshotTuning(0, 0, 0, 0)
    assert lib.rar_oneshot_allreduce_premul(s, r, 2, 16, _lib.DTYPE["float32"], None,
                                            ctypes.byref(t), None) == _lib.INVALID_ARGUMENT


def test_planner_matches_oracle_split_random():
    """The host planner and the oracle's geometry agree on random launches:
    any ring size, sparse or dense masks, every protocol and dtype, buffer
    sizes on each protocol's quantum, and groups of ragged counts (zeros
    included)."""
    from hypothesis import given, settings, strategies as st

    quantum = {"SIMPLE": 512, "LL": 256, "LL128": 2048}

    @settings(max_examples=300, deadline=None, derandomize=True)
    @given(N=st.integers(2, 64), mask=st.integers(1, 2 ** 64 - 1),
           proto=st.sampled_from(["SIMPLE", "LL", "LL128"]),
           units=st.integers(1, 64), cs=st.sampled_from([2, 4]),
           dt=st.sampled_from(["int32", "float32", "bfloat16"]),
           counts=st.lists(st.integers(0, 300000), min_size=1, max_size=40))
    def check(N, mask, proto, units, cs, dt, counts):
        buff = 8 * quantum[proto] * units
        ours, cmax = rar.plan_pieces(N, mask, proto, buff, cs, dt, counts)
        theirs, ocmax = oracle.geometry(N, mask, proto, buff, cs, dt, counts)
        assert cmax == ocmax
        assert ours == theirs

    check()


def test_plan_pieces_buffer_checks_and_count_query():
    """rar_plan_pieces with cap = 0 and no buffer returns the piece count
    only; a negative cap or a NULL buffer with cap > 0 is an invalid
    argument."""
    lib = _lib.load()
    counts = (ctypes.c_size_t * 2)(100000, 7)
    n, cmax = ctypes.c_int(), ctypes.c_int64()
    rc = lib.rar_plan_pieces(4, 0xF, _lib.PROTO["SIMPLE"], 65536, 4, _lib.DTYPE["float32"], 2,
                             counts, None, 0, ctypes.byref(n), ctypes.byref(cmax))
    assert rc == 0
    ours, _ = rar.plan_pieces(4, 0xF, "SIMPLE", 65536, 4, "float32", [100000, 7])
    assert n.value == len(ours)
    for cap, buf in ((-1, None), (4, None)):
        rc = lib.rar_plan_pieces(4, 0xF, _lib.PROTO["SIMPLE"], 65536, 4, _lib.DTYPE["float32"], 2,
                                 counts, buf, cap, ctypes.byref(n), ctypes.byref(cmax))
        assert rc == _lib.INVALID_ARGUMENT


def _ptrs(vals):
    return (ctypes.c_void_p * len(vals))(*vals)


@pytest.mark.parametrize("entry", ["ring", "oneshot"])
def test_overlapping_ranks_rejected_before_any_device_call(entry):
    """Buffers of different ranks that overlap are refused on the host (no
    HIP call is made: this container has no GPU, so any device call would
    fail with a HIP error instead)."""
    lib = _lib.load()
    N, count, base = 4, 1000, 1 << 32
    order = (ctypes.c_int * N)(0, 2, 3, 1)
    sends = [base + r * 8192 for r in range(N)]
    cases = {
        "recv of rank 1 inside send of rank 2": (sends, [base + 65536 + r * 8192 for r in range(N)],
                                                  {1: sends[2] + 4}),
        "two ranks share a send buffer": ([sends[0], sends[0], sends[2], sends[3]], None, {}),
        "recv of rank 3 = send of rank 0": (sends, [base + 65536 + r * 8192 for r in range(N)],
                                            {3: sends[0]}),
    }
    for what, (s, r, patch) in cases.items():
        s = list(s)
        r = list(r) if r is not None else [base + 65536 + k * 8192 for k in range(N)]
        for k, v in patch.items():
            r[k] = v
        if entry == "ring":
            rc = lib.ring_allreduce(_ptrs(s), _ptrs(r), N, count, _lib.DTYPE["float32"], 0, order,
                                    _lib.PROTO["SIMPLE"], 2, 0, 0, None)
        else:
            rc = lib.rar_oneshot_allreduce(_ptrs(s), _ptrs(r), N, count, _lib.DTYPE["float32"], 0,
                                           None, None)
        assert rc == _lib.INVALID_ARGUMENT, what
        assert b"overlap" in lib.rar_get_last_error(), what


def test_ring_allreduce_checks_arguments_on_the_host():
    lib = _lib.load()
    N = 4
    order = (ctypes.c_int * N)(0, 1, 1, 2)   # not a permutation
    s = _ptrs([(1 << 32) + k * 8192 for k in range(N)])
    r = _ptrs([(1 << 33) + k * 8192 for k in range(N)])
    assert lib.ring_allreduce(s, r, N, 100, 1, 0, order, 2, 1, 0, 0, None) == _lib.INVALID_ARGUMENT
    order = (ctypes.c_int * N)(0, 1, 2, 3)
    # misaligned fp32 buffer, bad dtype, bad operator, bad chunk steps
    bad = _ptrs([(1 << 32) + 2] + [(1 << 32) + k * 8192 for k in range(1, N)])
    assert lib.ring_allreduce(bad, r, N, 100, 1, 0, order, 2, 1, 0, 0, None) == _lib.INVALID_ARGUMENT
    assert lib.ring_allreduce(s, r, N, 100, 7, 0, order, 2, 1, 0, 0, None) == _lib.INVALID_ARGUMENT
    assert lib.ring_allreduce(s, r, N, 100, 1, 9, order, 2, 1, 0, 0, None) == _lib.INVALID_ARGUMENT
    assert lib.ring_allreduce(s, r, N, 100, 1, 0, order, 2, 1, 0, 8, None) == _lib.INVALID_ARGUMENT
    # nothing to move: success without touching the device
    assert lib.ring_allreduce(None, None, N, 0, 1, 0, order, 2, 1, 0, 0, None) == _lib.SUCCESS


def test_group_discard_rejects_null():
    lib = _lib.load()
    assert lib.rar_group_discard(None) == _lib.INVALID_ARGUMENT


def test_group_context_discards_on_error(monkeypatch):
    """Comm.group(): a body that raises drops the queued calls (the C call
    rar_group_discard) and launches nothing; the body's exception is the one
    that propagates.  Checked against a stand-in library that records calls."""
    calls = []

    class FakeLib:
        def rar_group_start(self, h):
            calls.append("start")
            return 0

        def rar_group_end(self, h, s):
            calls.append("end")
            return 0

        def rar_group_discard(self, h):
            calls.append("discard")
            return 0

    monkeypatch.setattr(_lib, "load", lambda: FakeLib())
    monkeypatch.setattr(rar, "_stream_handle", lambda s: None)
    c = rar.Comm.__new__(rar.Comm)
    c._h = ctypes.c_void_p(1)
    with pytest.raises(KeyError):
        with c.group():
            raise KeyError("queueing failed")
    assert calls == ["start", "discard"]
    calls.clear()
    with c.group():
        pass
    assert calls == ["start", "end"]
    c._h = None


# ---- GRAPH lines (rar_graph_text) ----------------------------------------

def _graph_lines(nranks, rings, mask):
    return rar.graph_text(nranks, rings, mask).splitlines()


@pytest.mark.parametrize("key,n", [("n2", 2), ("n3", 3), ("n4", 4)])
def test_graph_text_reproduces_the_pages_channel_rings(key, n):
    """Course 12 "GRAPH 重建": with the pages' base rings duplicated over 12
    channels, channel c runs base ring c mod len(base); each line lists that
    ring from rank 0."""
    with open(os.path.join(ROOT, "tests", "golden", "graph_rings.json")) as f:
        g = json.load(f)[key]
    base, nch = g["base"], g["channels"]
    lines = _graph_lines(n, base, (1 << nch) - 1)
    assert len(lines) == nch
    for c, line in enumerate(lines):
        want = base[c % len(base)]
        assert line == f"Channel {c:02d}/{nch:02d} : " + " ".join(map(str, want))


def test_graph_text_the_pages_single_line():
    """Course 12 "Graph 如何变成完整 ring" prints the ring 0-2-3-1 of channel 2
    of 12 as "Channel 02/12 : 0 2 3 1"; any rotation of the ring order walks
    the same connector graph, so it prints the same line."""
    for order in ([0, 2, 3, 1], [2, 3, 1, 0], [3, 1, 0, 2], [1, 0, 2, 3]):
        assert _graph_lines(4, order, (1 << 12) - 1)[2] == "Channel 02/12 : 0 2 3 1"
    # N=2, one channel: a single line with the one ring
    assert _graph_lines(2, [1, 0], 1) == ["Channel 00/01 : 0 1"]


def test_graph_text_sparse_mask_and_reversed_ring():
    lines = _graph_lines(4, [0, 1, 2, 3], (1 << 63) | (1 << 9) | 1)
    assert lines == ["Channel 00/64 : 0 1 2 3", "Channel 09/64 : 0 1 2 3", "Channel 63/64 : 0 1 2 3"]
    # the reversed ring walks next the other way round
    assert _graph_lines(4, [3, 2, 1, 0], 1) == ["Channel 00/01 : 0 3 2 1"]


def test_graph_text_errors_and_sizes():
    lib = _lib.load()
    ring = (ctypes.c_int * 4)(0, 2, 3, 1)
    n = ctypes.c_size_t(0)
    assert lib.rar_graph_text(4, 1, ring, 0xFFF, None, 0, ctypes.byref(n)) == 0
    assert n.value == 12 * len("Channel 00/12 : 0 2 3 1\n")
    small = ctypes.create_string_buffer(10)
    m = ctypes.c_size_t(0)
    assert lib.rar_graph_text(4, 1, ring, 0xFFF, small, 10, ctypes.byref(m)) == 1
    assert m.value == n.value and b"needed" in lib.rar_get_last_error()
    bad = (ctypes.c_int * 4)(0, 2, 2, 1)
    assert lib.rar_graph_text(4, 1, bad, 1, None, 0, None) == 1
    assert lib.rar_graph_text(4, 1, ring, 0, None, 0, None) == 1
    assert lib.rar_graph_text(4, 0, ring, 1, None, 0, None) == 1
    assert lib.rar_graph_text(1, 1, ring, 1, None, 0, None) == 1
    assert lib.rar_graph_text(4, 1, None, 1, None, 0, None) == 1
    # a base ring that is not a permutation fails even if no channel uses it
    two = (ctypes.c_int * 8)(0, 1, 2, 3, 0, 0, 1, 2)
    assert lib.rar_graph_text(4, 2, two, 1, None, 0, None) == 1
