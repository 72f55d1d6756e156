"""CPU oracle for the ring AllReduce hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (the HIP library and its Python binding) never does, and shares no code
with it.

Two independent descriptions of the same computation live here:

* ``ring_sim.cpp`` (loaded through ctypes): a sequential simulator of the
  N-rank state machine -- connectors with head/tail credit over FIFO slots, LL
  and LL128 line formats with step+1 flags, the runRing primitive sequence and
  the channel split -- following the two course pages
  [C12] "NCCL 专家课程 12：Ring AllReduce 逐步推导、真实 Ring 与 Channel 并行" and
  [C23] "NCCL 专家课程 23：Device Kernel、Primitives、Step/Credit 与 LL Flag".
* ``closed_form.py``: the result written out directly -- for every element,
  the ordered fold of the N inputs that the ring produces, with no FIFOs.

Parity pinned to the readings, not to the pages, for floating results at the
large workloads: the pages print no output values.  The pins are listed in the
tests (`tests/test_oracle_*.py`).
"""
import ctypes
import os

import numpy as np

from . import build as _build

PROTO = {"LL": 0, "LL128": 1, "SIMPLE": 2}
DTYPE = {"int32": 0, "float32": 1, "bfloat16": 2}
OPS = {0: "send", 1: "recvReduceSend", 2: "directRecvReduceCopySend",
       3: "directRecvCopySend", 4: "directRecv"}
OK, DEADLOCK, INVALID, CORRUPT = 0, 1, 2, 3
RED = {"sum": 0, "prod": 1, "max": 2, "min": 3, "avg": 4, "premulsum": 5}
FAULTS = {"none": 0, "drop_recv_head": 1, "tail_before_payload": 2, "ll_flag2_missing": 3,
          "ll_constant_flag": 4, "ll128_flag_missing": 5, "ll128_flag_before_data": 6}


class Piece(ctypes.Structure):
    _fields_ = [("channel", ctypes.c_int32), ("channel_id", ctypes.c_int32),
                ("work", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("grid_offset", ctypes.c_int64), ("channel_count", ctypes.c_int64),
                ("chunk_count", ctypes.c_int64)]


class Call(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("channel_id", ctypes.c_int32),
                ("work", ctypes.c_int32), ("op", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("loop", ctypes.c_int32),
                ("offset", ctypes.c_int64), ("nelem", ctypes.c_int64)]


class Stats(ctypes.Structure):
    _fields_ = [("send_ops", ctypes.c_int64 * 64), ("recv_ops", ctypes.c_int64 * 64),
                ("payload_sent", ctypes.c_int64 * 64), ("wire_sent", ctypes.c_int64 * 64),
                ("units_run", ctypes.c_int64), ("calls_recorded", ctypes.c_int64),
                ("deadlock_rank", ctypes.c_int32), ("deadlock_channel", ctypes.c_int32),
                ("deadlock_send_step", ctypes.c_int64), ("deadlock_recv_step", ctypes.c_int64)]


_lib = None


def lib():
    """Load the compiled simulator, building it first if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        i32p = ctypes.POINTER(ctypes.c_int)
        L.orc_ring_setup.argtypes = [ctypes.c_int, i32p, i32p, i32p, i32p]
        L.orc_ring_schedule.argtypes = [ctypes.c_int, ctypes.c_int, i32p, i32p]
        L.orc_geometry.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_int, ctypes.c_size_t,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(Piece),
                                   ctypes.c_int, ctypes.POINTER(ctypes.c_int64)]
        L.orc_allreduce.argtypes = [ctypes.c_int, i32p, ctypes.c_uint64, ctypes.c_int,
                                    ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_size_t),
                                    ctypes.POINTER(ctypes.c_void_p),
                                    ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_int,
                                    ctypes.c_uint64, ctypes.c_int, ctypes.POINTER(Stats),
                                    ctypes.POINTER(Call), ctypes.c_int64]
        L.orc_allreduce_rings.argtypes = [ctypes.c_int, ctypes.c_int, i32p, ctypes.c_uint64,
                                          ctypes.c_int, ctypes.c_size_t, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int,
                                          ctypes.POINTER(ctypes.c_size_t),
                                          ctypes.POINTER(ctypes.c_void_p),
                                          ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                          ctypes.c_int, ctypes.c_uint64, ctypes.c_int,
                                          ctypes.POINTER(Stats), ctypes.POINTER(Call),
                                          ctypes.c_int64]
        L.orc_stream_fault.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_int64),
                                       ctypes.POINTER(ctypes.c_int64),
                                       ctypes.POINTER(ctypes.c_int64)]
        L.orc_allreduce_premul.argtypes = [ctypes.c_int, ctypes.c_int, i32p, ctypes.c_uint64,
                                           ctypes.c_int, ctypes.c_size_t, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int,
                                           ctypes.POINTER(ctypes.c_size_t),
                                           ctypes.POINTER(ctypes.c_void_p),
                                           ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                           ctypes.c_int, ctypes.POINTER(Stats),
                                           ctypes.POINTER(Call), ctypes.c_int64]
        L.orc_ll_wrap.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, i32p, ctypes.c_int, ctypes.POINTER(ctypes.c_int64)]
        L.orc_bf16_round.argtypes = [ctypes.c_double]
        L.orc_bf16_round.restype = ctypes.c_uint16
        _lib = L
    return _lib


def _ints(seq):
    arr = (ctypes.c_int * len(seq))(*[int(x) for x in seq])
    return arr


def ring_setup(ring_order):
    """Return (index, prev, next) lists indexed by user rank, or None if invalid."""
    n = len(ring_order)
    idx, prv, nxt = (ctypes.c_int * n)(), (ctypes.c_int * n)(), (ctypes.c_int * n)()
    rc = lib().orc_ring_setup(n, _ints(ring_order), idx, prv, nxt)
    if rc != OK:
        return None
    return list(idx), list(prv), list(nxt)


def ring_schedule(nranks, ring_index):
    """The 2N-1 (op name, chunk) rows of one loop for the rank at ``ring_index``."""
    ops, chunks = (ctypes.c_int * (2 * nranks - 1))(), (ctypes.c_int * (2 * nranks - 1))()
    k = lib().orc_ring_schedule(nranks, ring_index, ops, chunks)
    assert k == 2 * nranks - 1
    return [(OPS[ops[i]], chunks[i]) for i in range(k)]


def geometry(nranks, mask, proto, buff_size, chunk_steps, dtype, counts):
    """Pieces of the channel split: list of dicts, plus the protocol's chunk maximum."""
    counts = list(counts)
    carr = (ctypes.c_size_t * len(counts))(*counts)
    cap = 64 * (len(counts) + 1) + 64
    pieces = (Piece * cap)()
    cmax = ctypes.c_int64()
    n = lib().orc_geometry(nranks, mask, PROTO[proto], buff_size, chunk_steps, DTYPE[dtype],
                           len(counts), carr, pieces, cap, ctypes.byref(cmax))
    if n < 0:
        return None, None
    assert n <= cap
    out = [dict(channel=p.channel, channel_id=p.channel_id, work=p.work,
                grid_offset=p.grid_offset, channel_count=p.channel_count,
                chunk_count=p.chunk_count) for p in pieces[:n]]
    return out, cmax.value


def allreduce(inputs, ring_order, mask, proto, buff_size, chunk_steps, dtype, *,
              in_place=False, slots=8, sched=0, seed=0, drop_recv_head=False,
              direct=False, log_calls=False, op="sum", ll_wrap8=False, direct_read=False,
              scalars=None, threads=None):
    """Run the simulator.

    ``inputs`` is a list over works of arrays shaped [N, count] holding the raw
    elements (int32, float32, or uint16 bit patterns for bfloat16).
    ``ring_order`` is one ring, or a list of rings (channel id c runs ring
    c mod len(rings)).  ``op="premulsum"`` needs ``scalars``, an array
    [works, N] of payload-type elements (rank r's scalar for work w).
    ``threads``: run the channels in parallel on that many threads (0 = one
    per hardware thread), each channel with the round-robin schedule; the
    outputs are those of any interleaving.  Returns
    (rc, outputs, stats, calls): outputs is a list over works of [N, count]
    arrays in the same representation.
    """
    rings = [list(r) for r in ring_order] if isinstance(ring_order[0], (list, tuple)) \
        else [list(ring_order)]
    N = len(rings[0])
    if isinstance(inputs, np.ndarray):
        inputs = [inputs]
    works = [np.ascontiguousarray(x) for x in inputs]
    counts = [int(x.shape[1]) for x in works]
    keep = []
    send_ptrs = (ctypes.c_void_p * (N * len(works)))()
    recv_ptrs = (ctypes.c_void_p * (N * len(works)))()
    outs = []
    for w, x in enumerate(works):
        assert x.shape[0] == N
        rows_in = [np.array(x[r], copy=True) for r in range(N)]
        rows_out = rows_in if in_place else [np.zeros_like(x[r]) for r in range(N)]
        keep.append((rows_in, rows_out))
        for r in range(N):
            send_ptrs[w * N + r] = rows_in[r].ctypes.data
            recv_ptrs[w * N + r] = rows_out[r].ctypes.data
        outs.append(rows_out)
    carr = (ctypes.c_size_t * len(counts))(*counts)
    stats = Stats()
    cap = 0
    log = None
    if log_calls:
        cap = 1 << 20
        log = (Call * cap)()
    if threads is not None:
        assert not log_calls, "the channel-parallel mode keeps no call log"
        sched, seed = 2, int(threads)
    options = (1 if drop_recv_head else 0) | (2 if direct else 0) | (4 if ll_wrap8 else 0) | \
        (16 if direct_read else 0) | (RED[op] << 8)
    flat = [r for ring in rings for r in ring]
    assert all(len(ring) == N for ring in rings)
    if op == "premulsum":
        sc = np.ascontiguousarray(scalars).reshape(len(works), N)
        rc = lib().orc_allreduce_premul(N, len(rings), _ints(flat), mask, PROTO[proto], buff_size,
                                        chunk_steps, DTYPE[dtype], len(works), carr, send_ptrs,
                                        recv_ptrs, sc.ctypes.data, slots, sched, seed, options,
                                        ctypes.byref(stats), log, cap)
    else:
        rc = lib().orc_allreduce_rings(N, len(rings), _ints(flat), mask, PROTO[proto], buff_size,
                                       chunk_steps, DTYPE[dtype], len(works), carr, send_ptrs,
                                       recv_ptrs, slots, sched, seed, options, ctypes.byref(stats),
                                       log, cap)
    calls = []
    if log_calls:
        for c in log[:stats.calls_recorded]:
            calls.append(dict(rank=c.rank, channel_id=c.channel_id, work=c.work, op=OPS[c.op],
                              chunk=c.chunk, loop=c.loop, offset=c.offset, nelem=c.nelem))
    outputs = [np.stack(rows_out) for (_, rows_out) in keep]
    return rc, outputs, stats, calls


def stream_fault(proto, fault, slots, nsteps=64):
    """Single-connector fault model; returns (outcome, steps_done, consumed, bad_step)."""
    done, cons, bad = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    rc = lib().orc_stream_fault(PROTO[proto], FAULTS[fault], slots, nsteps, ctypes.byref(done),
                                ctypes.byref(cons), ctypes.byref(bad))
    name = {OK: "complete", DEADLOCK: "deadlock", CORRUPT: "corrupt", INVALID: "invalid"}[rc]
    return name, done.value, cons.value, bad.value


def ll_wrap(flag_bits, cleanup, slots, cap, lines_of, nsteps):
    """LL flag-generation model of one connector; returns (outcome, bad_step)."""
    bad = ctypes.c_int64()
    rc = lib().orc_ll_wrap(flag_bits, int(cleanup), slots, cap, len(lines_of), _ints(lines_of),
                           nsteps, ctypes.byref(bad))
    name = {OK: "complete", DEADLOCK: "deadlock", CORRUPT: "corrupt", INVALID: "invalid"}[rc]
    return name, bad.value


def bf16_round(v: float) -> int:
    return int(lib().orc_bf16_round(float(v)))
