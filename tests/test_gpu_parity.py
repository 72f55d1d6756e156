"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer and floating results must match bit for bit: the kernel follows the
same ring fold order as the oracle, so max-abs error is 0 by construction and
any difference is a bug.  Small cases compare against the state-machine
simulator; full-size workloads compare every element against the oracle's
closed form (int32: against the plain sum)."""
import numpy as np
import pytest

import oracle
from oracle import closed_form as cf
from ring_all_reduce_channelmask_amd import workloads as wl

from .gpu_util import assert_bits_equal, run_hip

pytestmark = pytest.mark.gpu

SMALL_BUFF = {"SIMPLE": 8 * 1024, "LL": 8 * 512, "LL128": 8 * 2048}


def _comm(**kw):
    import ring_all_reduce_channelmask_amd as rar
    return rar.Comm(**kw)


def _rand(dtype, shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    if dtype == "int32":
        return rng.integers(-2 ** 31, 2 ** 31, size=shape).astype(np.int32)
    v = (rng.standard_normal(shape) * scale).astype(np.float32)
    if dtype == "float32":
        return v
    return wl._bf16_bits(v.ravel()).reshape(shape)


def _check_vs_sim(comm, inputs, dtype, buff, cs, in_place=False, sched=0):
    got = run_hip(comm, inputs, dtype, in_place=in_place)
    rc, want, _, _ = oracle.allreduce(inputs, comm.rings, comm.mask, comm.proto, buff, cs,
                                      dtype, sched=sched)
    assert rc == oracle.OK
    for w in range(len(inputs)):
        assert_bits_equal(got[w], want[w], f"work {w}")


SMALL = []
for proto in ("SIMPLE", "LL", "LL128"):
    for dtype in ("float32", "bfloat16", "int32"):
        for (N, order, mask, count) in [(2, [1, 0], 0x1, 1), (3, [2, 0, 1], 0x5, 1001),
                                        (4, [0, 2, 3, 1], 0xF, 65539),
                                        (8, [0, 3, 1, 6, 2, 7, 5, 4], 0x3, 40000)]:
            SMALL.append((proto, dtype, N, order, mask, count))


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[0]}-{c[1]}-N{c[2]}-{c[5]}" for c in SMALL])
def test_small_vs_simulator(case):
    proto, dtype, N, order, mask, count = case
    buff = SMALL_BUFF[proto]
    comm = _comm(nranks=N, ring_order=order, mask=mask, proto=proto, buff_size=buff,
                 chunk_steps=4 if proto == "SIMPLE" else 0, lanes=2, waves=4)
    x = _rand(dtype, (N, count), count + N)
    _check_vs_sim(comm, [x], dtype, buff, 4)
    comm.close()


@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
def test_in_place_equals_out_of_place(proto):
    buff = SMALL_BUFF[proto]
    comm = _comm(nranks=4, ring_order=[0, 2, 3, 1], mask=0x7, proto=proto, buff_size=buff,
                 chunk_steps=2 if proto == "SIMPLE" else 0)
    x = _rand("float32", (4, 30011), 5)
    _check_vs_sim(comm, [x], "float32", buff, 2, in_place=True)
    _check_vs_sim(comm, [x], "float32", buff, 2, in_place=False)
    comm.close()


@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
def test_lanes_and_waves_do_not_change_bits(proto):
    """Lanes split slices across workgroups and waves across threads; the
    result bits must not depend on either."""
    buff = SMALL_BUFF[proto] * 4
    x = _rand("bfloat16", (4, 100003), 6)
    ref = None
    for lanes, waves in [(1, 1), (1, 8), (3, 2), (4, 4), (8, 8)]:
        comm = _comm(nranks=4, ring_order=[0, 2, 3, 1], mask=0xA, proto=proto, buff_size=buff,
                     lanes=lanes, waves=waves)
        got = run_hip(comm, [x], "bfloat16")[0]
        comm.close()
        if ref is None:
            rc, want, _, _ = oracle.allreduce([x], [0, 2, 3, 1], 0xA, proto, buff, 4, "bfloat16")
            assert rc == oracle.OK
            assert_bits_equal(got, want[0], f"lanes {lanes} waves {waves}")
            ref = got
        assert_bits_equal(got, ref, f"lanes {lanes} waves {waves}")


@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
def test_edge_counts(proto):
    """Empty and tiny inputs: count 0 launches nothing and moves no step;
    8 elements over 8 ranks leave most chunks empty (empty slices post)."""
    import torch
    buff = SMALL_BUFF[proto]
    comm = _comm(nranks=8, ring_order=list(range(8)), mask=0x3, proto=proto, buff_size=buff)
    before = comm.query_state()
    t = [torch.zeros(0, device="cuda") for _ in range(8)]
    comm.allreduce(t, [torch.zeros(0, device="cuda") for _ in range(8)])
    torch.cuda.synchronize()
    assert comm.query_state() == before
    for count in (1, 3, 8, 17, 64, 129):
        x = np.random.default_rng(count).integers(-8, 9, size=(8, count)).astype(np.float32)
        got = run_hip(comm, [x], "float32")[0]
        for r in range(8):
            np.testing.assert_array_equal(got[r], x.sum(axis=0))
    comm.close()


def test_subnormal_and_signed_zero_fp32_bf16():
    """IEEE behaviour without flush-to-zero: subnormal sums and -0.0."""
    rng = np.random.default_rng(8)
    f = (rng.standard_normal((4, 4096)) * 2.0 ** -140).astype(np.float32)
    f[:, :16] = -0.0
    comm = _comm(nranks=4, ring_order=[0, 1, 2, 3], mask=0x1, proto="SIMPLE",
                 buff_size=SMALL_BUFF["SIMPLE"])
    _check_vs_sim(comm, [f], "float32", SMALL_BUFF["SIMPLE"], 4)
    b = wl._bf16_bits((rng.standard_normal(4 * 4096) * 2.0 ** -128).astype(np.float32))
    _check_vs_sim(comm, [b.reshape(4, 4096)], "bfloat16", SMALL_BUFF["SIMPLE"], 4)
    comm.close()


@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
def test_many_launches_on_one_comm(proto):
    """Steps persist across launches (monotonic head/tail/flags, no reset):
    1000 back-to-back collectives of varying size on one communicator, so
    slots and LL flag generations wrap many times over."""
    import torch
    buff = SMALL_BUFF[proto]
    comm = _comm(nranks=4, ring_order=[0, 2, 3, 1], mask=0x3, proto=proto, buff_size=buff,
                 lanes=2, waves=2)
    x = np.random.default_rng(9).integers(-1000, 1000, size=(4, 3001)).astype(np.int32)
    from .gpu_util import to_device, to_host
    sends = [to_device(x[r], "int32") for r in range(4)]
    recvs = [torch.zeros_like(s) for s in sends]
    sizes = [3001, 1, 2048, 777, 0, 3000]
    for i in range(1000):
        n = sizes[i % len(sizes)]
        comm.allreduce([s[:n] for s in sends], [r[:n] for r in recvs])
    torch.cuda.synchronize()
    assert comm.async_error() == 0
    n = sizes[999 % len(sizes)]
    for r in range(4):
        np.testing.assert_array_equal(to_host(recvs[r], "int32")[:n], x[:, :n].sum(axis=0))
    got = run_hip(comm, [x], "int32")[0]
    for r in range(4):
        np.testing.assert_array_equal(got[r], x.sum(axis=0))
    comm.close()


def test_group_fused_and_chained_batches():
    """Fused works over a sparse mask; 300 works give more than 16 pieces per
    channel, so batches chain through next_jump."""
    mask = 0b101101010011
    comm = _comm(nranks=4, ring_order=[0, 1, 2, 3], mask=mask, proto="LL")
    xs = [_rand("bfloat16", (4, c), 50 + i) for i, c in enumerate([7168] * 8 + [1, 5, 4096])]
    _check_vs_sim(comm, xs, "bfloat16", 512 * 1024, 4)
    xs = [_rand("float32", (4, 100 + 37 * i), 500 + i) for i in range(300)]
    _check_vs_sim(comm, xs, "float32", 512 * 1024, 4)
    comm.close()


def test_ring_allreduce_one_shot_entry():
    import ring_all_reduce_channelmask_amd as rar
    import torch
    from .gpu_util import to_device, to_host
    x = _rand("float32", (4, 50000), 12)
    sends = [to_device(x[r], "float32") for r in range(4)]
    recvs = [torch.empty_like(s) for s in sends]
    for _ in range(2):  # second call reuses the cached communicator
        rar.ring_allreduce(sends, recvs, [0, 2, 3, 1], proto="SIMPLE", nchannels=3,
                           buff_size=SMALL_BUFF["SIMPLE"], chunk_steps=4)
    torch.cuda.synchronize()
    rc, want, _, _ = oracle.allreduce([x], [0, 2, 3, 1], 0x7, "SIMPLE", SMALL_BUFF["SIMPLE"], 4,
                                      "float32")
    for r in range(4):
        assert_bits_equal(to_host(recvs[r], "float32"), want[0][r], f"rank {r}")


def test_dropped_head_credit_stalls_after_nccl_steps_and_watchdog_ends_it():
    """The pages' fault model on the real kernel (Course 23, "状态机故障注入":
    dropping recv head deadlocks after exactly NCCL_STEPS slots), forced from
    the host by a test flag.  Every sender lane stops with tail = 8 and head =
    0, the kernel's bounded waits give up after 2 ms, every workgroup exits,
    the communicator reports RAR_ABORTED, and a fresh one still works."""
    import ring_all_reduce_channelmask_amd as rar
    import torch
    from ring_all_reduce_channelmask_amd import _lib
    from .gpu_util import to_device
    comm = _comm(nranks=4, ring_order=[0, 1, 2, 3], mask=0x3, proto="SIMPLE",
                 buff_size=SMALL_BUFF["SIMPLE"], lanes=2, waves=2, timeout_us=2000,
                 debug_flags=1)
    x = _rand("float32", (4, 1 << 16), 13)
    sends = [to_device(x[r], "float32") for r in range(4)]
    recvs = [torch.empty_like(s) for s in sends]
    comm.allreduce(sends, recvs)
    torch.cuda.synchronize()
    assert comm.async_error() == _lib.ABORTED
    state = comm.query_state()
    tails, heads = state[0::2], state[1::2]
    assert len(tails) == 4 * 2 * 2
    assert set(tails) == {8} and set(heads) == {0}
    with pytest.raises(rar.RarError) as e:
        comm.allreduce(sends, recvs)
    assert e.value.code == _lib.ABORTED
    comm.close()
    fresh = _comm(nranks=4, ring_order=[0, 1, 2, 3], mask=0x3, proto="SIMPLE",
                  buff_size=SMALL_BUFF["SIMPLE"])
    _check_vs_sim(fresh, [x[:, :5000].copy()], "float32", SMALL_BUFF["SIMPLE"], 4)
    fresh.close()


@pytest.mark.parametrize("proto", ["LL", "LL128"])
def test_dropped_head_stalls_ll_protocols_after_nccl_steps(proto):
    """The same fault in the flag protocols: with receivers never handing
    slots back, every workgroup completes exactly NCCL_STEPS sending units
    (the timeline records one per completed unit; the loop's final receive
    sends nothing) and then waits for credit that never comes; the bounded
    waits end the launch with RAR_ABORTED."""
    import ring_all_reduce_channelmask_amd as rar
    import torch
    from ring_all_reduce_channelmask_amd import _lib
    from .gpu_util import to_device
    comm = _comm(nranks=4, ring_order=[0, 2, 3, 1], mask=0x3, proto=proto,
                 buff_size=SMALL_BUFF[proto], lanes=2, waves=2, timeout_us=2000,
                 debug_flags=_lib.DEBUG_DROP_RECV_HEAD | _lib.DEBUG_TRACE)
    x = _rand("float32", (4, 1 << 16), 14)
    sends = [to_device(x[r], "float32") for r in range(4)]
    recvs = [torch.empty_like(s) for s in sends]
    comm.allreduce(sends, recvs)
    torch.cuda.synchronize()
    assert comm.async_error() == _lib.ABORTED
    sending = {}
    for rec in comm.read_trace():
        key = (rec["rank"], rec["channel_id"], rec["lane"])
        sending[key] = sending.get(key, 0) + (rec["op"] != 4)  # 4 = recv
    assert len(sending) == 4 * 2 * 2
    assert set(sending.values()) == {8}
    assert set(comm.query_state()[1::2]) == {0}
    with pytest.raises(rar.RarError) as e:
        comm.allreduce(sends, recvs)
    assert e.value.code == _lib.ABORTED
    comm.close()


# ------------------------------------------------------------- full sizes
def _bench_tuning():
    import bench  # the launch shapes bench.py times
    return bench.TUNING


@pytest.mark.parametrize("key", list(wl.WORKLOADS))
def test_workload_full_size(key):
    """Every workload at its full size; the 64 MiB Simple case in the launch
    configuration the benchmark times.  Compared element by element with the
    oracle's closed form (int32 with the plain sum)."""
    w = wl.WORKLOADS[key]
    xs = wl.inputs_for(w)
    tune = _bench_tuning().get(key, {})
    comm = _comm(nranks=w.nranks, ring_order=list(w.ring_order), mask=w.mask, proto=w.proto,
                 buff_size=w.buff_size, chunk_steps=w.chunk_steps if w.proto == "SIMPLE" else 0,
                 **tune)
    got = run_hip(comm, xs, w.dtype)
    comm.close()
    want = cf.allreduce(xs, list(w.ring_order), w.mask, w.proto, w.buff_size, w.chunk_steps,
                        w.dtype)
    for i in range(len(xs)):
        if w.dtype == "int32":
            s = (xs[i].astype(np.int64).sum(axis=0) & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
            np.testing.assert_array_equal(want[i], s)
        for r in range(w.nranks):
            assert_bits_equal(got[i][r], want[i], f"{key} work {i} rank {r}")
    if w.dtype != "int32":
        # max-abs error against the oracle is exactly zero
        diff = max(float(np.max(np.abs(cf._to_f64(got[i][0], w.dtype) -
                                       cf._to_f64(want[i], w.dtype)))) for i in range(len(xs)))
        assert diff == 0.0


@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_ranks_spread_over_xcds(proto, dtype):
    """Placement 1 puts the ranks of every (channel, lane) pipeline on
    different XCDs, so every hop crosses L2s and the publication must take
    the agent-scope release; results must not change."""
    buff = SMALL_BUFF[proto] * 2
    comm = _comm(nranks=4, ring_order=[0, 2, 3, 1], mask=0xF, proto=proto, buff_size=buff,
                 lanes=2, waves=4, placement=1)
    x = _rand(dtype, (4, 120001), 21)
    _check_vs_sim(comm, [x], dtype, buff, 4)
    comm.close()


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
@pytest.mark.parametrize("spc", [1, 4])
def test_slices_per_chunk_same_bits(dtype, spc):
    """Slicing is timing only: 1 slice of 4 steps or 4 slices of 1 step give
    the same bits as the oracle's 2 slices of 2 steps (every call still
    consumes 4 steps)."""
    buff = SMALL_BUFF["SIMPLE"] * 4
    comm = _comm(nranks=4, ring_order=[0, 2, 3, 1], mask=0x7, proto="SIMPLE", buff_size=buff,
                 chunk_steps=4, lanes=3, waves=4, slices_per_chunk=spc)
    x = _rand(dtype, (4, 200003), 31)
    _check_vs_sim(comm, [x], dtype, buff, 4)
    comm.close()


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("placement", [0, 1])
def test_direct_variant_vs_oracle(dtype, in_place, placement):
    """Direct all-gather (into the next rank's receive buffer) against the
    oracle's direct simulation and its FIFO simulation: same bits; with the
    ranks spread over XCDs the direct writes need the write-back publication."""
    buff = SMALL_BUFF["SIMPLE"] * 2
    comm = _comm(nranks=4, ring_order=[0, 2, 3, 1], mask=0x5, proto="SIMPLE", buff_size=buff,
                 lanes=3, waves=4, direct=1, placement=placement)
    x = _rand(dtype, (4, 150011), 41)
    got = run_hip(comm, [x], dtype, in_place=in_place)[0]
    comm.close()
    for direct in (True, False):
        rc, want, _, _ = oracle.allreduce([x], [0, 2, 3, 1], 0x5, "SIMPLE", buff, 4, dtype,
                                          direct=direct)
        assert rc == oracle.OK
        assert_bits_equal(got, want[0], f"direct={direct}")


def test_direct_variant_full_size_and_many_launches():
    """The 64 MiB workload with the direct variant, bit for bit against the
    closed form, then 200 back-to-back launches of a small one on one comm."""
    import torch
    from .gpu_util import to_device, to_host
    w = wl.WORKLOADS["simple_64m"]
    xs = wl.inputs_for(w)
    comm = _comm(nranks=4, ring_order=list(w.ring_order), mask=w.mask, proto="SIMPLE",
                 buff_size=w.buff_size, chunk_steps=4, lanes=5, waves=8, direct=1, launch_mode=1)
    got = run_hip(comm, xs, "float32")[0]
    want = cf.allreduce(xs, list(w.ring_order), w.mask, "SIMPLE", w.buff_size, 4, "float32")[0]
    for r in range(4):
        assert_bits_equal(got[r], want, f"rank {r}")
    x = np.random.default_rng(3).integers(-1000, 1000, size=(4, 77777)).astype(np.int32)
    sends = [to_device(x[r], "int32") for r in range(4)]
    recvs = [torch.zeros_like(s) for s in sends]
    for _ in range(200):
        comm.allreduce(sends, recvs)
    torch.cuda.synchronize()
    assert comm.async_error() == 0
    for r in range(4):
        np.testing.assert_array_equal(to_host(recvs[r], "int32"), x.sum(axis=0))
    comm.close()


def test_direct_variant_rejected_for_ll():
    import ring_all_reduce_channelmask_amd as rar
    from ring_all_reduce_channelmask_amd import _lib
    for proto in ("LL", "LL128"):
        with pytest.raises(rar.RarError) as e:
            _comm(nranks=4, ring_order=[0, 1, 2, 3], mask=1, proto=proto, direct=1)
        assert e.value.code == _lib.UNSUPPORTED


# ------------------------------------------------- per-channel rings
def _graph(key):
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "graph_rings.json")) as f:
        return json.load(f)[key]


@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
@pytest.mark.parametrize("key", ["n4", "n3"])
def test_per_channel_rings_vs_simulator(proto, dtype, key):
    """The graph layouts of the course page: every channel id runs its own
    ring, the base rings repeat over the later channels; the per-channel fold
    order must match the simulator bit for bit."""
    g = _graph(key)
    N = len(g["base"][0])
    buff = SMALL_BUFF[proto]
    comm = _comm(nranks=N, ring_order=g["base"], mask=(1 << g["channels"]) - 1, proto=proto,
                 buff_size=buff, chunk_steps=4 if proto == "SIMPLE" else 0, lanes=2, waves=4)
    x = _rand(dtype, (N, 90017), 51 + N)
    _check_vs_sim(comm, [x], dtype, buff, 4)
    comm.close()


def test_per_channel_rings_follow_channel_id_not_dense_index():
    """With a sparse mask, channel id c (not the c-th active channel) picks
    ring c mod nrings; mask 0b1010_1010 under three rings runs rings
    1, 0, 2, 1 on channels 1, 3, 5, 7."""
    rings = [[0, 1, 2, 3], [0, 3, 2, 1], [0, 2, 1, 3]]
    buff = SMALL_BUFF["SIMPLE"]
    comm = _comm(nranks=4, ring_order=rings, mask=0xAA, proto="SIMPLE", buff_size=buff,
                 lanes=2, waves=4)
    x = _rand("float32", (4, 70001), 61)
    got = run_hip(comm, [x], "float32")[0]
    comm.close()
    want = cf.allreduce([x], rings, 0xAA, "SIMPLE", buff, 4, "float32")[0]
    for r in range(4):
        assert_bits_equal(got[r], want, f"rank {r}")
    dense = cf.allreduce([x], [rings[(1 + 2 * n) % 3] for n in range(4)] * 16, 0xF, "SIMPLE",
                         buff, 4, "float32")[0]
    assert not np.array_equal(dense, cf.allreduce([x], [rings[n % 3] for n in range(4)] * 16,
                                                  0xF, "SIMPLE", buff, 4, "float32")[0])
    assert_bits_equal(got[0], dense, "channel ids 1,3,5,7 = rings 1,0,2,1")


@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_per_channel_rings_full_size_direct_and_spread(dtype):
    """The six four-rank rings over 12 channels at the benchmark's 64 MiB
    size, with the direct all-gather and with the ranks spread over XCDs,
    every element against the closed form."""
    g = _graph("n4")
    count = 16 << 20 if dtype == "float32" else 32 << 20
    x = _rand(dtype, (4, count), 71)
    want = cf.allreduce([x], g["base"], 0xFFF, "SIMPLE", 4 << 20, 4, dtype)[0]
    for kw in (dict(direct=1), dict(placement=1)):
        comm = _comm(nranks=4, ring_order=g["base"], mask=0xFFF, proto="SIMPLE",
                     buff_size=4 << 20, chunk_steps=4, lanes=5, waves=8, launch_mode=1, **kw)
        got = run_hip(comm, [x], dtype)[0]
        comm.close()
        for r in range(4):
            assert_bits_equal(got[r], want, f"{kw} rank {r}")


# ------------------------------------------------- LL flag wrap test mode
@pytest.mark.parametrize("lanes", [1, 3])
def test_ll_flag_wrap_mode_over_many_wraps(lanes):
    """LL with 8-bit flags (debug bit 2): launches of varying size on one
    communicator carry every connector through several wraps of the flag and
    several slot cleanups; every launch matches the closed form."""
    import ring_all_reduce_channelmask_amd as rar
    buff = SMALL_BUFF["LL"]
    comm = _comm(nranks=4, ring_order=[0, 2, 3, 1], mask=0x3, proto="LL", buff_size=buff,
                 lanes=lanes, waves=2, debug_flags=rar._lib.DEBUG_LL_FLAG_WRAP8)
    rng = np.random.default_rng(lanes)
    for i, count in enumerate([20011, 7, 40000, 333, 61111, 1, 25000]):
        x = _rand("float32", (4, count), 100 + i)
        got = run_hip(comm, [x], "float32")[0]
        want = cf.allreduce([x], [0, 2, 3, 1], 0x3, "LL", buff, 4, "float32")[0]
        for r in range(4):
            assert_bits_equal(got[r], want, f"launch {i} rank {r}")
    steps = comm.query_state()
    assert min(steps[1::2]) > 4 * 256, "each connector should have crossed several wraps"
    comm.close()


# ------------------------------------------------- direct read
@pytest.mark.parametrize("direct", [2, 3])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("N", [2, 3, 5])
def test_direct_read_vs_oracle(direct, dtype, in_place, N):
    """Direct read (bit 1), alone and with the direct write: the loop's first
    receive reads the previous rank's send buffer.  N = 2 takes it in the
    fused final step, N > 2 in the first recvReduceSend.  Same bits as the
    oracle's direct simulation and its FIFO simulation."""
    order = [[1, 0], [2, 0, 1], [0, 3, 1, 4, 2]][[2, 3, 5].index(N)]
    buff = SMALL_BUFF["SIMPLE"] * 2
    comm = _comm(nranks=N, ring_order=order, mask=0x5, proto="SIMPLE", buff_size=buff,
                 lanes=3, waves=4, direct=direct)
    x = _rand(dtype, (N, 150011), 61 + N)
    got = run_hip(comm, [x], dtype, in_place=in_place)[0]
    comm.close()
    for kw in (dict(direct=bool(direct & 1), direct_read=True), dict()):
        rc, want, _, _ = oracle.allreduce([x], order, 0x5, "SIMPLE", buff, 4, dtype, **kw)
        assert rc == oracle.OK
        for r in range(N):
            assert_bits_equal(got[r], want[0][r], f"{kw} rank {r}")


@pytest.mark.parametrize("placement", [0, 1])
def test_direct_read_write_full_size_and_many_launches(placement):
    """64 MiB with both direct variants in the benchmark's launch shape, 100
    launches on one communicator, every element against the closed form."""
    import torch
    import ring_all_reduce_channelmask_amd as rar
    from .gpu_util import to_device, to_host
    w = wl.WORKLOADS["simple_64m"]
    x = wl.inputs_for(w)[0]
    tune = dict(_bench_tuning()["simple_64m"])
    tune.update(direct=3, placement=placement)
    comm = _comm(nranks=4, ring_order=list(w.ring_order), mask=w.mask, proto="SIMPLE",
                 buff_size=w.buff_size, chunk_steps=4, **tune)
    sends = [to_device(x[r], "float32") for r in range(4)]
    recvs = [torch.empty_like(t) for t in sends]
    for _ in range(100):
        comm.allreduce(sends, recvs)
    torch.cuda.synchronize()
    assert comm.async_error() == 0
    comm.close()
    want = cf.allreduce([x], list(w.ring_order), w.mask, "SIMPLE", w.buff_size, 4, "float32")[0]
    for r in range(4):
        assert_bits_equal(to_host(recvs[r], "float32"), want, f"rank {r}")


# ------------------------------------------------- works dealt to lanes
@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
def test_dealt_works_vs_simulator(proto, dtype):
    """Lanes that take a channel's works in turn instead of splitting every
    step: a fused group over a sparse mask with a work count that is not a
    multiple of the lanes, ragged sizes, a single work (one lane busy, the
    others idle), and a group long enough to chain batches.  Same bits as the
    simulator, launch after launch on one communicator."""
    mask = 0b1011
    buff = SMALL_BUFF[proto]
    cs = 4 if proto == "SIMPLE" else 0
    comm = _comm(nranks=4, ring_order=[0, 2, 3, 1], mask=mask, proto=proto, buff_size=buff,
                 chunk_steps=cs, lanes=3, waves=2, deal_works=1)
    groups = [
        [_rand(dtype, (4, c), 700 + i) for i, c in enumerate([5000, 1, 777, 3001, 64, 9999, 17])],
        [_rand(dtype, (4, 20011), 720)],
        [_rand(dtype, (4, 50 + 13 * i), 730 + i) for i in range(70)],
    ]
    for xs in groups + groups[:1]:
        _check_vs_sim(comm, xs, dtype, buff, 4)
    comm.close()


@pytest.mark.parametrize("placement", [0, 1])
def test_dealt_works_with_direct_ops_and_in_place(placement):
    """Dealt works under the Simple direct variants, a non-sum operator and in
    place, with ranks spread over XCDs or not."""
    buff = SMALL_BUFF["SIMPLE"]
    xs = [_rand("float32", (4, c), 760 + i) for i, c in enumerate([4099, 12000, 5, 800, 2500])]
    for direct in (0, 1, 3):
        comm = _comm(nranks=4, ring_order=[1, 3, 0, 2], mask=0x6, proto="SIMPLE", buff_size=buff,
                     chunk_steps=4, lanes=2, waves=4, deal_works=1, direct=direct,
                     placement=placement)
        got = run_hip(comm, xs, "float32", in_place=True)
        want = cf.allreduce(xs, [1, 3, 0, 2], 0x6, "SIMPLE", buff, 4, "float32")
        for i in range(len(xs)):
            for r in range(4):
                assert_bits_equal(got[i][r], want[i], f"direct {direct} work {i} rank {r}")
        got = run_hip(comm, xs, "float32", op="max")
        want = cf.allreduce(xs, [1, 3, 0, 2], 0x6, "SIMPLE", buff, 4, "float32", op="max")
        for i in range(len(xs)):
            for r in range(4):
                assert_bits_equal(got[i][r], want[i], f"max direct {direct} work {i} rank {r}")
        comm.close()


# ------------------------------------------------- the maxima
@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
def test_maximum_ranks_and_channels(proto, dtype):
    """64 ranks on a random ring over the first and last channel ids, and 2
    ranks over all 64 channels, in a ragged group; bit for bit with the
    closed form (int32 also with the plain wrapped sum)."""
    buff = SMALL_BUFF[proto]
    cs = 4 if proto == "SIMPLE" else 0
    rng = np.random.default_rng(64)
    order = [int(v) for v in rng.permutation(64)]
    for N, ring, mask, counts in ((64, order, (1 << 63) | 1, [1, 5003, 64 * 37 + 3]),
                                  (2, [1, 0], (1 << 64) - 1, [100003, 7])):
        comm = _comm(nranks=N, ring_order=ring, mask=mask, proto=proto, buff_size=buff,
                     chunk_steps=cs, lanes=1, waves=2)
        xs = [_rand(dtype, (N, c), 640 + c) for c in counts]
        got = run_hip(comm, xs, dtype)
        comm.close()
        want = cf.allreduce(xs, ring, mask, proto, buff, 4, dtype)
        for i, x in enumerate(xs):
            if dtype == "int32":
                s = (x.astype(np.int64).sum(axis=0) & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
                np.testing.assert_array_equal(want[i], s)
            for r in range(N):
                assert_bits_equal(got[i][r], want[i], f"N {N} work {i} rank {r}")



@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128", "oneshot"])
def test_more_than_2g_elements(proto):
    """A collective of 2^31 + 5 int32 elements (8 GiB per buffer) over 64
    channels, so element offsets, channel offsets and byte offsets all pass
    2^31.  int32 sums wrap, so the result does not depend on the fold order:
    every element is checked on the device against the plain wrapped sum."""
    import torch
    count, block = (1 << 31) + 5, 1 << 27
    sends = [torch.empty(count, dtype=torch.int32, device="cuda") for _ in range(2)]
    want = torch.empty(count, dtype=torch.int32, device="cuda")
    for lo in range(0, count, block):
        i = torch.arange(lo, min(lo + block, count), dtype=torch.int64, device="cuda")
        x0 = (i * 2654435761 + 12345) & 0xFFFFFFFF
        x1 = (i * 40503 + 977) & 0xFFFFFFFF
        wrap = lambda v: torch.where(v >= 1 << 31, v - (1 << 32), v).to(torch.int32)
        sends[0][lo:lo + i.numel()] = wrap(x0)
        sends[1][lo:lo + i.numel()] = wrap(x1)
        want[lo:lo + i.numel()] = wrap((x0 + x1) & 0xFFFFFFFF)
    del i, x0, x1
    recvs = [torch.empty_like(s) for s in sends]
    if proto == "oneshot":
        import ring_all_reduce_channelmask_amd as rar
        rar.oneshot_allreduce(sends, recvs)
        torch.cuda.synchronize()
    else:
        comm = _comm(nranks=2, ring_order=[1, 0], mask=(1 << 64) - 1, proto=proto, launch_mode=1)
        comm.allreduce(sends, recvs)
        torch.cuda.synchronize()
        assert comm.async_error() == 0
        comm.close()
    for r in range(2):
        assert torch.equal(recvs[r], want), f"rank {r}"


@pytest.mark.parametrize("dtype", ["int32", "float32", "bfloat16"])
@pytest.mark.parametrize("op", ["sum", "prod", "avg", "premulsum"])
def test_ll128_benchmark_shape_every_dtype_and_operator(dtype, op):
    """LL128 in the launch shape the benchmark uses (16 lanes x 4 waves over
    12 channels: 768 workgroups, three per CU, possible because the LL128
    kernels keep to three waves' registers per SIMD; fp32 and int32 spill a
    few registers),
    for every payload type and the operators with the heaviest kernels, on
    a ragged 3-collective group, bit for bit against the closed form."""
    rng = np.random.default_rng([["int32", "float32", "bfloat16"].index(dtype),
                                 ["sum", "prod", "avg", "premulsum"].index(op)])
    import bench
    tune = dict(bench.TUNING["ll128_64m"])
    assert (tune["lanes"], tune["waves"]) == (16, 4)
    comm = _comm(nranks=4, ring_order=[0, 2, 3, 1], mask=0xFFF, proto="LL128", **tune)
    counts = [1 << 20, 123457, 5]
    if dtype == "int32":
        xs = [rng.integers(-2 ** 31, 2 ** 31, size=(4, c)).astype(np.int32) for c in counts]
    else:
        xs = [_rand(dtype, (4, c), int(rng.integers(1 << 20))) for c in counts]
    scs = [_rand(dtype, (4,), 7 + i) for i in range(len(counts))] if op == "premulsum" else None
    if scs is not None and dtype == "int32":
        scs = [rng.integers(-9, 10, size=4).astype(np.int32) for _ in counts]
    got = run_hip(comm, xs, dtype, op=op, scalars=scs)
    comm.close()
    want = cf.allreduce(xs, [0, 2, 3, 1], 0xFFF, "LL128", 4915200, 4, dtype, op=op,
                        scalars=None if scs is None else np.stack(scs))
    for i in range(len(xs)):
        for r in range(4):
            assert_bits_equal(got[i][r], want[i], f"{dtype} {op} work {i} rank {r}")


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
@pytest.mark.parametrize("waves", [1, 3, 8])
@pytest.mark.parametrize("extra", [0, 1, 13])
def test_ll128_iteration_boundaries(dtype, waves, extra):
    """LL128 receivers wait for one flag per wave iteration (U groups of 8
    lines: U = 4 for 4-byte payloads, 3 for bf16) and then read that
    iteration's lines.  A lane's step holds two whole iterations of every
    wave plus `extra` lines (none, one, or a partial group), over one and two
    lanes, and the runRing tail loop cuts a smaller chunk; every result bit
    matches the simulator."""
    U = 3 if dtype == "bfloat16" else 4
    es = 2 if dtype == "bfloat16" else 4
    lines = 2 * 8 * waves * U + extra
    for lanes in (1, 2):
        # a lane's slot is a whole number of 256-byte units: size the buffer
        # so that each lane's step holds `lines` lines
        lane_step = 256 * -(-lines * 128 // 256)
        buff = 8 * lanes * lane_step
        chunk_bytes = lanes * lines * 120
        count = (4 * chunk_bytes + 4 * chunk_bytes // 2) // es + 7
        x = _rand(dtype, (4, count), 100 + waves + extra + lanes)
        comm = _comm(nranks=4, ring_order=[0, 2, 3, 1], mask=0x1, proto="LL128", buff_size=buff,
                     lanes=lanes, waves=waves)
        _check_vs_sim(comm, [x], dtype, buff, 4)
        comm.close()
