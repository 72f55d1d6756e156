"""Parity of the strict-scope publication mode, of per-work wave counts, and
of launches that reuse a cached launch plan, against the oracle.

* strict_scope = 1 publishes Simple tails, LL lines and LL128 flags at agent
  scope with the release even to a receiver on the same XCD: the fallback
  should the same-L2 path stop holding.  Full-size parity at the 64 MiB
  workloads (4 ranks Simple and LL128; 8 ranks bf16 and int32) in the launch
  shapes the benchmark times, plus small cases of every protocol and dtype.
* waves_by_size = 1 gives the small works of a group fewer waves, so one
  batch mixes wave counts and RunWorkBatch fences every change with a
  barrier; the per-unit trace shows the mix.
* A communicator keeps the last launch plan; launches that change pointers,
  counts, operator or group composition must not reuse it."""
import numpy as np
import pytest

import oracle
from oracle import closed_form as cf
from ring_all_reduce_channelmask_amd import workloads as wl

from .gpu_util import assert_bits_equal, run_hip, to_device, to_host

pytestmark = pytest.mark.gpu

SMALL_BUFF = {"SIMPLE": 8 * 1024, "LL": 8 * 512, "LL128": 8 * 2048}


def _rand(dtype, shape, seed):
    rng = np.random.default_rng(seed)
    if dtype == "int32":
        return rng.integers(-2 ** 31, 2 ** 31, size=shape).astype(np.int32)
    v = rng.standard_normal(shape).astype(np.float32)
    return v if dtype == "float32" else wl._bf16_bits(v.ravel()).reshape(shape)


def _comm(**kw):
    import ring_all_reduce_channelmask_amd as rar
    return rar.Comm(**kw)


# ------------------------------------------------------------ strict scope
@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
def test_strict_scope_small_vs_simulator(proto, dtype):
    buff = SMALL_BUFF[proto] * 2
    comm = _comm(nranks=4, ring_order=[0, 2, 3, 1], mask=0xF, proto=proto, buff_size=buff,
                 lanes=2, waves=4, strict_scope=1)
    xs = [_rand(dtype, (4, 90001), 31), _rand(dtype, (4, 333), 32)]
    got = run_hip(comm, xs, dtype)
    rc, want, _, _ = oracle.allreduce(xs, [0, 2, 3, 1], 0xF, proto, buff, 4, dtype)
    assert rc == oracle.OK
    for i in range(2):
        assert_bits_equal(got[i], want[i], f"work {i}")
    comm.close()


@pytest.mark.parametrize("key", ["simple_64m", "ll128_64m", "bf16_n8", "int32_n8"])
def test_strict_scope_full_size(key):
    import bench
    w = wl.WORKLOADS[key]
    xs = wl.inputs_for(w)
    comm = _comm(nranks=w.nranks, ring_order=list(w.ring_order), mask=w.mask, proto=w.proto,
                 buff_size=w.buff_size, chunk_steps=w.chunk_steps if w.proto == "SIMPLE" else 0,
                 strict_scope=1, **bench.TUNING[key])
    got = run_hip(comm, xs, w.dtype)
    comm.close()
    want = cf.allreduce(xs, list(w.ring_order), w.mask, w.proto, w.buff_size, w.chunk_steps,
                        w.dtype)
    for r in range(w.nranks):
        assert_bits_equal(got[0][r], want[0], f"{key} strict rank {r}")


# --------------------------------------------------------- waves by size
@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
@pytest.mark.parametrize("deal", [0, 1])
def test_mixed_wave_counts_in_one_batch(proto, deal):
    """A group whose works differ in size by orders of magnitude on the same
    channels: with waves_by_size the small ones run on fewer waves, so the
    batch mixes wave counts (seen in the trace), and the results are the
    oracle's."""
    import ring_all_reduce_channelmask_amd as rar
    from ring_all_reduce_channelmask_amd import _lib
    # buffers whose chunks fill all 8 waves for the large works
    buff = {"SIMPLE": 256 << 10, "LL": 256 << 10, "LL128": 8 * 2048 * 8}[proto]
    mask, order, dtype = 0b1011, [0, 2, 3, 1], "float32"
    comm = rar.Comm(4, order, mask, proto=proto, buff_size=buff, lanes=2, waves=8,
                    waves_by_size=1, deal_works=deal, debug_flags=_lib.DEBUG_TRACE)
    counts = [200003, 40, 7, 150001, 3, 90000, 64, 1]
    xs = [_rand(dtype, (4, c), 40 + i) for i, c in enumerate(counts)]
    got = run_hip(comm, xs, dtype)
    rc, want, _, _ = oracle.allreduce(xs, order, mask, proto, buff, 4, dtype)
    assert rc == oracle.OK
    for i in range(len(xs)):
        assert_bits_equal(got[i], want[i], f"{proto} work {i}")
    waves_seen = {}
    for rec in comm.read_trace():
        waves_seen.setdefault((rec["rank"], rec["channel_id"], rec["lane"]), set()).add(rec["waves"])
    assert max(len(v) for v in waves_seen.values()) >= 2, waves_seen
    assert all(1 <= x <= 8 for v in waves_seen.values() for x in v)
    comm.close()


def test_fused_group_full_size_with_waves_by_size():
    import bench
    w = wl.WORKLOADS["fused_ll"]
    xs = wl.inputs_for(w)
    comm = _comm(nranks=w.nranks, ring_order=list(w.ring_order), mask=w.mask, proto=w.proto,
                 buff_size=w.buff_size, waves_by_size=1, **bench.TUNING["fused_ll"])
    got = run_hip(comm, xs, w.dtype)
    comm.close()
    want = cf.allreduce(xs, list(w.ring_order), w.mask, w.proto, w.buff_size, w.chunk_steps, w.dtype)
    for i in range(len(xs)):
        for r in range(w.nranks):
            assert_bits_equal(got[i][r], want[i], f"work {i} rank {r}")


# ------------------------------------------------------------ plan cache
@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
def test_cached_plan_follows_pointer_count_and_operator_changes(proto):
    import torch
    buff = SMALL_BUFF[proto] * 2
    order, mask, dtype = [0, 2, 3, 1], 0xF, "float32"
    comm = _comm(nranks=4, ring_order=order, mask=mask, proto=proto, buff_size=buff, lanes=2,
                 waves=2, launch_mode=1)
    n1, n2 = 50001, 777
    A = [[to_device(r, dtype) for r in _rand(dtype, (4, n1), 51 + k)] for k in range(2)]
    out = [[torch.empty_like(t) for t in A[0]] for _ in range(2)]
    small = [to_device(r, dtype) for r in _rand(dtype, (4, n2), 60)]
    small_out = [torch.empty_like(t) for t in small]

    def check(sends, recvs, op="sum", what=""):
        torch.cuda.synchronize()
        x = np.stack([to_host(t, dtype) for t in sends])
        want = cf.allreduce([x], order, mask, proto, buff, 4, dtype, op=op)[0]
        for r in range(4):
            assert_bits_equal(to_host(recvs[r], dtype), want, f"{what} rank {r}")

    seq = [(A[0], out[0], "sum"), (A[0], out[0], "sum"),     # repeat: the cached plan
           (A[1], out[0], "sum"),                            # other send buffers
           (A[0], out[1], "sum"),                            # other receive buffers
           (small, small_out, "sum"),                        # other count
           (A[0], out[0], "max"),                            # other operator
           (A[0], out[0], "sum")]
    for k, (s, r, op) in enumerate(seq):
        for t in r:
            t.fill_(0)
        comm.allreduce(s, r, op=op)
        check(s, r, op, f"launch {k}")
    # groups: the same two collectives, then in the other order, then one swapped
    for k, pairs in enumerate([[(A[0], out[0]), (small, small_out)],
                               [(A[0], out[0]), (small, small_out)],
                               [(small, small_out), (A[0], out[0])],
                               [(A[1], out[1]), (small, small_out)]]):
        for _, r in pairs:
            for t in r:
                t.fill_(0)
        with comm.group():
            for s, r in pairs:
                comm.allreduce(s, r)
        torch.cuda.synchronize()
        xs = [np.stack([to_host(t, dtype) for t in s]) for s, _ in pairs]
        want = cf.allreduce(xs, order, mask, proto, buff, 4, dtype)
        for (s, r), wv in zip(pairs, want):
            for q in range(4):
                assert_bits_equal(to_host(r[q], dtype), wv, f"group {k} rank {q}")
    assert comm.async_error() == 0
    comm.close()


@pytest.mark.parametrize("placement", [0, 1])
def test_comm_graph_text_lists_rings_and_lane_xcds(placement):
    """The communicator's GRAPH lines are the rings rar_graph_text prints for
    its layout, and each geometry line names the XCD of every lane's
    workgroups: pipeline q = n * lanes + lane on XCD q mod 8 (placement 0,
    one XCD per pipeline), rank r of it on XCD (q + r) mod 8 (placement 1)."""
    import ring_all_reduce_channelmask_amd as rar
    rings = [[0, 1, 2, 3], [0, 2, 3, 1]]
    mask = 0b1011
    c = _comm(nranks=4, ring_order=rings, mask=mask, proto="SIMPLE", lanes=3, waves=2,
              placement=placement, launch_mode=1)
    lines = c.graph().splitlines()
    assert lines[0::2] == rar.graph_text(4, rings, mask).splitlines()
    for n, g in enumerate(lines[1::2]):
        head, xcds = g.split("XCD per lane:")
        assert head.startswith("  lanes 3, waves 2, FIFO ")
        got = xcds.split()
        assert len(got) == 3
        for lane, x in enumerate(got):
            q = n * 3 + lane
            want = str(q % 8) if placement == 0 else "/".join(str((q + r) % 8) for r in range(4))
            assert x == want, (n, lane, x, want)
