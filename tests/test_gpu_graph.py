"""Launches captured into a HIP graph and replayed.

Steps, flags and the placement handshake's launch count live on the device,
and a plan that fits travels inside the kernel arguments, so a captured
allreduce is a plain kernel node: every replay is one more launch on the
communicator.  Each replay is checked against the oracle's closed form, with
eager launches on the same communicator and fresh inputs between replays."""
import numpy as np
import pytest

from oracle import closed_form as cf
from ring_all_reduce_channelmask_amd import workloads as wl

from .gpu_util import assert_bits_equal, to_device, to_host

pytestmark = pytest.mark.gpu

BUFF = {"SIMPLE": 8 * 1024, "LL": 8 * 512, "LL128": 8 * 2048}


def _rand(dtype, shape, seed):
    rng = np.random.default_rng(seed)
    if dtype == "int32":
        return rng.integers(-2 ** 31, 2 ** 31, size=shape).astype(np.int32)
    v = rng.standard_normal(shape).astype(np.float32)
    return v if dtype == "float32" else wl._bf16_bits(v.ravel()).reshape(shape)


def _fill(tensors, x, dtype):
    for t, row in zip(tensors, x):
        t.copy_(to_device(row, dtype))


def _captured_replays(proto, dtype, **shape):
    import torch
    import ring_all_reduce_channelmask_amd as rar
    order, mask, buff = [0, 2, 3, 1], 0b1011, BUFF[proto]
    cs = 4 if proto == "SIMPLE" else 0
    comm = rar.Comm(4, order, mask, proto=proto, buff_size=buff, chunk_steps=cs, lanes=2,
                    waves=2, launch_mode=1, **shape)
    counts = [30011, 777]  # one collective, then a group of two
    sends = [[torch.empty(c, dtype=getattr(torch, dtype), device="cuda") for _ in range(4)]
             for c in counts]
    recvs = [[torch.empty_like(t) for t in s] for s in sends]
    extra_in = [to_device(r, dtype) for r in _rand(dtype, (4, 5003), 900)]
    extra_out = [torch.empty_like(t) for t in extra_in]
    _fill(sends[0], _rand(dtype, (4, counts[0]), 901), dtype)
    _fill(sends[1], _rand(dtype, (4, counts[1]), 902), dtype)
    comm.allreduce(sends[0], recvs[0])  # eager launch before the capture
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        comm.allreduce(sends[0], recvs[0])
        with comm.group():
            comm.allreduce(sends[1], recvs[1])
            comm.allreduce(sends[0], recvs[0])
    torch.cuda.synchronize()

    for rep in range(3):
        xs = [_rand(dtype, (4, c), 910 + 10 * rep + i) for i, c in enumerate(counts)]
        for s, x in zip(sends, xs):
            _fill(s, x, dtype)
        for r in recvs:
            for t in r:
                t.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert comm.async_error() == 0
        # the graph's last node reduced group [sends[1], sends[0]]
        want = cf.allreduce([xs[1], xs[0]], order, mask, proto, buff, 4, dtype)
        for i, w in ((1, want[0]), (0, want[1])):
            for r in range(4):
                assert_bits_equal(to_host(recvs[i][r], dtype), w, f"replay {rep} coll {i} rank {r}")
        # an eager launch of another size between replays
        comm.allreduce(extra_in, extra_out)
        torch.cuda.synchronize()
        want = cf.allreduce([np.stack([to_host(t, dtype) for t in extra_in])], order, mask, proto,
                            buff, 4, dtype)[0]
        for r in range(4):
            assert_bits_equal(to_host(extra_out[r], dtype), want, f"eager after replay {rep}")
    comm.close()


@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_captured_allreduce_replays_match_oracle(proto, dtype):
    _captured_replays(proto, dtype)


@pytest.mark.parametrize("proto", ["SIMPLE", "LL128"])
@pytest.mark.parametrize("shape", [dict(placement=1), dict(deal_works=1)],
                         ids=["spread", "dealt"])
def test_captured_replays_spread_and_dealt(proto, shape):
    """The same with every rank of a pipeline on another XCD (the launch count
    decides the placement each replay), and with works dealt to lanes."""
    _captured_replays(proto, "float32", **shape)


def test_capture_rejects_what_cannot_replay():
    """A cooperative launch, and a plan too large to travel inline, are
    refused under capture, before anything is enqueued."""
    import torch
    import ring_all_reduce_channelmask_amd as rar
    from ring_all_reduce_channelmask_amd import _lib
    x = [torch.ones(4096, device="cuda") for _ in range(4)]
    y = [torch.empty_like(t) for t in x]
    coop = rar.Comm(4, [0, 1, 2, 3], 0x3, proto="LL", launch_mode=0)
    big = rar.Comm(4, [0, 1, 2, 3], (1 << 40) - 1, proto="LL", launch_mode=1)
    for comm, why in ((coop, "cooperative"), (big, "inline")):
        graph = torch.cuda.CUDAGraph()
        with pytest.raises(rar.RarError) as e:
            with torch.cuda.graph(graph):
                comm.allreduce(x, y)
        assert e.value.code == _lib.UNSUPPORTED and why in str(e.value)
        torch.cuda.synchronize()
        comm.allreduce(x, y)  # the communicator still works eagerly
        torch.cuda.synchronize()
        assert all(torch.equal(t, torch.full_like(t, 4.0)) for t in y)
        comm.close()


def test_captured_oneshot_replays():
    """The one-shot kernel carries everything in its arguments: captured once,
    it recomputes from the inputs present at each replay."""
    import torch
    import ring_all_reduce_channelmask_amd as rar
    from oracle import oneshot
    n = 100003
    x = [torch.empty(n, device="cuda") for _ in range(4)]
    y = [torch.empty_like(t) for t in x]
    graph = torch.cuda.CUDAGraph()
    _fill(x, _rand("float32", (4, n), 950), "float32")
    with torch.cuda.graph(graph):
        rar.oneshot_allreduce(x, y)
    for rep in range(3):
        xs = _rand("float32", (4, n), 951 + rep)
        _fill(x, xs, "float32")
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = oneshot.allreduce(xs, "float32")
        for r in range(4):
            assert_bits_equal(y[r].cpu().numpy(), want, f"replay {rep} rank {r}")


@pytest.mark.parametrize("key", ["simple_4k", "ll_512k", "simple_64m", "ll128_64m"])
def test_benchmark_shapes_replayed_from_a_graph(key):
    """The ring workloads at full size in the launch shape the benchmark
    times (its TUNING table), captured once and replayed with fresh inputs,
    an eager launch of the same communicator after each replay; every
    result bit for bit against the closed form."""
    import torch
    import bench
    import ring_all_reduce_channelmask_amd as rar
    w = wl.WORKLOADS[key]
    N, count = w.nranks, w.counts[0]
    cs = w.chunk_steps if w.proto == "SIMPLE" else 0
    comm = rar.Comm(N, list(w.ring_order), w.mask, proto=w.proto, buff_size=w.buff_size,
                    chunk_steps=cs, **bench.TUNING[key])
    sends = [torch.empty(count, dtype=getattr(torch, w.dtype), device="cuda") for _ in range(N)]
    recvs = [torch.empty_like(t) for t in sends]
    _fill(sends, wl.inputs_for(w)[0], w.dtype)
    comm.allreduce(sends, recvs)  # eager launch before the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        comm.allreduce(sends, recvs)
    torch.cuda.synchronize()
    for rep in range(2):
        x = _rand(w.dtype, (N, count), 1000 + rep)
        _fill(sends, x, w.dtype)
        for t in recvs:
            t.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert comm.async_error() == 0
        want = cf.allreduce([x], list(w.ring_order), w.mask, w.proto, w.buff_size, w.chunk_steps,
                            w.dtype)[0]
        for r in range(N):
            assert_bits_equal(to_host(recvs[r], w.dtype), want, f"{key} replay {rep} rank {r}")
        for t in recvs:
            t.fill_(0)
        comm.allreduce(sends, recvs)
        torch.cuda.synchronize()
        assert comm.async_error() == 0
        for r in range(N):
            assert_bits_equal(to_host(recvs[r], w.dtype), want, f"{key} eager {rep} rank {r}")
    del graph
    comm.close()
