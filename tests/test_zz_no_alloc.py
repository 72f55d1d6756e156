"""ring_allreduce_noalloc, the entry point that allocates nothing, against
ring_allreduce, the entry point it is a variant of: the same arguments must
give the same bits.  Two calls in a row, the second with a smaller input
(the library's static array keeps what the first call left in it), for every
protocol and payload type; a shape too large for the array is refused; and
the call captured into a HIP graph replays correctly with eager work in
between."""
import ctypes

import numpy as np
import pytest

from oracle import closed_form as cf
from ring_all_reduce_channelmask_amd import workloads as wl

from .gpu_util import assert_bits_equal, to_device, to_host

pytestmark = pytest.mark.gpu

# proto, dtype, ring, channels, buff_size (0 = default), chunk_steps, the two counts
CASES = [
    ("SIMPLE", "float32", [0, 2, 3, 1], 12, 1 << 20, 4, (1 << 20) + 13, 50001),
    ("SIMPLE", "int32", [0, 3, 1, 6, 2, 7, 5, 4], 16, 256 << 10, 2, 600007, 4099),
    ("SIMPLE", "bfloat16", [0, 1, 2, 3], 1, 64 << 10, 4, 1024, 333),
    ("LL", "float32", [0, 2, 3, 1], 4, 0, 0, 131072, 777),
    ("LL", "bfloat16", [0, 1, 2, 3], 7, 0, 0, 104 * 7168, 7168),
    ("LL128", "float32", [0, 2, 3, 1], 4, 8 * 2048 * 16, 0, 300007, 120 * 64 + 5),
    ("LL128", "bfloat16", [0, 2, 1], 3, 8 * 2048 * 8, 0, 90001, 301),
]


def _rand(dtype, shape, seed):
    rng = np.random.default_rng(seed)
    if dtype == "int32":
        return rng.integers(-2 ** 27, 2 ** 27, size=shape).astype(np.int32)
    v = rng.standard_normal(shape).astype(np.float32)
    return v if dtype == "float32" else wl._bf16_bits(v.ravel()).reshape(shape)


def _run(fn, x, dtype, ring, proto, C, buff, cs):
    import torch
    import ring_all_reduce_channelmask_amd as rar
    sends = [to_device(row, dtype) for row in x]
    recvs = [torch.full_like(t, 0) for t in sends]
    getattr(rar, fn)(sends, recvs, ring, proto=proto, nchannels=C, buff_size=buff, chunk_steps=cs)
    torch.cuda.synchronize()
    return np.stack([to_host(t, dtype) for t in recvs])


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-n{len(c[2])}-c{c[3]}" for c in CASES])
def test_noalloc_matches_ring_allreduce_twice(case):
    proto, dtype, ring, C, buff, cs, n1, n2 = case
    N = len(ring)
    for k, n in enumerate((n1, n2)):
        x = _rand(dtype, (N, n), 1000 * k + n % 997)
        want = _run("ring_allreduce", x, dtype, ring, proto, C, buff, cs)
        got = _run("ring_allreduce_noalloc", x, dtype, ring, proto, C, buff, cs)
        assert_bits_equal(got, want, f"{proto} {dtype} call {k} count {n}")
        if n <= 200000:
            # and the fold the pages define, for the smaller sizes
            dflt = {"SIMPLE": 4 << 20, "LL": 512 << 10, "LL128": 4915200}[proto]
            oc = cf.allreduce([x], ring, (1 << C) - 1, proto, buff or dflt, cs or 4, dtype)[0]
            for r in range(N):
                assert_bits_equal(got[r], oc, f"{proto} {dtype} call {k} rank {r} vs closed form")


def test_noalloc_refuses_a_shape_beyond_its_array():
    import torch
    from ring_all_reduce_channelmask_amd import _lib
    lib = _lib.load()
    N = 4
    # LL128 at its default buffer over 12 channels: 4 x 12 x 4.9 MB of FIFO
    sends = [torch.zeros(1000, device="cuda") for _ in range(N)]
    recvs = [torch.zeros(1000, device="cuda") for _ in range(N)]
    arr = lambda ts: (ctypes.c_void_p * N)(*[t.data_ptr() for t in ts])  # noqa: E731
    order = (ctypes.c_int * N)(0, 2, 3, 1)
    rc = lib.ring_allreduce_noalloc(arr(sends), arr(recvs), N, 1000, _lib.DTYPE["float32"], 0, order,
                                    _lib.PROTO["LL128"], 12, 0, 0, None)
    assert rc == _lib.INVALID_ARGUMENT
    assert b"bytes of device state" in lib.rar_get_last_error()
    torch.cuda.synchronize()
    assert all(int(t.count_nonzero()) == 0 for t in recvs)


@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
def test_noalloc_graph_replays(proto):
    import torch
    import ring_all_reduce_channelmask_amd as rar
    ring, C, dtype = [0, 2, 3, 1], 3, "float32"
    buff = {"SIMPLE": 64 << 10, "LL": 0, "LL128": 8 * 2048 * 8}[proto]
    n = 70001
    sends = [torch.empty(n, device="cuda") for _ in range(4)]
    recvs = [torch.empty_like(t) for t in sends]
    x0 = _rand(dtype, (4, n), 7)
    for t, row in zip(sends, x0):
        t.copy_(to_device(row, dtype))
    rar.ring_allreduce_noalloc(sends, recvs, ring, proto=proto, nchannels=C, buff_size=buff)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rar.ring_allreduce_noalloc(sends, recvs, ring, proto=proto, nchannels=C, buff_size=buff)
    torch.cuda.synchronize()
    for rep in range(3):
        x = _rand(dtype, (4, n), 100 + rep)
        for t, row in zip(sends, x):
            t.copy_(to_device(row, dtype))
        for t in recvs:
            t.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = _run("ring_allreduce", x, dtype, ring, proto, C, buff, 0)
        assert_bits_equal(np.stack([to_host(t, dtype) for t in recvs]), want, f"replay {rep}")
        # an eager no-alloc call of another size between replays
        y = _rand(dtype, (4, 999), 200 + rep)
        got = _run("ring_allreduce_noalloc", y, dtype, ring, proto, C, buff, 0)
        assert_bits_equal(got, _run("ring_allreduce", y, dtype, ring, proto, C, buff, 0), "eager")
