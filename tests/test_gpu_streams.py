"""ring_allreduce's cached communicator reached from two streams and from two
threads: calls of the same shape share one set of FIFOs and step counters, so
the library orders a call on a new stream after the previous launch.  Every
call writes its own output buffers, and each is checked against the oracle's
closed form."""
import threading

import numpy as np
import pytest

from oracle import closed_form as cf
from ring_all_reduce_channelmask_amd import workloads as wl

from .gpu_util import assert_bits_equal, to_device, to_host

pytestmark = pytest.mark.gpu

BUFF = {"SIMPLE": 4 << 20, "LL": 512 << 10, "LL128": 4915200}


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
def test_same_shape_on_two_streams(proto):
    import torch
    import ring_all_reduce_channelmask_amd as rar
    order, C, n, reps = [0, 2, 3, 1], 3, 200003, 6
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    xs = [_rand((4, n), 70 + k) for k in range(2)]
    sends = [[to_device(r, "float32") for r in x] for x in xs]
    outs = [[[torch.empty_like(t) for t in sends[k]] for _ in range(reps)] for k in range(2)]
    torch.cuda.synchronize()
    for i in range(reps):
        for k in range(2):
            with torch.cuda.stream(streams[k]):
                rar.ring_allreduce(sends[k], outs[k][i], order, proto=proto, nchannels=C,
                                   stream=streams[k])
    torch.cuda.synchronize()
    for k in range(2):
        want = cf.allreduce([xs[k]], order, (1 << C) - 1, proto, BUFF[proto], 4, "float32")[0]
        for i in range(reps):
            for r in range(4):
                assert_bits_equal(to_host(outs[k][i][r], "float32"), want, f"stream {k} call {i} rank {r}")


def test_same_shape_from_two_threads():
    import torch
    import ring_all_reduce_channelmask_amd as rar
    order, C, n, reps, proto = [0, 1, 2, 3], 2, 65537, 8, "LL"
    xs = [_rand((4, n), 80 + k) for k in range(2)]
    sends = [[to_device(r, "float32") for r in x] for x in xs]
    outs = [[[torch.empty_like(t) for t in sends[k]] for _ in range(reps)] for k in range(2)]
    torch.cuda.synchronize()
    errors = []

    def worker(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for i in range(reps):
                    rar.ring_allreduce(sends[k], outs[k][i], order, proto=proto, nchannels=C, stream=s)
            s.synchronize()
        except Exception as e:  # reported below
            errors.append(e)

    th = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k in range(2):
        want = cf.allreduce([xs[k]], order, (1 << C) - 1, proto, BUFF[proto], 4, "float32")[0]
        for i in range(reps):
            for r in range(4):
                assert_bits_equal(to_host(outs[k][i][r], "float32"), want, f"thread {k} call {i} rank {r}")


def test_cache_release_waits_for_the_launch_and_next_call_rebuilds():
    """ring_allreduce_cache_release right after a launch, with no
    synchronize in between: it waits for that launch before freeing the
    communicator, and the next call of the shape builds a fresh one whose
    output has the same bits."""
    import torch
    import ring_all_reduce_channelmask_amd as rar
    order, C, n = [0, 2, 3, 1], 4, 300007
    for proto in ("SIMPLE", "LL128"):
        x = _rand((4, n), 90)
        sends = [to_device(r, "float32") for r in x]
        outs = [[torch.empty_like(t) for t in sends] for _ in range(3)]
        torch.cuda.synchronize()
        rar.ring_allreduce_cache_release()  # whatever earlier tests cached
        for i in range(3):
            rar.ring_allreduce(sends, outs[i], order, proto=proto, nchannels=C)
            rar.ring_allreduce_cache_release()
        rar.ring_allreduce_cache_release()  # nothing left: a no-op
        torch.cuda.synchronize()
        want = cf.allreduce([x], order, (1 << C) - 1, proto, BUFF[proto], 4, "float32")[0]
        for i in range(3):
            for r in range(4):
                assert_bits_equal(to_host(outs[i][r], "float32"), want, f"{proto} call {i} rank {r}")
