"""Parity of the one-shot AllReduce kernel (through the C ABI) with the
one-shot oracle: bit for bit for every dtype, at small ragged sizes, at the
benchmark's full sizes, in place, and for every launch shape."""
import numpy as np
import pytest

from oracle import oneshot
from ring_all_reduce_channelmask_amd import workloads as wl

from .gpu_util import assert_bits_equal, to_device, to_host

pytestmark = pytest.mark.gpu


def _rand(dtype, shape, seed):
    rng = np.random.default_rng(seed)
    if dtype == "int32":
        return rng.integers(-2 ** 31, 2 ** 31, size=shape).astype(np.int32)
    v = rng.standard_normal(shape).astype(np.float32)
    return v if dtype == "float32" else wl._bf16_bits(v.ravel()).reshape(shape)


def _run(x, dtype, in_place=False, **tune):
    import torch
    import ring_all_reduce_channelmask_amd as rar
    N = x.shape[0]
    sends = [to_device(x[r], dtype) for r in range(N)]
    recvs = sends if in_place else [torch.full_like(t, 0x7F if dtype != "float32" else float("nan"))
                                    for t in sends]
    rar.oneshot_allreduce(sends, recvs, **tune)
    torch.cuda.synchronize()
    return np.stack([to_host(t, dtype) for t in recvs])


CASES = [(N, c) for N in (2, 3, 4, 8) for c in (1, 7, 8, 9, 1000, 65539)] + [(64, 4099), (5, 1 << 20)]


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
@pytest.mark.parametrize("N,count", CASES, ids=[f"N{n}-{c}" for n, c in CASES])
def test_small_vs_oracle(dtype, N, count):
    x = _rand(dtype, (N, count), N * 131 + count)
    got = _run(x, dtype)
    want = oneshot.allreduce(x, dtype)
    for r in range(N):
        assert_bits_equal(got[r], want, f"rank {r}")


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
def test_in_place(dtype):
    x = _rand(dtype, (4, 100003), 7)
    got = _run(x, dtype, in_place=True)
    want = oneshot.allreduce(x, dtype)
    for r in range(4):
        assert_bits_equal(got[r], want, f"rank {r}")


@pytest.mark.parametrize("tune", [dict(workgroups=1), dict(workgroups=7, waves=1, unroll=1),
                                  dict(waves=8, unroll=4), dict(workgroups=4096, unroll=4),
                                  dict(waves=2, unroll=2)])
def test_launch_shape_does_not_change_bits(tune):
    x = _rand("bfloat16", (6, 300007), 9)
    got = _run(x, "bfloat16", **tune)
    want = oneshot.allreduce(x, "bfloat16")
    for r in range(6):
        assert_bits_equal(got[r], want, f"{tune} rank {r}")


def test_empty_and_repeated_launches():
    import torch
    import ring_all_reduce_channelmask_amd as rar
    e = [torch.empty(0, device="cuda") for _ in range(3)]
    rar.oneshot_allreduce(e, [torch.empty(0, device="cuda") for _ in range(3)])
    x = _rand("float32", (3, 50001), 11)
    sends = [to_device(x[r], "float32") for r in range(3)]
    recvs = [torch.empty_like(t) for t in sends]
    for _ in range(200):
        rar.oneshot_allreduce(sends, recvs)
    torch.cuda.synchronize()
    want = oneshot.allreduce(x, "float32")
    for r in range(3):
        assert_bits_equal(to_host(recvs[r], "float32"), want, f"rank {r}")


@pytest.mark.parametrize("key", ["simple_64m", "bf16_n8", "int32_n8"])
def test_full_size_workloads(key):
    """The benchmark's sizes and inputs (4 x 64 MiB fp32; 8 x 64 MiB bf16;
    8 x 128 MiB int32), every element against the oracle."""
    w = wl.WORKLOADS[key]
    x = wl.inputs_for(w)[0]
    import bench
    got = _run(x, w.dtype, **bench.ONESHOT_TUNING.get(key, {}))
    want = oneshot.allreduce(x, w.dtype)
    if w.dtype == "int32":
        s = (x.astype(np.int64).sum(axis=0) & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
        np.testing.assert_array_equal(want, s)
    for r in range(w.nranks):
        assert_bits_equal(got[r], want, f"{key} rank {r}")
