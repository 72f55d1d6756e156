"""User buffers aligned only to their element size: the ring (all protocols,
in place, direct variant) and the one-shot, bit for bit against the oracle.
Each rank's buffers sit at a different offset from a 16-byte boundary."""
import numpy as np
import pytest

import oracle
from oracle import closed_form as cf
from oracle import oneshot
from ring_all_reduce_channelmask_amd import workloads as wl

from .gpu_util import assert_bits_equal, to_host

pytestmark = pytest.mark.gpu

SMALL_BUFF = {"SIMPLE": 8 * 1024, "LL": 8 * 512, "LL128": 8 * 2048}


def _rand(dtype, shape, seed):
    rng = np.random.default_rng(seed)
    if dtype == "int32":
        return rng.integers(-2 ** 31, 2 ** 31, size=shape).astype(np.int32)
    v = rng.standard_normal(shape).astype(np.float32)
    return v if dtype == "float32" else wl._bf16_bits(v.ravel()).reshape(shape)


def _offset_tensor(row, dtype, off):
    """A device tensor holding `row`, starting `off` elements past a 16-byte
    boundary (a view into a larger allocation)."""
    import torch
    tdt = {"float32": torch.float32, "int32": torch.int32, "bfloat16": torch.bfloat16}[dtype]
    big = torch.zeros(row.size + 16, dtype=tdt, device="cuda")
    t = big[off:off + row.size]
    src = np.ascontiguousarray(row)
    if dtype == "bfloat16":
        t.view(torch.int16).copy_(torch.from_numpy(src.view(np.int16)))
    else:
        t.copy_(torch.from_numpy(src))
    assert t.data_ptr() % 16 == (off * t.element_size()) % 16
    return big, t


def _buffers(x, dtype, in_place, send_offs, recv_offs):
    keep, sends, recvs = [], [], []
    for r in range(x.shape[0]):
        b, s = _offset_tensor(x[r], dtype, send_offs[r])
        keep.append(b)
        sends.append(s)
        if in_place:
            recvs.append(s)
        else:
            b2, t = _offset_tensor(np.zeros_like(x[r]), dtype, recv_offs[r])
            keep.append(b2)
            recvs.append(t)
    return keep, sends, recvs


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
def test_ring_misaligned_vs_simulator(proto, dtype, in_place):
    import torch
    import ring_all_reduce_channelmask_amd as rar
    N, count = 4, 70003
    x = _rand(dtype, (N, count), 41)
    keep, sends, recvs = _buffers(x, dtype, in_place, [1, 2, 3, 0], [3, 1, 0, 2])
    buff = SMALL_BUFF[proto]
    comm = rar.Comm(N, [0, 2, 3, 1], 0x7, proto=proto, buff_size=buff,
                    chunk_steps=4 if proto == "SIMPLE" else 0, lanes=2, waves=4)
    comm.allreduce(sends, recvs)
    torch.cuda.synchronize()
    comm.close()
    rc, want, _, _ = oracle.allreduce([x], [0, 2, 3, 1], 0x7, proto, buff, 4, dtype)
    assert rc == oracle.OK
    for r in range(N):
        assert_bits_equal(to_host(recvs[r], dtype), want[0][r], f"rank {r}")


@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_direct_variant_misaligned(dtype):
    import torch
    import ring_all_reduce_channelmask_amd as rar
    N, count = 4, 200001
    x = _rand(dtype, (N, count), 43)
    keep, sends, recvs = _buffers(x, dtype, False, [0, 1, 2, 3], [1, 2, 3, 1])
    comm = rar.Comm(N, [0, 2, 3, 1], 0x5, proto="SIMPLE", buff_size=2 * SMALL_BUFF["SIMPLE"],
                    lanes=3, waves=4, direct=1)
    comm.allreduce(sends, recvs)
    torch.cuda.synchronize()
    comm.close()
    want = cf.allreduce([x], [0, 2, 3, 1], 0x5, "SIMPLE", 2 * SMALL_BUFF["SIMPLE"], 4, dtype)[0]
    for r in range(N):
        assert_bits_equal(to_host(recvs[r], dtype), want, f"rank {r}")


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
def test_oneshot_misaligned(dtype):
    import torch
    import ring_all_reduce_channelmask_amd as rar
    N, count = 5, 100019
    x = _rand(dtype, (N, count), 47)
    keep, sends, recvs = _buffers(x, dtype, False, [1, 0, 3, 2, 1], [2, 3, 0, 1, 3])
    rar.oneshot_allreduce(sends, recvs)
    torch.cuda.synchronize()
    want = oneshot.allreduce(x, dtype)
    for r in range(N):
        assert_bits_equal(to_host(recvs[r], dtype), want, f"rank {r}")


def test_ring_full_size_misaligned():
    """The 64 MiB Simple workload in the benchmark's launch shape with every
    buffer one element off a 16-byte boundary."""
    import torch
    import ring_all_reduce_channelmask_amd as rar
    import bench
    w = wl.WORKLOADS["simple_64m"]
    x = wl.inputs_for(w)[0]
    keep, sends, recvs = _buffers(x, "float32", False, [1] * 4, [1] * 4)
    comm = rar.Comm(4, list(w.ring_order), w.mask, proto="SIMPLE", buff_size=w.buff_size,
                    chunk_steps=4, **bench.TUNING["simple_64m"])
    comm.allreduce(sends, recvs)
    torch.cuda.synchronize()
    comm.close()
    want = cf.allreduce([x], list(w.ring_order), w.mask, "SIMPLE", w.buff_size, 4, "float32")[0]
    for r in range(4):
        assert_bits_equal(to_host(recvs[r], "float32"), want, f"rank {r}")
