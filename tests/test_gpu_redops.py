"""Parity of every reduction operator (prod, max, min, avg; sum is covered
everywhere else) between the HIP kernels and the oracle, bit for bit: the
ring under all three protocols against the simulator, the fused group, the
benchmark's 64 MiB size against the closed form, and the one-shot."""
import numpy as np
import pytest

import oracle
from oracle import closed_form as cf
from oracle import oneshot
from ring_all_reduce_channelmask_amd import workloads as wl

from .gpu_util import assert_bits_equal, run_hip, to_device, to_host

pytestmark = pytest.mark.gpu

SMALL_BUFF = {"SIMPLE": 8 * 1024, "LL": 8 * 512, "LL128": 8 * 2048}
OPS = ["prod", "max", "min", "avg"]


def _draw(dtype, shape, seed, op):
    rng = np.random.default_rng(seed)
    if dtype == "int32":
        lim = 2 ** 31 if op != "avg" else 2 ** 20
        return rng.integers(-lim, lim, size=shape).astype(np.int32)
    v = (1 + 0.1 * rng.standard_normal(shape)) if op == "prod" else rng.standard_normal(shape)
    v = v.astype(np.float32)
    return v if dtype == "float32" else wl._bf16_bits(v.ravel()).reshape(shape)


def _comm(**kw):
    import ring_all_reduce_channelmask_amd as rar
    return rar.Comm(**kw)


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
def test_ring_ops_vs_simulator(op, dtype, proto):
    buff = SMALL_BUFF[proto]
    comm = _comm(nranks=4, ring_order=[0, 2, 3, 1], mask=0x7, proto=proto, buff_size=buff,
                 chunk_steps=4 if proto == "SIMPLE" else 0, lanes=2, waves=4)
    x = _draw(dtype, (4, 50021), 13, op)
    got = run_hip(comm, [x], dtype, op=op)[0]
    comm.close()
    rc, want, _, _ = oracle.allreduce([x], [0, 2, 3, 1], 0x7, proto, buff, 4, dtype, op=op)
    assert rc == oracle.OK
    for r in range(4):
        assert_bits_equal(got[r], want[0][r], f"{op} {dtype} {proto} rank {r}")


@pytest.mark.parametrize("op", OPS)
def test_ring_ops_direct_variant(op):
    buff = SMALL_BUFF["SIMPLE"] * 2
    comm = _comm(nranks=5, ring_order=[0, 3, 1, 4, 2], mask=0x5, proto="SIMPLE", buff_size=buff,
                 lanes=3, waves=4, direct=1)
    x = _draw("bfloat16", (5, 70001), 17, op)
    got = run_hip(comm, [x], "bfloat16", op=op)[0]
    comm.close()
    want = cf.allreduce([x], [0, 3, 1, 4, 2], 0x5, "SIMPLE", buff, 4, "bfloat16", op=op)[0]
    for r in range(5):
        assert_bits_equal(got[r], want, f"{op} rank {r}")


@pytest.mark.parametrize("op", OPS)
def test_ring_ops_fused_group(op):
    """A fused group (several works per channel) with a post-op in every work."""
    xs = [_draw("float32", (3, c), 20 + c, op) for c in (1, 4097, 30000, 7)]
    comm = _comm(nranks=3, ring_order=[2, 0, 1], mask=0b1011, proto="LL", buff_size=8 * 512)
    got = run_hip(comm, xs, "float32", op=op)
    comm.close()
    want = cf.allreduce(xs, [2, 0, 1], 0b1011, "LL", 8 * 512, 4, "float32", op=op)
    for i in range(len(xs)):
        for r in range(3):
            assert_bits_equal(got[i][r], want[i], f"{op} work {i} rank {r}")


def test_group_mixing_operators_is_rejected():
    import torch
    import ring_all_reduce_channelmask_amd as rar
    comm = _comm(nranks=2, ring_order=[0, 1], mask=0x1, proto="SIMPLE")
    t = [torch.zeros(64, device="cuda") for _ in range(2)]
    with pytest.raises(rar.RarError):
        with comm.group():
            comm.allreduce(t, t, op="sum")
            comm.allreduce(t, t, op="max")
    comm.close()


@pytest.mark.parametrize("op", ["avg", "max"])
def test_ring_ops_full_size(op):
    """64 MiB per rank, the benchmark's launch shape, against the closed form."""
    w = wl.WORKLOADS["simple_64m"]
    x = wl.inputs_for(w)[0]
    import bench
    comm = _comm(nranks=4, ring_order=list(w.ring_order), mask=w.mask, proto="SIMPLE",
                 buff_size=w.buff_size, chunk_steps=4, **bench.TUNING["simple_64m"])
    got = run_hip(comm, [x], "float32", op=op)[0]
    comm.close()
    want = cf.allreduce([x], list(w.ring_order), w.mask, "SIMPLE", w.buff_size, 4, "float32",
                        op=op)[0]
    for r in range(4):
        assert_bits_equal(got[r], want, f"{op} rank {r}")


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
def test_oneshot_ops_vs_oracle(op, dtype):
    import torch
    import ring_all_reduce_channelmask_amd as rar
    x = _draw(dtype, (6, 100005), 31, op)
    sends = [to_device(x[r], dtype) for r in range(6)]
    recvs = [torch.empty_like(t) for t in sends]
    rar.oneshot_allreduce(sends, recvs, op=op)
    torch.cuda.synchronize()
    want = oneshot.allreduce(x, dtype, op)
    for r in range(6):
        assert_bits_equal(to_host(recvs[r], dtype), want, f"{op} {dtype} rank {r}")


# ------------------------------------------------------------ PreMulSum
def _scal(dtype, vals):
    v = np.asarray(vals, dtype=np.float64)
    if dtype == "int32":
        return v.astype(np.int32)
    if dtype == "float32":
        return v.astype(np.float32)
    return wl._bf16_bits(v.astype(np.float32))


def _run_premul(comm, xs, dtype, scs, in_place=False):
    import torch
    from .gpu_util import to_device
    N = comm.nranks
    sends = [[to_device(x[r], dtype) for r in range(N)] for x in xs]
    recvs = [s if in_place else [torch.empty_like(t) for t in s] for s in sends]
    if len(xs) == 1:
        comm.allreduce(sends[0], recvs[0], op="premulsum", scalars=scs[0])
    else:
        with comm.group():
            for s, r, sc in zip(sends, recvs, scs):
                comm.allreduce(s, r, op="premulsum", scalars=sc)
    torch.cuda.synchronize()
    return [np.stack([to_host(t, dtype) for t in r]) for r in recvs]


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
def test_ring_premulsum_vs_simulator(dtype, proto):
    buff = SMALL_BUFF[proto]
    comm = _comm(nranks=4, ring_order=[0, 2, 3, 1], mask=0x7, proto=proto, buff_size=buff,
                 chunk_steps=4 if proto == "SIMPLE" else 0, lanes=2, waves=4)
    x = _draw(dtype, (4, 50021), 81, "sum")
    sc = _scal(dtype, [3, -2, 0.5, 7] if dtype != "int32" else [3, -2, 5, 7])
    got = _run_premul(comm, [x], dtype, [sc])[0]
    comm.close()
    rc, want, _, _ = oracle.allreduce([x], [0, 2, 3, 1], 0x7, proto, buff, 4, dtype,
                                      op="premulsum", scalars=sc)
    assert rc == oracle.OK
    for r in range(4):
        assert_bits_equal(got[r], want[0][r], f"{dtype} {proto} rank {r}")


@pytest.mark.parametrize("direct", [1, 2, 3])
@pytest.mark.parametrize("in_place", [False, True])
def test_ring_premulsum_direct_variants(direct, in_place):
    buff = SMALL_BUFF["SIMPLE"] * 2
    order = [0, 3, 1, 4, 2]
    comm = _comm(nranks=5, ring_order=order, mask=0x5, proto="SIMPLE", buff_size=buff,
                 lanes=3, waves=4, direct=direct)
    x = _draw("bfloat16", (5, 70001), 83, "sum")
    sc = _scal("bfloat16", [0.5, -1.25, 3.0, 1.0, -0.75])
    got = _run_premul(comm, [x], "bfloat16", [sc], in_place=in_place)[0]
    comm.close()
    want = cf.allreduce([x], order, 0x5, "SIMPLE", buff, 4, "bfloat16", op="premulsum",
                        scalars=sc)[0]
    for r in range(5):
        assert_bits_equal(got[r], want, f"direct {direct} rank {r}")


def test_ring_premulsum_fused_group_own_scalars():
    xs = [_draw("float32", (3, c), 90 + c, "sum") for c in (1, 4097, 30000, 7)]
    scs = [_scal("float32", [1 + i, -0.5 * i, 2.0]) for i in range(len(xs))]
    comm = _comm(nranks=3, ring_order=[2, 0, 1], mask=0b1011, proto="LL", buff_size=8 * 512)
    got = _run_premul(comm, xs, "float32", scs)
    comm.close()
    want = cf.allreduce(xs, [2, 0, 1], 0b1011, "LL", 8 * 512, 4, "float32", op="premulsum",
                        scalars=np.stack(scs))
    for i in range(len(xs)):
        for r in range(3):
            assert_bits_equal(got[i][r], want[i], f"work {i} rank {r}")


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
def test_oneshot_premulsum_vs_oracle(dtype):
    import torch
    import ring_all_reduce_channelmask_amd as rar
    x = _draw(dtype, (6, 100005), 87, "sum")
    sc = _scal(dtype, [1, -2, 0.25, 3, -0.5, 5] if dtype != "int32" else [1, -2, 9, 3, -77, 5])
    sends = [to_device(x[r], dtype) for r in range(6)]
    recvs = [torch.empty_like(t) for t in sends]
    rar.oneshot_allreduce(sends, recvs, op="premulsum", scalars=sc)
    torch.cuda.synchronize()
    want = oneshot.allreduce(x, dtype, "premulsum", sc)
    for r in range(6):
        assert_bits_equal(to_host(recvs[r], dtype), want, f"{dtype} rank {r}")
