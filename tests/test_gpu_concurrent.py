"""The plain launch (launch_mode 1, the benchmark's) beside other work: ring
launches issued on one stream while large matrix products run on a second
(default-priority) stream wait for the device behind or beside them, complete
without the wait watchdog firing, and give the oracle's bits.  (On MI355X the
products hold the CUs until they end, so the ring launches finish just after
them.)  Every wait in the kernel is bounded: a failure would end in the
watchdog's abort, not a hang."""
import numpy as np
import pytest

from oracle import closed_form as cf

from .gpu_util import assert_bits_equal, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("proto,lanes,waves", [("SIMPLE", 10, 4), ("LL128", 16, 4), ("LL", 8, 4)])
def test_plain_launch_beside_a_busy_stream(proto, lanes, waves):
    import torch
    import ring_all_reduce_channelmask_amd as rar
    from ring_all_reduce_channelmask_amd import _lib
    order, mask, n, reps = [0, 2, 3, 1], 0xFFF, 4 << 20, 4
    comm = rar.Comm(4, order, mask, proto=proto, lanes=lanes, waves=waves, launch_mode=1,
                    timeout_us=5_000_000)
    x = np.random.default_rng([60, lanes]).uniform(-1, 1, (4, n)).astype(np.float32)
    sends = [to_device(r, "float32") for r in x]
    outs = [[torch.empty_like(t) for t in sends] for _ in range(reps)]
    a = torch.randn(8192, 8192, device="cuda")
    side, main = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        prods = [a @ a for _ in range(3)]
    with torch.cuda.stream(main):
        for i in range(reps):
            comm.allreduce(sends, outs[i], stream=main)
    torch.cuda.synchronize()
    assert comm.async_error() == _lib.SUCCESS, "the wait watchdog fired"
    assert all(torch.isfinite(p).all().item() for p in prods)
    comm.close()
    want = cf.allreduce([x], order, mask, proto, {"SIMPLE": 4 << 20, "LL": 512 << 10,
                                                  "LL128": 4915200}[proto], 4, "float32")[0]
    for i in range(reps):
        for r in range(4):
            assert_bits_equal(to_host(outs[i][r], "float32"), want, f"{proto} call {i} rank {r}")
