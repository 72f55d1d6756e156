"""Many back-to-back launches on one communicator at full size, with inputs
that change between launches: every FIFO slot is rewritten many times over,
so a receiver that read a stale line (from an earlier step or launch) or a
line before its data arrived would show up as a wrong element.

int32 sum is exact and independent of the fold order, so each launch is
checked against the plain wrap-around sum of its inputs (a property that
holds at any size; the element-by-element comparison with the oracle's
closed form runs in test_gpu_parity.py).  The launch shapes are the
benchmark's, in both workgroup placements and in strict scope."""
import pytest

pytestmark = pytest.mark.gpu


def _launches(proto, lanes, waves, placement=0, strict=0, launches=12, count=16 << 20):
    import torch
    import ring_all_reduce_channelmask_amd as rar
    N, order, mask = 4, [0, 2, 3, 1], 0xFFF
    comm = rar.Comm(N, order, mask, proto=proto, lanes=lanes, waves=waves, launch_mode=1,
                    placement=placement, strict_scope=strict)
    g = torch.Generator(device="cuda").manual_seed(7)
    base = [torch.randint(-2 ** 31, 2 ** 31 - 1, (count,), dtype=torch.int32, device="cuda",
                          generator=g) for _ in range(N)]
    recvs = [torch.empty_like(b) for b in base]
    try:
        for k in range(launches):
            # launch k changes rank k mod N's input by k + 1 everywhere and one
            # element of every rank by a launch-specific amount
            sends = [b.clone() for b in base]
            sends[k % N] += k + 1
            for r in range(N):
                sends[r][(k * 7919 + r * 104729) % count] ^= (k + 1) << 20
            want = torch.stack(sends).to(torch.int64).sum(dim=0)
            want = ((want + 2 ** 31) % 2 ** 32 - 2 ** 31).to(torch.int32)
            for t in recvs:
                t.fill_(0x5A5A5A5A)
            comm.allreduce(sends, recvs)
            torch.cuda.synchronize()
            assert comm.async_error() == 0, f"watchdog fired at launch {k}"
            for r in range(N):
                bad = torch.nonzero(recvs[r] != want)
                assert bad.numel() == 0, (f"launch {k} rank {r}: {bad.numel()} elements differ, "
                                          f"first at {bad[:4].flatten().tolist()}")
    finally:
        comm.close()


@pytest.mark.parametrize("placement", [0, 1])
def test_ll128_repeated_full_size_launches(placement):
    _launches("LL128", 16, 4, placement=placement)


def test_ll128_repeated_full_size_launches_strict_scope():
    _launches("LL128", 16, 4, strict=1, launches=4)


@pytest.mark.parametrize("placement", [0, 1])
def test_simple_repeated_full_size_launches(placement):
    _launches("SIMPLE", 10, 4, placement=placement)


def test_ll_repeated_full_size_launches():
    _launches("LL", 8, 4, launches=6)
