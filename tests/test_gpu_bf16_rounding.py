"""bf16 rounding in the kernel, edge by edge.  With two ranks every output
element is one hop, RNE_bf16(x0 op x1) (avg: the sum over 2, rounded once;
PreMulSum: each input scaled and rounded, then the sum), so each input pair
below aims at one edge of round-to-nearest-even: exact ties to even in both
directions, sums that overflow to infinity or stay at the largest finite
value, subnormal sums, signed zeros, products that round, plus random pairs.
All three protocols, compared bit for bit with the oracle (which rounds the
exact binary64 result)."""
import numpy as np
import pytest

import oracle

from .gpu_util import assert_bits_equal, run_hip

pytestmark = pytest.mark.gpu

SMALL_BUFF = {"SIMPLE": 8 * 1024, "LL": 8 * 512, "LL128": 8 * 2048}


def _edge_pairs(seed):
    """[2, n] uint16 bf16 bit patterns (no NaN)."""
    rng = np.random.default_rng(seed)
    cols = []
    # ties: a normal bf16 a and b = +-half an ulp of a, so a + b lies exactly
    # halfway between two bf16 values (the even one must win)
    a = rng.integers(0x0080, 0x7F00, 20000, dtype=np.uint32) | (rng.integers(0, 2, 20000, dtype=np.uint32) << 15)
    exp = (a >> 7) & 0xFF
    half = ((exp - 8).clip(1, 254) << 7).astype(np.uint32) | (rng.integers(0, 2, 20000, dtype=np.uint32) << 15)
    cols.append(np.stack([a, half]))
    # near-ties: a plus 3/4 or 1/4 of an ulp (rounds away from / towards a)
    q = (((exp - 9).clip(1, 254) << 7) | (1 << 6)).astype(np.uint32)
    cols.append(np.stack([a, q]))
    # overflow: the largest finite bf16 plus itself, plus half an ulp, plus less
    big = np.full(300, 0x7F7F, np.uint32) | (rng.integers(0, 2, 300, dtype=np.uint32) << 15)
    cols.append(np.stack([big, big]))
    # 0x7F7F = (2 - 2^-7) * 2^127, whose ulp is 2^120: half an ulp (2^119,
    # exponent field 0xF6) makes a tie that rounds to even, up to infinity;
    # a quarter ulp (0xF5) rounds back down to 0x7F7F
    cols.append(np.stack([big, (big & 0x8000) | (0xF6 << 7)]))
    cols.append(np.stack([big, (big & 0x8000) | (0xF5 << 7)]))
    # subnormals: exponent field 0, any mantissa and sign
    sub = rng.integers(0, 0x80, (2, 5000), dtype=np.uint32) | (rng.integers(0, 2, (2, 5000), dtype=np.uint32) << 15)
    cols.append(sub)
    # signed zeros
    z = np.array([[0x0000, 0x8000, 0x8000, 0x0000], [0x8000, 0x8000, 0x0000, 0x0000]], np.uint32)
    cols.append(np.repeat(z, 25, axis=1))
    # random finite pairs over the whole exponent range
    r = rng.integers(0, 0x7F80, (2, 20000), dtype=np.uint32) | (rng.integers(0, 2, (2, 20000), dtype=np.uint32) << 15)
    cols.append(r)
    x = np.concatenate(cols, axis=1).astype(np.uint16)
    assert not (((x & 0x7FFF) > 0x7F80).any())  # no NaN
    return np.ascontiguousarray(x)


@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
@pytest.mark.parametrize("op", ["sum", "prod", "avg", "premulsum"])
def test_bf16_rounding_edges(proto, op):
    import ring_all_reduce_channelmask_amd as rar
    x = _edge_pairs(91)
    buff = SMALL_BUFF[proto]
    comm = rar.Comm(2, [0, 1], 0x3, proto=proto, buff_size=buff,
                    chunk_steps=4 if proto == "SIMPLE" else 0, lanes=2, waves=4)
    scalars = None
    if op == "premulsum":
        # 1.5 and -0.75 as bf16: products that round, then a sum that rounds
        scalars = [np.array([0x3FC0, 0xBF40], np.uint16)]
    got = run_hip(comm, [x], "bfloat16", op=op, scalars=scalars)[0]
    comm.close()
    rc, want, _, _ = oracle.allreduce([x], [0, 1], 0x3, proto, buff, 4, "bfloat16", op=op,
                                      scalars=np.stack(scalars) if scalars else None)
    assert rc == oracle.OK
    for r in range(2):
        assert_bits_equal(got[r], want[0][r], f"{proto} {op} rank {r}")
