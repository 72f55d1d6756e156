"""Pins of the oracle's reduction operators (prod, max, min, avg) against
hand-derived values, exact arithmetic and numpy; and agreement between the
simulator and the closed form for every operator (no GPU)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import closed_form as cf
from ring_all_reduce_channelmask_amd import workloads

SMALL_BUFF = {"SIMPLE": 8 * 1024, "LL": 8 * 512, "LL128": 8 * 2048}
OPS = ["sum", "prod", "max", "min", "avg"]


def _draw(dtype, shape, seed, op):
    rng = np.random.default_rng(seed)
    if dtype == "int32":
        lim = 2 ** 31 if op != "avg" else 2 ** 20
        return rng.integers(-lim, lim, size=shape).astype(np.int32)
    # products of many values stay in range: draw near 1 for prod
    v = (1 + 0.1 * rng.standard_normal(shape)) if op == "prod" else rng.standard_normal(shape)
    v = v.astype(np.float32)
    return v if dtype == "float32" else workloads._bf16_bits(v.ravel()).reshape(shape)


def _sim(x, op, dtype, proto="SIMPLE", order=(0, 2, 3, 1), mask=0x7, **kw):
    rc, out, _, _ = oracle.allreduce([x], list(order), mask, proto, SMALL_BUFF[proto], 4, dtype,
                                     op=op, **kw)
    assert rc == oracle.OK
    for r in range(1, x.shape[0]):
        np.testing.assert_array_equal(out[0][r], out[0][0])
    return out[0][0]


def _f32(bits_or_vals, dtype):
    return cf._to_f64(bits_or_vals, dtype)


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
def test_simulator_matches_closed_form(op, dtype, proto):
    x = _draw(dtype, (4, 30011), 7, op)
    got = _sim(x, op, dtype, proto, sched=1, seed=3)
    want = cf.allreduce([x], [0, 2, 3, 1], 0x7, proto, SMALL_BUFF[proto], 4, dtype, op=op)[0]
    np.testing.assert_array_equal(got, want)


def test_int32_prod_is_wrapped_exact_product():
    x = _draw("int32", (3, 5000), 1, "prod")
    got = _sim(x, "prod", "int32", order=(0, 1, 2))
    for j in range(0, 5000, 11):
        p = 1
        for r in range(3):
            p *= int(x[r, j])
        p %= 2 ** 32
        assert int(got[j]) == (p - 2 ** 32 if p >= 2 ** 31 else p)


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
def test_max_min_equal_numpy(dtype):
    """Without ties max / min do not depend on the fold order."""
    x = _draw(dtype, (5, 20000), 2, "max")
    vals = x.astype(np.int64) if dtype == "int32" else _f32(x, dtype)
    for op, fn in (("max", np.argmax), ("min", np.argmin)):
        got = _sim(x, op, dtype, order=(0, 3, 1, 4, 2), mask=0x3)
        pick = fn(vals, axis=0)
        np.testing.assert_array_equal(got, x[pick, np.arange(x.shape[1])])


def test_max_keeps_the_first_of_equal_values():
    """Reading: x replaces the partial only when strictly larger.  Ring 0-1,
    rank 0 holds -0.0 and rank 1 holds +0.0 in four elements that all fall in
    chunk 0 (owner rank 0): the fold starts at rank 1, so +0.0 stays."""
    x = np.array([[-0.0] * 4, [0.0] * 4], dtype=np.float32)
    got = _sim(x, "max", "float32", order=(0, 1), mask=0x1)
    assert not np.signbit(got).any()
    got = _sim(x[::-1].copy(), "max", "float32", order=(0, 1), mask=0x1)
    assert np.signbit(got).all()


def _rne_f32(q: Fraction) -> Fraction:
    if q == 0:
        return q
    a = abs(q)
    e = 0
    while a >= 2 ** (e + 1):
        e += 1
    while a < 2 ** e:
        e -= 1
    ulp = Fraction(2) ** (max(e, -126) - 23)
    k = a / ulp
    fl = k.numerator // k.denominator
    rem = k - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl * ulp if q > 0 else -fl * ulp


def test_fp32_prod_rounds_every_hop_exactly():
    """Ring 0-1-2 with four fp32 elements: all of them sit in chunk 0, owned by
    rank 0, so the fold is ((x1 * x2) * x0), each product rounded to nearest
    even in fp32 -- checked in exact rationals."""
    rng = np.random.default_rng(11)
    for _ in range(150):
        x = (rng.standard_normal((3, 4)) * np.exp2(rng.integers(-20, 20, (3, 4)))).astype(
            np.float32)
        got = _sim(x, "prod", "float32", order=(0, 1, 2), mask=0x1)
        for j in range(4):
            f = [Fraction(float(x[r, j])) for r in range(3)]
            want = _rne_f32(_rne_f32(f[1] * f[2]) * f[0])
            assert Fraction(float(got[j])) == want


def test_avg_hand_values():
    """avg = the final sum divided by N, rounded once: int32 truncates toward
    zero (7/4 = 1, -7/4 = -1); fp32 10/4 = 2.5 and 1/3 rounds to 0x3EAAAAAB;
    bf16 1/3 rounds to 0x3EAB (0.333984375)."""
    xi = np.zeros((4, 8), dtype=np.int32)
    xi[0, :4], xi[0, 4:] = 7, -7
    got = _sim(xi, "avg", "int32")
    assert got[:4].tolist() == [1] * 4 and got[4:].tolist() == [-1] * 4
    xf = np.tile(np.array([[1.0], [2.0], [3.0], [4.0]], dtype=np.float32), (1, 8))
    assert (_sim(xf, "avg", "float32") == 2.5).all()
    x3 = np.zeros((3, 8), dtype=np.float32)
    x3[1] = 1.0
    got = _sim(x3, "avg", "float32", order=(0, 1, 2), mask=0x1)
    assert (got.view(np.uint32) == 0x3EAAAAAB).all()
    xb = workloads._bf16_bits(x3.ravel()).reshape(3, 8)
    got = _sim(xb, "avg", "bfloat16", order=(0, 1, 2), mask=0x1)
    assert (got == 0x3EAB).all()


def test_avg_is_sum_then_divide():
    """avg equals the sum's bits divided by N and rounded once, element by
    element, for every dtype."""
    for dtype in ("float32", "bfloat16", "int32"):
        x = _draw(dtype, (4, 9001), 5, "avg")
        s = _sim(x, "sum", dtype)
        a = _sim(x, "avg", dtype)
        if dtype == "int32":
            want = [int(v / 4) if v >= 0 else -int(-v / 4) for v in s.astype(np.int64)]
            np.testing.assert_array_equal(a, np.array(want, dtype=np.int32))
        else:
            q = [Fraction(float(v)) / 4 for v in _f32(s, dtype)]
            if dtype == "float32":
                np.testing.assert_array_equal(a, np.array([float(v) for v in q], dtype=np.float32))
            else:
                # division by 4 is exact unless it leaves the normal range
                np.testing.assert_array_equal(_f32(a, dtype), np.array([float(v) for v in q]))


def test_unknown_op_is_rejected(monkeypatch):
    monkeypatch.setitem(oracle.RED, "bogus", 5)
    rc, _, _, _ = oracle.allreduce([np.ones((2, 8), dtype=np.float32)], [0, 1], 0x1, "SIMPLE",
                                   8192, 4, "float32", op="bogus")
    assert rc == oracle.INVALID


# ------------------------------------------------------------ PreMulSum
def _scalars(dtype, vals):
    v = np.asarray(vals, dtype=np.float64)
    if dtype == "int32":
        return v.astype(np.int32)
    if dtype == "float32":
        return v.astype(np.float32)
    return workloads._bf16_bits(v.astype(np.float32))


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
def test_premulsum_simulator_matches_closed_form(dtype, proto):
    x = _draw(dtype, (4, 20011), 17, "sum")
    sc = _scalars(dtype, [3, -2, 0.5, 7] if dtype != "int32" else [3, -2, 5, 7])
    rc, out, _, _ = oracle.allreduce([x], [0, 2, 3, 1], 0x7, proto, SMALL_BUFF[proto], 4, dtype,
                                     op="premulsum", scalars=sc, sched=1, seed=2)
    assert rc == oracle.OK
    want = cf.allreduce([x], [0, 2, 3, 1], 0x7, proto, SMALL_BUFF[proto], 4, dtype,
                        op="premulsum", scalars=sc)[0]
    for r in range(4):
        np.testing.assert_array_equal(out[0][r], want)


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
def test_premulsum_unit_scalars_is_the_sum(dtype):
    x = _draw(dtype, (4, 9001), 18, "sum")
    got = _sim_premul(x, dtype, _scalars(dtype, [1, 1, 1, 1]))
    np.testing.assert_array_equal(got, _sim(x, "sum", dtype))


def _sim_premul(x, dtype, sc, **kw):
    rc, out, _, _ = oracle.allreduce([x], [0, 2, 3, 1], 0x7, "SIMPLE", SMALL_BUFF["SIMPLE"], 4,
                                     dtype, op="premulsum", scalars=sc, **kw)
    assert rc == oracle.OK
    return out[0][0]


def test_premulsum_power_of_two_scalars_scale_the_sum_exactly():
    """Scaling every input by 1/4 scales each rounded partial by 1/4 too
    (binary floating point, no underflow): the result is the sum's bits
    times 1/4."""
    x = _draw("float32", (4, 9001), 19, "sum")
    got = _sim_premul(x, "float32", _scalars("float32", [0.25] * 4))
    np.testing.assert_array_equal(got, _sim(x, "sum", "float32") * np.float32(0.25))


def test_premulsum_integer_values_are_exact_and_per_rank():
    """Distinct integer scalars on small integer inputs: the result is the
    exact sum of s_r * x_r, so a scalar applied to the wrong rank's input
    shows up."""
    rng = np.random.default_rng(20)
    v = rng.integers(-8, 9, size=(4, 5000)).astype(np.float32)
    s = [1, 2, 3, 4]
    want = sum(s[r] * v[r].astype(np.float64) for r in range(4))
    for direct_read in (False, True):
        got = _sim_premul(v, "float32", _scalars("float32", s), direct_read=direct_read)
        np.testing.assert_array_equal(got.astype(np.float64), want)
    xi = rng.integers(-2 ** 31, 2 ** 31, size=(4, 3000)).astype(np.int32)
    si = [7, -3, 12345, -99999]
    gi = _sim_premul(xi, "int32", _scalars("int32", si))
    for j in range(0, 3000, 13):
        t = sum(si[r] * int(xi[r, j]) for r in range(4)) % 2 ** 32
        assert int(gi[j]) == (t - 2 ** 32 if t >= 2 ** 31 else t)


def test_premulsum_rounds_the_product_once():
    """fp32: float32(1/3) * 3 = 1.0000000298... rounds to 1.0 before the add."""
    x = np.zeros((4, 4), dtype=np.float32)
    x[1] = 3.0
    got = _sim_premul(x, "float32", _scalars("float32", [1.0, np.float32(1 / 3), 1.0, 1.0]))
    assert (got == 1.0).all()


def test_premulsum_direct_read_scales_the_previous_input():
    x = _draw("float32", (4, 30011), 21, "sum")
    sc = _scalars("float32", [0.5, -1.5, 3.0, 1.25])
    base = _sim_premul(x, "float32", sc)
    for kw in (dict(direct=True), dict(direct_read=True), dict(direct=True, direct_read=True)):
        np.testing.assert_array_equal(_sim_premul(x, "float32", sc, **kw), base)
