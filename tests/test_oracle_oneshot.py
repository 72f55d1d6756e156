"""Pins of the one-shot AllReduce oracle against values fixed by hand, by
exact arithmetic and by library routines (no GPU)."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import oneshot
from ring_all_reduce_channelmask_amd import workloads


def _f32_rne_exact(q: Fraction) -> np.float32:
    """Exact rational round-to-nearest-even to fp32 (normal range)."""
    if q == 0:
        return np.float32(0)
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
    v = np.float32(float(fl * ulp))
    return -v if q < 0 else v


def test_fold_order_hand_example():
    """[2^24, 1, 1, -2^24]: in rank order 2^24 + 1 ties to even (2^24) twice,
    then cancels to 0; the exact sum is 2 and the reverse order gives 2."""
    x = np.array([[2.0 ** 24], [1.0], [1.0], [-2.0 ** 24]], dtype=np.float32)
    assert oneshot.allreduce(x, "float32")[0] == 0.0
    assert oneshot.allreduce(x[::-1], "float32")[0] == 2.0


def test_bf16_rounds_once_at_the_end():
    """[1, 2^-8, 2^-8, 0] in bf16: accumulated in fp32 the sum is exactly
    1 + 2^-7 (bits 0x3F81); rounding to bf16 after every add would tie to even
    at 1 + 2^-8 twice and give 1.0 (0x3F80)."""
    x = workloads._bf16_bits(np.array([1.0, 2.0 ** -8, 2.0 ** -8, 0.0], dtype=np.float32))
    assert int(oneshot.allreduce(x.reshape(4, 1), "bfloat16")[0]) == 0x3F81


def test_fp32_adds_equal_exact_rational_rne():
    """Each step is the exact rational sum rounded to nearest even in fp32."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((5, 300)) * np.exp2(rng.integers(-30, 30, (5, 300)))).astype(
        np.float32)
    got = oneshot.allreduce(x, "float32")
    for j in range(x.shape[1]):
        acc = np.float32(x[0, j])
        for k in range(1, 5):
            acc = _f32_rne_exact(Fraction(float(acc)) + Fraction(float(x[k, j])))
        assert got[j] == acc, j


def test_two_ranks_is_numpy_float32_add():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 10000)).astype(np.float32)
    np.testing.assert_array_equal(oneshot.allreduce(x, "float32"), x[0] + x[1])


def test_int32_is_wrapped_exact_sum():
    rng = np.random.default_rng(5)
    for N in (2, 3, 8, 64):
        x = rng.integers(-2 ** 31, 2 ** 31, size=(N, 500)).astype(np.int32)
        got = oneshot.allreduce(x, "int32")
        for j in range(0, 500, 7):
            s = sum(int(v) for v in x[:, j]) % 2 ** 32
            assert int(got[j]) == (s - 2 ** 32 if s >= 2 ** 31 else s)


def test_integer_valued_floats_are_exact():
    rng = np.random.default_rng(6)
    for dtype in ("float32", "bfloat16"):
        v = rng.integers(-8, 9, size=(16, 4000)).astype(np.float32)
        x = v if dtype == "float32" else workloads._bf16_bits(v.ravel()).reshape(v.shape)
        got = oneshot.allreduce(x, dtype)
        f = got if dtype == "float32" else \
            (got.astype(np.uint32) << 16).view(np.float32)
        np.testing.assert_array_equal(f, v.sum(axis=0))


@pytest.mark.parametrize("N", [2, 4, 8, 64])
def test_error_bound(N):
    """fp32: |fold - exact| <= gamma_{N-1} sum|x| (recursive summation bound,
    Higham, Accuracy and Stability of Numerical Algorithms, ch. 4); bf16 adds
    one final rounding, |r - s| <= 2^-8 |s| for the fp32 sum s."""
    rng = np.random.default_rng(N)
    v = rng.standard_normal((N, 20000)).astype(np.float32)
    exact = v.astype(np.float64).sum(axis=0)
    u = 2.0 ** -24
    gamma = (N - 1) * u / (1 - (N - 1) * u)
    s = oneshot.allreduce(v, "float32").astype(np.float64)
    assert (np.abs(s - exact) <= gamma * np.abs(v.astype(np.float64)).sum(axis=0)).all()
    xb = workloads._bf16_bits(v.ravel()).reshape(v.shape)
    vb = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    sb = oneshot.allreduce(xb, "bfloat16")
    r = (sb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ex_b = vb.sum(axis=0)
    bound = gamma * np.abs(vb).sum(axis=0) * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(ex_b) + 2.0 ** -133
    assert (np.abs(r - ex_b) <= bound).all()


def test_algorithmic_bytes():
    assert oneshot.algorithmic_bytes(64 << 20, 4) == 8 * (64 << 20)


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
def test_max_min_equal_numpy(dtype):
    rng = np.random.default_rng(21)
    if dtype == "int32":
        x = rng.integers(-2 ** 31, 2 ** 31, size=(6, 5000)).astype(np.int32)
        vals = x.astype(np.int64)
    else:
        v = rng.standard_normal((6, 5000)).astype(np.float32)
        x = v if dtype == "float32" else workloads._bf16_bits(v.ravel()).reshape(v.shape)
        vals = v if dtype == "float32" else (x.astype(np.uint32) << 16).view(np.float32)
    for op, fn in (("max", np.argmax), ("min", np.argmin)):
        np.testing.assert_array_equal(oneshot.allreduce(x, dtype, op),
                                      x[fn(vals, axis=0), np.arange(5000)])


def test_prod_hand_values_and_int32_wrap():
    """fp32: 2 * 0.5 * 4 * 8 = 32 exactly; (1 + 2^-12) * (1 + 2^-12) = 1 + 2^-11
    + 2^-24 ties to even at 1 + 2^-11.  int32: the low 32 bits of the exact
    product."""
    x = np.array([[2.0, 1 + 2 ** -12], [0.5, 1 + 2 ** -12], [4.0, 1.0], [8.0, 1.0]],
                 dtype=np.float32)
    got = oneshot.allreduce(x, "float32", "prod")
    assert got[0] == 32.0 and got[1] == np.float32(1 + 2 ** -11)
    rng = np.random.default_rng(22)
    xi = rng.integers(-2 ** 31, 2 ** 31, size=(5, 300)).astype(np.int32)
    gi = oneshot.allreduce(xi, "int32", "prod")
    for j in range(300):
        p = 1
        for r in range(5):
            p *= int(xi[r, j])
        p %= 2 ** 32
        assert int(gi[j]) == (p - 2 ** 32 if p >= 2 ** 31 else p)


def test_bf16_prod_accumulates_in_fp32():
    """bf16 (1 + 2^-7) squared is 1 + 2^-6 + 2^-14: kept in the fp32
    accumulator, times 1 it still rounds to 1 + 2^-6 (0x3F82) once at the end;
    and (1 + 2^-7)^2 * (1 + 2^-7) = 1 + 3*2^-7 + ... rounds to 0x3F83."""
    one_p = 1 + 2 ** -7
    x = workloads._bf16_bits(np.array([[one_p, one_p], [one_p, one_p], [1.0, one_p]],
                                      dtype=np.float32).ravel()).reshape(3, 2)
    got = oneshot.allreduce(x, "bfloat16", "prod")
    assert int(got[0]) == 0x3F82 and int(got[1]) == 0x3F83


def test_avg_hand_values():
    xi = np.array([[7, -7], [0, 0], [0, 0], [0, 0]], dtype=np.int32)
    assert oneshot.allreduce(xi, "int32", "avg").tolist() == [1, -1]
    xf = np.array([[1.0, 1.0], [2.0, 0.0], [3.0, 0.0]], dtype=np.float32)
    got = oneshot.allreduce(xf, "float32", "avg")
    assert got[0] == 2.0 and got.view(np.uint32)[1] == 0x3EAAAAAB
    xb = workloads._bf16_bits(xf.ravel()).reshape(3, 2)
    assert oneshot.allreduce(xb, "bfloat16", "avg").tolist() == [0x4000, 0x3EAB]


def test_premulsum_pins():
    rng = np.random.default_rng(30)
    v = rng.integers(-8, 9, size=(5, 3000)).astype(np.float32)
    s = np.array([1, -2, 3, 4, -5], dtype=np.float32)
    np.testing.assert_array_equal(oneshot.allreduce(v, "float32", "premulsum", s).astype(np.float64),
                                  sum(float(s[r]) * v[r].astype(np.float64) for r in range(5)))
    x = rng.standard_normal((4, 3000)).astype(np.float32)
    np.testing.assert_array_equal(oneshot.allreduce(x, "float32", "premulsum", np.ones(4, np.float32)),
                                  oneshot.allreduce(x, "float32"))
    xi = rng.integers(-2 ** 31, 2 ** 31, size=(3, 500)).astype(np.int32)
    si = np.array([3, -7, 1001], dtype=np.int32)
    gi = oneshot.allreduce(xi, "int32", "premulsum", si)
    for j in range(500):
        t = sum(int(si[r]) * int(xi[r, j]) for r in range(3)) % 2 ** 32
        assert int(gi[j]) == (t - 2 ** 32 if t >= 2 ** 31 else t)
    # bf16: scalar x input exact in the fp32 accumulator, rounded once at the end
    xb = workloads._bf16_bits(np.array([[1.0], [2.0 ** -8]], dtype=np.float32).ravel()).reshape(2, 1)
    sb = workloads._bf16_bits(np.array([1.0, 2.0], dtype=np.float32))
    assert int(oneshot.allreduce(xb, "bfloat16", "premulsum", sb)[0]) == 0x3F81
