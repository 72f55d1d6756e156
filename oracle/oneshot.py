"""One-shot AllReduce, written out -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
use this module; the product path never does.

What it computes [C2 "5 Symmetric Memory" and "6.1 LSA"]: with every rank's
buffer reachable by plain loads, one kernel finishes the reduction in a
single hop instead of the ring's 2(N-1) hops.  Each rank loads the element
from all N inputs, reduces in registers and writes its own output.  Every
rank must end with the same bits, so the fold order is fixed:

    acc = x_0 ;  acc = acc + x_k  for k = 1 .. N-1        (user-rank order)

Readings (the pages fix neither): the fold runs in user-rank order; fp32
adds round to fp32 (IEEE, nearest-even) after every addition; bfloat16 inputs
are widened to fp32, accumulated in fp32 exactly as above, and rounded to
bfloat16 (nearest-even) once at the end -- no FIFO sits between the adds, so
nothing forces a rounding per hop; int32 wraps modulo 2^32.

Operators: sum; prod (rounded like the sum, low 32 bits for int32); max / min
(the accumulator is replaced only by a strictly larger / smaller input); avg
(the sum, then divided by N and rounded once; int32 truncates toward zero).

[C2] "cishoon.github.io/posts/ai-infra/nccl" (NCCL notes: symmetric memory,
LSA device API, one-shot AllReduce).
"""
import numpy as np

from .closed_form import _round_bf16


def _bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _add_f32(a, b):
    """IEEE fp32 addition, round to nearest even.  The exact sum of two fp32
    values rounded to binary64 and then to fp32 equals the directly rounded
    sum: 53 >= 2*24 + 2, so the double rounding is innocuous."""
    return (a.astype(np.float64) + b.astype(np.float64)).astype(np.float32)


def _mul_f32(a, b):
    """IEEE fp32 product: exact in binary64 (at most 48 significant bits),
    then rounded once."""
    return (a.astype(np.float64) * b.astype(np.float64)).astype(np.float32)


def _step(acc, v, op, wide):
    """acc <- acc (op) v.  ``wide`` is the accumulator's numpy type."""
    if op in ("max", "min"):
        take = v > acc if op == "max" else v < acc
        return np.where(take, v, acc)
    if wide == "int":
        au, vu = acc.view(np.uint32), v.view(np.uint32)
        if op == "prod":
            return ((au.astype(np.uint64) * vu.astype(np.uint64)) & 0xFFFFFFFF) \
                .astype(np.uint32).view(np.int32)
        return (au + vu).view(np.int32)  # wraps modulo 2^32
    return _mul_f32(acc, v) if op == "prod" else _add_f32(acc, v)


def _scale(s, x, dtype):
    """PreMulSum: rank input times its scalar, in the accumulator's precision
    (fp32 rounds once; bf16 x bf16 is exact in fp32; int32 keeps the low 32
    bits)."""
    if dtype == "int32":
        su = np.asarray(s).astype(np.int32).view(np.uint32).astype(np.uint64)
        xu = x.astype(np.int32).view(np.uint32).astype(np.uint64)
        return ((su * xu) & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
    if dtype == "float32":
        return _mul_f32(np.float32(s) * np.ones_like(x, dtype=np.float32), x.astype(np.float32))
    return _mul_f32(_bf16_to_f32(np.full(x.shape, s, dtype=np.uint16)), _bf16_to_f32(x))


def allreduce(x, dtype, op="sum", scalars=None):
    """x: [N, count] array of raw elements (int32 / float32 / uint16 bf16
    bits).  Returns the [count] array every rank must hold.  PreMulSum
    (``scalars``: one payload-type element per rank) scales each input in
    the accumulator's precision, then sums."""
    x = np.asarray(x)
    N = x.shape[0]
    if op == "premulsum":
        scaled = [_scale(scalars[r], x[r], dtype) for r in range(N)]
        if dtype == "int32":
            acc = scaled[0]
            for k in range(1, N):
                acc = _step(acc, scaled[k], "sum", "int")
            return acc
        acc = scaled[0]
        for k in range(1, N):
            acc = _add_f32(acc, scaled[k])
        return acc if dtype == "float32" else _round_bf16(acc.astype(np.float64))
    if dtype == "int32":
        acc = x[0].astype(np.int32)
        for k in range(1, N):
            acc = _step(acc, x[k].astype(np.int32), op, "int")
        if op == "avg":
            q = np.abs(acc.astype(np.int64)) // N
            acc = np.where(acc < 0, -q, q).astype(np.int32)
        return acc
    if dtype == "float32":
        acc = x[0].astype(np.float32)
        for k in range(1, N):
            acc = _step(acc, x[k].astype(np.float32), op, "f32")
        if op == "avg":
            acc = (acc.astype(np.float64) / N).astype(np.float32)  # 53 >= 2*24+2: one rounding
        return acc
    if dtype == "bfloat16":
        acc = _bf16_to_f32(x[0])
        for k in range(1, N):
            acc = _step(acc, _bf16_to_f32(x[k]), op, "f32")
        a64 = acc.astype(np.float64)
        return _round_bf16(a64 / N if op == "avg" else a64)
    raise ValueError(dtype)


def algorithmic_bytes(message_bytes, nranks):
    """Bytes the one-shot must move when all N ranks share one memory: each
    input read once (N*M) and each output written once (N*M)."""
    return 2 * nranks * message_bytes
