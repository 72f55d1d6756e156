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


def allreduce(x, dtype):
    """x: [N, count] array of raw elements (int32 / float32 / uint16 bf16
    bits).  Returns the [count] array every rank must hold."""
    x = np.asarray(x)
    N = x.shape[0]
    if dtype == "int32":
        acc = x[0].astype(np.int32).view(np.uint32)
        for k in range(1, N):
            acc = acc + x[k].astype(np.int32).view(np.uint32)  # wraps modulo 2^32
        return acc.view(np.int32)
    if dtype == "float32":
        acc = x[0].astype(np.float32)
        for k in range(1, N):
            acc = _add_f32(acc, x[k].astype(np.float32))
        return acc
    if dtype == "bfloat16":
        acc = _bf16_to_f32(x[0])
        for k in range(1, N):
            acc = _add_f32(acc, _bf16_to_f32(x[k]))
        return _round_bf16(acc.astype(np.float64))
    raise ValueError(dtype)


def algorithmic_bytes(message_bytes, nranks):
    """Bytes the one-shot must move when all N ranks share one memory: each
    input read once (N*M) and each output written once (N*M)."""
    return 2 * nranks * message_bytes
