"""Bandwidth figures of an AllReduce, in the convention of the NCCL course
pages: algBW = M / t and busBW = algBW * 2(N-1)/N with GB = 1e9, where M is
the message size of one rank.  Each rank sends 2(N-1) chunks of M/N
[NCCL 专家课程 12, "为什么是 2(N-1) 次发送"].

The algorithmic HBM bytes of one ring AllReduce on a single device that hosts
all N ranks count, per loop of N chunks of M/N each, the reads and writes
every primitive must make (f = FIFO bytes per payload byte: Simple 1, LL 2,
LL128 16/15):

    send 1+f, recvReduceSend 1+2f, recvReduceCopySend 2+2f,
    recvCopySend 1+2f, recv 1+f

Summed over the N ranks: B = [4 + 4f + 2(N-2)(2f+1)] * M.
"""
from fractions import Fraction

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD's published peak (8 TB/s)

FIFO_FACTOR = {"SIMPLE": Fraction(1), "LL": Fraction(2), "LL128": Fraction(16, 15)}


def algbw_gbps(message_bytes: float, seconds: float) -> float:
    return message_bytes / seconds / 1e9


def busbw_gbps(message_bytes: float, seconds: float, nranks: int) -> float:
    return algbw_gbps(message_bytes, seconds) * 2.0 * (nranks - 1) / nranks


def algorithmic_bytes(message_bytes: int, nranks: int, proto: str, direct: bool = False,
                      direct_read: bool = False) -> float:
    """HBM bytes the ring schedule must move for one collective, all ranks.

    The direct write (Simple) puts the all-gather half straight into the
    next rank's receive buffer: recvReduceCopySend moves f + 3 (FIFO in, own
    input, own output, next output), recvCopySend 2 (own output in, next
    output out), recv 0.  Summed: B = [4 + 2f + (N-2)(3 + 2f)] * M, which is
    (5N-4) M for Simple.  The direct read (Simple) drops the loop's opening
    send (1 + f) and has the next rank read the raw input from the sender's
    buffer instead of the FIFO (the same f = 1 bytes): 2 M less."""
    f = FIFO_FACTOR[proto]
    if direct:
        per_m = (1 + f) + (f + 3) + (nranks - 2) * ((1 + 2 * f) + 2)
    else:
        per_m = 4 + 4 * f + 2 * (nranks - 2) * (2 * f + 1)
    if direct_read:
        per_m -= 1 + f
    return float(per_m * message_bytes)


def oneshot_algorithmic_bytes(message_bytes: int, nranks: int) -> float:
    """HBM bytes of the one-shot AllReduce with all ranks in one memory: every
    input read once and every output written once, 2 N M."""
    return float(2 * nranks * message_bytes)
