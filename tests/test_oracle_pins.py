"""Pins of the CPU oracle against what the NCCL course pages print or fix.

Each test names the page and section it checks.  None of these tests touch the
GPU or the HIP library.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import closed_form as cf
from ring_all_reduce_channelmask_amd import metrics, workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")
# small FIFOs (valid for each protocol) so that short inputs still run many loops
SMALL_BUFF = {"SIMPLE": 8 * 1024, "LL": 8 * 512, "LL128": 8 * 2048}


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- ring set-up
def test_ring_index_tables():
    """Course 12, "ring index 如何计算": both printed tables."""
    g = gold("ring_tables.json")["ring_index_tables"]
    for key in ("0-1-2-3", "0-2-3-1"):
        idx, prv, nxt = oracle.ring_setup(g[key]["order"])
        for rank, ring_index, p, n in g[key]["rows"]:
            assert (idx[rank], prv[rank], nxt[rank]) == (ring_index, p, n), (key, rank)


def test_acceptance_answers():
    """Course 12, "验收题" questions 1 and 2."""
    g = gold("ring_tables.json")["acceptance"]
    q1 = g["q1"]
    idx, prv, nxt = oracle.ring_setup(q1["order"])
    assert (idx[q1["rank"]], prv[q1["rank"]], nxt[q1["rank"]]) == \
        (q1["ring_index"], q1["prev"], q1["next"])
    q2 = g["q2"]
    assert oracle.ring_schedule(q2["nranks"], q2["ring_index"])[0] == ("send", q2["first_send_chunk"])


def test_ring_rotation_is_same_ring():
    """Course 12, "ring index 如何计算": the index is the distance from rank 0,
    so a rotated listing of the same ring gives the same indices."""
    a = oracle.ring_setup([0, 2, 3, 1])
    b = oracle.ring_setup([3, 1, 0, 2])
    assert a == b


@pytest.mark.parametrize("order", [[0, 1, 1, 2], [0, 1, 2, 4], [0], [], [-1, 0, 1]])
def test_ring_validation_rejects(order):
    """Course 12, "Graph 如何变成完整 ring": a ring must visit every rank once
    and loop back."""
    assert oracle.ring_setup(order) is None


# ---------------------------------------------------------------- schedule
def test_first_send_table():
    """Course 12, "源码步骤一：初始 send": rank -> first chunk, next."""
    g = gold("ring_tables.json")["first_send"]
    idx, _, nxt = oracle.ring_setup(g["order"])
    for rank, chunk, n in g["rows"]:
        assert oracle.ring_schedule(4, idx[rank])[0] == ("send", chunk)
        assert nxt[rank] == n


def test_rank0_schedule_from_simulator_log():
    """Course 12, "rank0 的完整操作序列": the 7 rows of rank 0 on ring 0-1-2-3,
    as executed by the state machine (not just the schedule generator)."""
    g = gold("ring_tables.json")["rank0_schedule"]
    x = np.ones((4, 1024), dtype=np.float32)
    rc, _, _, calls = oracle.allreduce([x], g["order"], 0x1, "SIMPLE", 65536, 4, "float32",
                                       log_calls=True)
    assert rc == oracle.OK
    r0 = [c for c in calls if c["rank"] == 0]
    assert len(r0) == len(g["rows"])
    _, prv, nxt = oracle.ring_setup(g["order"])
    for c, (seq, phase, prim, chunk, recv_from, send_to) in zip(r0, g["rows"]):
        assert c["op"] == prim and c["chunk"] == chunk, (seq, c)
        receives = prim != "send"
        sends = prim != "directRecv"
        assert (prv[0] if receives else None) == recv_from
        assert (nxt[0] if sends else None) == send_to


def test_rank0_chunks_by_phase():
    """Course 12, steps two, four and five: rank 0's chunk lists."""
    g = gold("ring_tables.json")["rank0_chunks_by_phase"]
    rows = oracle.ring_schedule(4, 0)
    for prim, chunks in g.items():
        if prim.startswith("_"):
            continue
        assert [c for (p, c) in rows if p == prim] == chunks


@pytest.mark.parametrize("N", [2, 3, 4, 5, 8, 16])
def test_schedule_counts(N):
    """Course 12, "为什么是 2(N-1) 次发送" and "Schedule 生成器的断言": 2N-1
    rows, 2N-2 sends and receives per rank, every chunk covered."""
    total = 0
    for ix in range(N):
        rows = oracle.ring_schedule(N, ix)
        total += len(rows)
        assert len(rows) == 2 * N - 1
        assert sum(p != "directRecv" for p, _ in rows) == 2 * N - 2
        assert sum(p != "send" for p, _ in rows) == 2 * N - 2
        assert {c for _, c in rows} == set(range(N))
    if N == 4:
        g = gold("ring_tables.json")["schedule_generator"]
        assert total == g["rows_total"]


# ---------------------------------------------------------------- geometry
def test_simple_chunk_geometry_small_buffers():
    """Course 23, "Buffer 到 Chunk 的实测公式": step = buffer/8, chunk = 4 steps.
    Observed in the simulator's primitive calls at 4 ranks x 4 channels with
    enough data that full loops occur (64 KiB and 1 MiB buffers)."""
    g = gold("chunk_geometry.json")["simple"]
    for buff, step, chunk in g["rows"][:2]:
        assert buff // g["nccl_steps"] == step
        celems = chunk // 4
        count = g["channels"] * g["nranks"] * celems * 2  # two full loops per channel
        x = np.zeros((4, count), dtype=np.float32)
        rc, _, _, calls = oracle.allreduce([x], [0, 1, 2, 3], 0xF, "SIMPLE", buff, 4, "float32",
                                           log_calls=True)
        assert rc == oracle.OK
        assert {c["nelem"] * 4 for c in calls} == {chunk}


def test_simple_chunk_geometry_4m():
    """Course 23, same table, 4 MiB buffer -> 2 MiB chunk (checked through the
    channel split; a full simulation at this size is in the slow suite)."""
    g = gold("chunk_geometry.json")["simple"]
    buff, step, chunk = g["rows"][2]
    pieces, cmax = oracle.geometry(4, 0xF, "SIMPLE", buff, 4, "float32", [16 << 20])
    assert cmax * 4 == chunk
    assert cf.chunk_max("SIMPLE", buff, 4, "float32") * 4 == chunk


@pytest.mark.slow
def test_simple_chunk_geometry_4m_full_run():
    """Course 23 TRACE shape itself: 4 channels, 64 MiB, 4 MiB buffer -> 2 MiB chunks."""
    x = np.zeros((4, 16 << 20), dtype=np.float32)
    rc, _, _, calls = oracle.allreduce([x], [0, 1, 2, 3], 0xF, "SIMPLE", 4 << 20, 4, "float32",
                                       log_calls=True)
    assert rc == oracle.OK
    assert {c["nelem"] * 4 for c in calls} == {2 << 20}


def test_ll_ll128_default_chunks_and_payload():
    """Course 23, "LL：Data 与 Flag 同 Line" (32 KiB chunk, 8 of 16 bytes) and
    "LL128：15/16 Payload" (576000-byte chunk, 120 of 128 bytes)."""
    g = gold("chunk_geometry.json")
    for proto, key, buff in (("LL", "ll", 512 * 1024), ("LL128", "ll128", 4915200)):
        cmax_bytes = cf.chunk_max(proto, buff, 4, "float32") * 4
        assert cmax_bytes == g[key]["default_chunk_bytes"]
        n = g[key]["default_chunk_bytes"] // 4
        x = np.ones((2, 2 * 2 * n), dtype=np.float32)  # two full loops at N=2
        rc, _, st, calls = oracle.allreduce([x], [0, 1], 0x1, proto, buff, 4, "float32",
                                            log_calls=True)
        assert rc == oracle.OK
        assert {c["nelem"] * 4 for c in calls} == {g[key]["default_chunk_bytes"]}
        ratio = Fraction(st.wire_sent[0], st.payload_sent[0])
        assert ratio == Fraction(g[key]["line_bytes"], g[key]["payload_per_line"])


def test_grid_is_popcount_and_block_n_is_nth_bit():
    """Course 23, "Kernel 如何把 Block 映射到 Channel" and the Nsight gridX
    rows: one block per set bit, block n runs the n-th set bit."""
    g = gold("chunk_geometry.json")["grid"]
    for nch, gridx in g["rows"]:
        mask = (1 << nch) - 1
        x = np.ones((4, 4096 * nch), dtype=np.int32)
        rc, _, _, calls = oracle.allreduce([x], [0, 1, 2, 3], mask, "SIMPLE", 65536, 4, "int32",
                                           log_calls=True)
        assert rc == oracle.OK
        assert len({c["channel_id"] for c in calls}) == gridx
    mask = workloads.WORKLOADS["fused_ll"].mask
    pieces, _ = oracle.geometry(4, mask, "LL", 512 * 1024, 4, "bfloat16", [7168] * 104)
    by_dense = sorted({(p["channel"], p["channel_id"]) for p in pieces})
    assert [cid for _, cid in by_dense] == [0, 1, 4, 6, 8, 9, 11]
    assert [n for n, _ in by_dense] == list(range(7))


def test_fused_group_split():
    """The fused group of 104 collectives over 7 sparse channels: every
    collective is covered exactly once, pieces are contiguous per channel."""
    pieces, cmax = oracle.geometry(4, 0b101101010011, "LL", 512 * 1024, 4, "bfloat16",
                                   [7168] * 104)
    assert cmax == 16384
    per_work = {}
    for p in pieces:
        per_work.setdefault(p["work"], []).append((p["grid_offset"], p["channel_count"]))
    for w in range(104):
        segs = sorted(per_work[w])
        pos = 0
        for off, cnt in segs:
            assert off == pos
            pos += cnt
        assert pos == 7168
    counts = [sum(1 for p in pieces if p["channel"] == n) for n in range(7)]
    assert counts == [15, 16, 16, 16, 16, 16, 15]


def test_invalid_parameters():
    x = np.ones((4, 64), dtype=np.float32)
    assert oracle.allreduce([x], [0, 1, 2, 3], 0, "SIMPLE", 65536, 4, "float32")[0] == oracle.INVALID
    assert oracle.allreduce([x], [0, 1, 2, 3], 1, "SIMPLE", 65536, 3, "float32")[0] == oracle.INVALID
    assert oracle.allreduce([x], [0, 1, 2, 2], 1, "SIMPLE", 65536, 4, "float32")[0] == oracle.INVALID
    assert oracle.allreduce([x], [0, 1, 2, 3], 1, "LL128", 1000, 4, "float32")[0] == oracle.INVALID


# ---------------------------------------------------------------- credit / flags
def test_fault_model_27_cases():
    """Course 23, "状态机故障注入": 9 scenarios x fifo_steps 2/4/8."""
    g = gold("fault_model.json")
    n = 0
    for proto, fault, expected, _ in g["rows"]:
        for slots in g["fifo_steps"]:
            outcome, done, consumed, bad = oracle.stream_fault(proto, fault, slots,
                                                               g["stream_steps"])
            assert outcome == expected, (proto, fault, slots)
            if fault == "none":
                assert done == consumed == g["stream_steps"]
            if fault == "drop_recv_head":
                assert done == slots  # stalls after exactly `slots` steps
            if fault == "ll_constant_flag":
                assert bad == slots  # the first slot wrap is where the ABA bites
            n += 1
    assert n == 27


@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
def test_collective_without_head_credit_deadlocks(proto):
    """A whole collective with receivers that never free slots stalls; the
    same collective with credit completes (Course 23, 排障树: a hang near the
    N-th chunk where N ~ NCCL_STEPS points at recv head credit)."""
    x = np.ones((4, 1 << 16), dtype=np.int32)
    buff = SMALL_BUFF[proto]
    rc, _, st, _ = oracle.allreduce([x], [0, 1, 2, 3], 0x1, proto, buff, 4, "int32",
                                    drop_recv_head=True)
    assert rc == oracle.DEADLOCK
    assert st.deadlock_send_step <= 8
    rc, out, _, _ = oracle.allreduce([x], [0, 1, 2, 3], 0x1, proto, buff, 4, "int32")
    assert rc == oracle.OK and (out[0] == 4).all()


@pytest.mark.parametrize("N", [2, 3, 4, 8])
def test_chunk_of_all_slots_deadlocks(N):
    """Why a chunk is at most NCCL_STEPS/2 steps (the pages' ALLREDUCE_CHUNKSTEPS
    = 4 of 8 slots, Course 23 "Buffer 到 Chunk 的实测公式"): with chunkSteps = 8
    the opening send fills every slot of the next rank's FIFO, and the next
    call both receives and sends, so every rank waits for send credit that
    only the blocked next rank could give.  chunkSteps 2 and 4 complete."""
    x = np.ones((N, 4096), dtype=np.int32)
    order = list(range(N))
    rc, _, st, _ = oracle.allreduce([x], order, 0x1, "SIMPLE", 8 * 1024, 8, "int32")
    assert rc == oracle.DEADLOCK
    assert st.deadlock_send_step == 8 and st.deadlock_recv_step == 0
    for cs in (2, 4):
        rc, out, _, _ = oracle.allreduce([x], order, 0x1, "SIMPLE", 8 * 1024, cs, "int32")
        assert rc == oracle.OK and (out[0] == N).all()


def test_empty_slices_still_post():
    """Course 23, "Slice Size" and 常见错误: empty slices must still wait and
    post, or ranks drift.  N=8 ranks and 8 fp32 elements leave most chunks
    empty; the collective must complete with the right sums."""
    rng = np.random.default_rng(11)
    x = rng.integers(-8, 9, size=(8, 8)).astype(np.float32)
    for proto in ("SIMPLE", "LL", "LL128"):
        rc, out, _, _ = oracle.allreduce([x], list(range(8)), 0x3, proto,
                                         workloads.DEFAULT_BUFF[proto], 4, "float32")
        assert rc == oracle.OK
        for r in range(8):
            np.testing.assert_array_equal(out[0][r], x.sum(axis=0))


# ---------------------------------------------------------------- values
def _wrap_sum(x):
    return (x.astype(np.int64).sum(axis=0) & 0xFFFFFFFF).astype(np.uint32).view(np.int32)


@pytest.mark.parametrize("proto", ["SIMPLE", "LL", "LL128"])
def test_int32_brute_force_random(proto):
    """Integer sums are order-free: every rank's output equals the plain sum
    (two's-complement wrap) for ragged sizes, several rings and masks."""
    rng = np.random.default_rng(7)
    for N, count, mask in [(2, 1, 0x1), (3, 77, 0x5), (4, 1000, 0xF), (5, 4099, 0x3),
                           (8, 3000, 0xFF), (4, 0, 0x1)]:
        order = list(rng.permutation(N))
        x = rng.integers(-2 ** 31, 2 ** 31, size=(N, count)).astype(np.int32)
        buff = SMALL_BUFF[proto]
        rc, out, _, _ = oracle.allreduce([x], order, mask, proto, buff, 4, "int32")
        assert rc == oracle.OK
        for r in range(N):
            np.testing.assert_array_equal(out[0][r], _wrap_sum(x))
        np.testing.assert_array_equal(
            cf.allreduce([x], order, mask, proto, buff, 4, "int32")[0], _wrap_sum(x))


def test_integer_valued_float_brute_force():
    """The 4 KiB workload: integer-valued fp32 in [-8, 8]; sums of at most 8
    such values are exact, so any order gives the plain sum."""
    w = workloads.WORKLOADS["simple_4k"]
    x = workloads.inputs_for(w)[0]
    rc, out, _, _ = oracle.allreduce([x], w.ring_order, w.mask, w.proto, w.buff_size,
                                     w.chunk_steps, w.dtype)
    assert rc == oracle.OK
    for r in range(w.nranks):
        np.testing.assert_array_equal(out[0][r], x.astype(np.float64).sum(axis=0))


def test_tiny_exhaustive_int32():
    """N in {2,3,4}, every ring order, every count 0..64, every protocol."""
    rng = np.random.default_rng(3)
    for N in (2, 3, 4):
        for order in itertools.permutations(range(N)):
            for proto in ("SIMPLE", "LL", "LL128"):
                buff = {"SIMPLE": 8 * 256, "LL": 8 * 64, "LL128": 8 * 256}[proto]
                for count in range(0, 65):
                    x = rng.integers(-1000, 1000, size=(N, count)).astype(np.int32)
                    mask = int(rng.integers(1, 16))
                    rc, out, _, _ = oracle.allreduce([x], list(order), mask, proto, buff, 2,
                                                     "int32")
                    assert rc == oracle.OK
                    want = x.sum(axis=0).astype(np.int32)
                    for r in range(N):
                        np.testing.assert_array_equal(out[0][r], want)


def test_fold_order_worked_example():
    """Ring 0-2-3-1 (Course 12, "先固定三个坐标系": position 0 -> rank 0,
    1 -> rank 2, 2 -> rank 3, 3 -> rank 1).  The chunk owned by position c is
    started by position c+1 and finished by its owner (steps one to three).
    With 16 fp32 elements every chunk holds 4 of them; values are chosen so
    that fp32 addition order changes the result."""
    order = [0, 2, 3, 1]
    pos_rank = [0, 2, 3, 1]
    x = np.zeros((4, 16), dtype=np.float32)
    vals = {0: 1.0e8, 2: 1.0, 3: -1.0e8, 1: 3.0}
    for r, v in vals.items():
        x[r, :] = v
    rc, out, _, _ = oracle.allreduce([x], order, 0x1, "SIMPLE", 65536, 4, "float32")
    assert rc == oracle.OK
    for c in range(4):
        fold = [pos_rank[(c + k) % 4] for k in range(1, 5)]
        acc = np.float32(vals[fold[0]])
        for r in fold[1:]:
            acc = np.float32(acc + np.float32(vals[r]))
        for rank in range(4):
            np.testing.assert_array_equal(out[0][rank, 4 * c:4 * c + 4], np.full(4, acc))
    # the four chunks fold in four different orders, and they do not all agree
    assert len({float(out[0][0, 4 * c]) for c in range(4)}) > 1


def _rne_bf16_exact(q: Fraction) -> int:
    """Exact rational round-to-nearest-even to bfloat16 bits (finite range)."""
    if q == 0:
        return 0
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    e = 0
    while a >= 2 ** (e + 1):
        e += 1
    while a < 2 ** e:
        e -= 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 7)
    k = a / ulp
    fl = k.numerator // k.denominator
    rem = k - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * ulp
    if v >= 2 ** 128:
        return sign | 0x7F80
    f = np.float32(float(v))
    return sign | int(f.view(np.uint32) >> 16)


def test_bf16_rounding_against_exact_rationals():
    """The oracle's bf16 rounding equals exact rational RNE, including ties,
    subnormals and the overflow threshold; and equals torch's float32 cast
    for float32-representable inputs (a library routine of the same rule)."""
    import torch
    specials = [1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -(1.0 + 2 ** -8),
                2 ** -126, 2 ** -133, 1.5 * 2 ** -133, 2.5 * 2 ** -133, 2 ** -134, 2 ** -135,
                (2 - 2 ** -7) * 2 ** 127, (2 - 2 ** -8) * 2 ** 127, 3.0e38, -0.0, 0.0]
    rng = np.random.default_rng(5)
    rand = list(rng.standard_normal(2000) * np.exp2(rng.integers(-140, 120, 2000)))
    for v in specials + rand:
        want = _rne_bf16_exact(Fraction(v)) if v != 0 else (0x8000 if np.signbit(v) else 0)
        assert oracle.bf16_round(v) == want, v
        assert int(cf._round_bf16(np.array([v]))[0]) == want, v
    f32 = (rng.standard_normal(20000) * np.exp2(rng.integers(-130, 120, 20000))).astype(np.float32)
    f32 = f32[np.isfinite(f32)]
    tb = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([oracle.bf16_round(float(v)) for v in f32[:3000]], dtype=np.uint16)
    np.testing.assert_array_equal(ours, tb[:3000])
    np.testing.assert_array_equal(cf._round_bf16(f32.astype(np.float64)), tb)


def test_bf16_per_hop_rounding_exact():
    """Per-hop rounding: each addition is rounded to bf16 before the next rank
    adds.  Checked against exact rational arithmetic on a 3-rank ring."""
    def bits_to_frac(b):
        return Fraction(float(np.uint32(int(b) << 16).view(np.float32)))
    rng = np.random.default_rng(9)
    order = [0, 1, 2]
    x32 = (rng.standard_normal((3, 48)) * 10).astype(np.float32)
    x = workloads._bf16_bits(x32).reshape(3, 48)
    rc, out, _, _ = oracle.allreduce([x], order, 0x1, "SIMPLE", 8 * 1024, 4, "bfloat16")
    assert rc == oracle.OK
    # 48 bf16 over 3 ranks: chunk = alignUp(16, 8) = 16 elements, owner c = e // 16
    for e in range(48):
        c = e // 16
        fold = [order[(c + k) % 3] for k in range(1, 4)]
        acc = int(x[fold[0], e])
        for r in fold[1:]:
            acc = _rne_bf16_exact(bits_to_frac(acc) + bits_to_frac(x[r, e]))
        for rank in range(3):
            assert int(out[0][rank, e]) == acc, e


# ------------------------------------------------- simulator vs closed form
CASES = [
    # N, order, mask, proto, buff, chunk_steps, dtype, count
    (4, [0, 2, 3, 1], 0xF, "LL", 8 * 2048, 4, "float32", 131072 // 16),
    (4, [0, 2, 3, 1], 0xFFF, "SIMPLE", 8 * 4096, 4, "float32", 100003),
    (4, [0, 2, 3, 1], 0xFFF, "LL128", 8 * 4096, 4, "float32", 100003),
    (8, [0, 3, 1, 6, 2, 7, 5, 4], 0xFFFF, "SIMPLE", 8 * 8192, 4, "bfloat16", 262147),
    (8, [0, 3, 1, 6, 2, 7, 5, 4], 0xFFFF, "SIMPLE", 8 * 8192, 2, "bfloat16", 99999),
    (3, [2, 0, 1], 0x5, "SIMPLE", 8 * 512, 2, "float32", 5001),
    (5, [4, 1, 0, 3, 2], 0x30, "LL", 8 * 1024, 4, "bfloat16", 7777),
    (2, [1, 0], 0x1, "LL128", 8 * 2048, 4, "float32", 3333),
]


def _draw(dtype, shape, seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(shape).astype(np.float32)
    return workloads._bf16_bits(v.ravel()).reshape(shape) if dtype == "bfloat16" else v


@pytest.mark.parametrize("case", CASES, ids=[f"{c[3]}-N{c[0]}-{c[6]}-{c[7]}" for c in CASES])
def test_simulator_matches_closed_form(case):
    N, order, mask, proto, buff, cs, dtype, count = case
    x = _draw(dtype, (N, count), count)
    rc, out, _, _ = oracle.allreduce([x], order, mask, proto, buff, cs, dtype)
    assert rc == oracle.OK
    want = cf.allreduce([x], order, mask, proto, buff, cs, dtype)[0]
    for r in range(N):
        np.testing.assert_array_equal(out[0][r].view(np.uint8), want.view(np.uint8))


def test_group_matches_closed_form():
    """Fused group: several collectives of uneven sizes in one launch."""
    counts = [7168] * 5 + [1, 999, 0, 4100]
    xs = [_draw("bfloat16", (4, c), 100 + i) for i, c in enumerate(counts)]
    rc, out, _, _ = oracle.allreduce(xs, [0, 1, 2, 3], 0b101101010011, "LL", 8 * 512, 4,
                                     "bfloat16")
    assert rc == oracle.OK
    want = cf.allreduce(xs, [0, 1, 2, 3], 0b101101010011, "LL", 8 * 512, 4, "bfloat16")
    for w in range(len(counts)):
        for r in range(4):
            np.testing.assert_array_equal(out[w][r], want[w])


def test_random_interleavings_and_in_place():
    """Results do not depend on how the ranks interleave, and in place equals
    out of place (Course 12, "正确性与稳定性": both were checked)."""
    x = _draw("float32", (4, 20011), 1)
    base = oracle.allreduce([x], [0, 2, 3, 1], 0x7, "SIMPLE", 8 * 1024, 4, "float32")[1][0]
    for proto in ("SIMPLE", "LL", "LL128"):
        buff = SMALL_BUFF[proto]
        ref = oracle.allreduce([x], [0, 2, 3, 1], 0x7, proto, buff, 4, "float32")[1][0]
        for seed in range(3):
            rc, out, _, _ = oracle.allreduce([x], [0, 2, 3, 1], 0x7, proto, buff, 4, "float32",
                                             sched=1, seed=seed)
            assert rc == oracle.OK
            np.testing.assert_array_equal(out[0], ref)
        rc, out, _, _ = oracle.allreduce([x], [0, 2, 3, 1], 0x7, proto, buff, 4, "float32",
                                         in_place=True)
        assert rc == oracle.OK
        np.testing.assert_array_equal(out[0], ref)
        for r in range(1, 4):
            np.testing.assert_array_equal(ref[r], ref[0])
    # chunking differs between protocols, so the fp32 bits may differ; values stay close
    assert np.abs(base[0] - ref[0]).max() < 1e-5


@pytest.mark.parametrize("dtype,u", [("float32", 2.0 ** -24), ("bfloat16", 2.0 ** -8)])
def test_recursive_summation_error_bound(dtype, u):
    """|fold - exact| <= gamma_{N-1} * sum |x_i| with gamma_k = k u / (1 - k u)
    (recursive summation bound, Higham, Accuracy and Stability of Numerical
    Algorithms, ch. 4), exact sum taken in binary64."""
    N = 8
    x = _draw(dtype, (N, 50000), 2)
    rc, out, _, _ = oracle.allreduce([x], [0, 3, 1, 6, 2, 7, 5, 4], 0xF, "SIMPLE", 8 * 4096, 4,
                                     dtype)
    assert rc == oracle.OK
    xf = cf._to_f64(x, dtype)
    exact = xf.sum(axis=0)
    bound = (N - 1) * u / (1 - (N - 1) * u) * np.abs(xf).sum(axis=0)
    got = cf._to_f64(out[0][0], dtype)
    assert (np.abs(got - exact) <= bound).all()


def test_bytes_sent_per_rank():
    """Course 12, "为什么是 2(N-1) 次发送": each rank sends 2(N-1) M/N bytes."""
    N, count = 4, 4 * 4096
    x = np.ones((N, count), dtype=np.float32)
    rc, _, st, _ = oracle.allreduce([x], [0, 1, 2, 3], 0x1, "SIMPLE", 65536, 4, "float32")
    assert rc == oracle.OK
    M = count * 4
    for r in range(N):
        assert st.payload_sent[r] == 2 * (N - 1) * M // N
        assert st.send_ops[r] == 2 * (N - 1) * (count // (N * 8192) or 1)


# ---------------------------------------------------------------- metric code
def test_busbw_reproduces_pages():
    """busbw = (M/t) * 2(N-1)/N reproduces every printed (time, busbw) pair to
    0.01 GB/s: the pages print two decimals and their busbw column is a
    median of per-run values, not always the ratio of the median time."""
    for N, M, t_us, bw, _ in gold("busbw.json")["rows"]:
        assert abs(metrics.busbw_gbps(M, t_us * 1e-6, N) - bw) <= 0.01


def test_algorithmic_bytes():
    """Simple (6N-4)M, LL (10N-8)M, LL128 with f = 16/15."""
    M = 1 << 26
    assert metrics.algorithmic_bytes(M, 4, "SIMPLE") == 20 * M
    assert metrics.algorithmic_bytes(M, 8, "SIMPLE") == 44 * M
    assert metrics.algorithmic_bytes(M, 4, "LL") == 32 * M
    assert abs(metrics.algorithmic_bytes(M, 4, "LL128") - 20.8 * M) < 1
    for N in (2, 3, 4, 8):
        assert metrics.algorithmic_bytes(M, N, "SIMPLE", direct=True) == (5 * N - 4) * M
        assert metrics.algorithmic_bytes(M, N, "SIMPLE", direct_read=True) == (6 * N - 6) * M
        assert metrics.algorithmic_bytes(M, N, "SIMPLE", direct=True,
                                         direct_read=True) == (5 * N - 6) * M



@pytest.mark.parametrize("proto,chunk_elems", [("SIMPLE", 1024), ("LL", 64), ("LL128", 480)])
@pytest.mark.parametrize("N", [2, 3, 4, 8])
def test_algorithmic_bytes_match_simulated_traffic(proto, chunk_elems, N):
    """The roofline's algorithmic bytes equal the traffic the simulator
    counts: every FIFO byte is written once and read once (2 x the wire bytes
    all ranks send) and every rank reads its input and writes its output once
    (2 N M).  Counts are whole loops of full chunks, so LL and LL128 lines are
    full and the wire/payload ratios exact (2 and 16/15)."""
    count = 2 * N * chunk_elems
    M = count * 4
    x = np.ones((N, count), dtype=np.float32)
    rc, _, st, _ = oracle.allreduce([x], list(range(N)), 0x1, proto, SMALL_BUFF[proto], 4,
                                    "float32")
    assert rc == oracle.OK
    wire = sum(st.wire_sent[r] for r in range(N))
    counted = 2 * wire + 2 * N * M
    assert abs(metrics.algorithmic_bytes(M, N, proto) - counted) <= 1e-9 * counted

# ------------------------------------------------------------- direct variant
@pytest.mark.parametrize("N", [2, 3, 4, 8])
def test_direct_variant_same_result_and_completes(N):
    """Direct read/write (Course 23, "发布顺序与 Fence": the direct primitives
    place data in the peer's user buffer and skip the send-credit wait, but
    steps and ordering remain): the all-gather half writes into the next rank's
    receive buffer.  The values are the same as through the FIFO, in place
    and out of place, under random interleavings, and nothing deadlocks."""
    rng = np.random.default_rng(N)
    order = [int(v) for v in rng.permutation(N)]
    x = _draw("float32", (N, 30011), N)
    base = oracle.allreduce([x], order, 0x5, "SIMPLE", SMALL_BUFF["SIMPLE"], 4, "float32")[1][0]
    for in_place in (False, True):
        for sched, seed in ((0, 0), (1, 1), (1, 2)):
            rc, out, _, _ = oracle.allreduce([x], order, 0x5, "SIMPLE", SMALL_BUFF["SIMPLE"], 4,
                                             "float32", in_place=in_place, sched=sched, seed=seed,
                                             direct=True)
            assert rc == oracle.OK
            np.testing.assert_array_equal(out[0], base)
    xi = rng.integers(-2 ** 31, 2 ** 31, size=(N, 5000)).astype(np.int32)
    rc, out, _, _ = oracle.allreduce([xi], order, 0x3, "SIMPLE", SMALL_BUFF["SIMPLE"], 2, "int32",
                                     direct=True)
    assert rc == oracle.OK
    for r in range(N):
        np.testing.assert_array_equal(out[0][r], _wrap_sum(xi))


def test_direct_variant_needs_simple():
    x = np.ones((4, 64), dtype=np.float32)
    for proto in ("LL", "LL128"):
        assert oracle.allreduce([x], [0, 1, 2, 3], 1, proto, SMALL_BUFF[proto], 4, "float32",
                                direct=True)[0] == oracle.INVALID


def test_direct_variant_bytes():
    """With direct all-gather each rank writes 2(N-1) chunks but reads its
    FIFO only in the reduce-scatter half: FIFO payload per rank is N M/N."""
    N, count = 4, 4 * 8192
    x = np.ones((N, count), dtype=np.float32)
    rc, _, st, _ = oracle.allreduce([x], [0, 1, 2, 3], 0x1, "SIMPLE", 65536, 4, "float32",
                                    direct=True)
    assert rc == oracle.OK
    M = count * 4
    for r in range(N):
        assert st.payload_sent[r] == 2 * (N - 1) * M // N


# ------------------------------------------------- per-channel rings (f2)
def test_per_channel_rings_graph_layout():
    """Course 12 "GRAPH 重建：N=4" and "为什么 channels 会重复": 12 channels
    over six base rings, channels 6-11 repeating 0-5.  In the simulator every
    channel's rank 0 follows its own ring's schedule (first send = chunk
    index-1 of that ring), and channel c and c+6 behave identically."""
    g = gold("graph_rings.json")["n4"]
    rings = g["base"]
    x = np.ones((4, 12 * 4 * 64), dtype=np.int32)
    rc, out, _, calls = oracle.allreduce([x], rings, (1 << g["channels"]) - 1, "SIMPLE",
                                         SMALL_BUFF["SIMPLE"], 4, "int32", log_calls=True)
    assert rc == oracle.OK and (out[0] == 4).all()
    for c in range(g["channels"]):
        ring = rings[c % len(rings)]
        idx, _, _ = oracle.ring_setup(ring)
        for rank in range(4):
            mine = [k for k in calls if k["channel_id"] == c and k["rank"] == rank]
            assert [(k["op"], k["chunk"]) for k in mine[:7]] == oracle.ring_schedule(4, idx[rank])


@pytest.mark.parametrize("key", ["n4", "n3", "n2"])
def test_per_channel_rings_match_closed_form(key):
    g = gold("graph_rings.json")[key]
    N = len(g["base"][0])
    x = _draw("float32", (N, 40009), N)
    rc, out, _, _ = oracle.allreduce([x], g["base"], (1 << g["channels"]) - 1, "SIMPLE",
                                     SMALL_BUFF["SIMPLE"], 4, "float32")
    assert rc == oracle.OK
    want = cf.allreduce([x], g["base"], (1 << g["channels"]) - 1, "SIMPLE",
                        SMALL_BUFF["SIMPLE"], 4, "float32")[0]
    for r in range(N):
        np.testing.assert_array_equal(out[0][r], want)
    # rings change the fold order of each channel, so the bits differ from one ring
    one = cf.allreduce([x], g["base"][0], (1 << g["channels"]) - 1, "SIMPLE",
                       SMALL_BUFF["SIMPLE"], 4, "float32")[0]
    if len(g["base"]) > 1:
        assert not np.array_equal(one, want)
    for proto in ("LL", "LL128"):
        rc, out, _, _ = oracle.allreduce([x], g["base"], (1 << g["channels"]) - 1, proto,
                                         SMALL_BUFF[proto], 4, "float32", sched=1, seed=7)
        assert rc == oracle.OK
        np.testing.assert_array_equal(
            out[0][0], cf.allreduce([x], g["base"], (1 << g["channels"]) - 1, proto,
                                    SMALL_BUFF[proto], 4, "float32")[0])


# ------------------------------------------------- direct read (f1)
@pytest.mark.parametrize("N", [2, 3, 4, 8])
def test_direct_read_same_result(N):
    """Direct read (course 23, "发布顺序与 Fence"): the first receive of every
    loop takes the previous rank's raw input from its send buffer instead of
    the FIFO.  The data is the same, so every value matches the FIFO path, in
    place and out of place, with and without the direct all-gather, under
    random interleavings.  Reading the wrong rank's buffer or offset would
    change the fold and fail here."""
    rng = np.random.default_rng(100 + N)
    order = [int(v) for v in rng.permutation(N)]
    x = _draw("float32", (N, 30011), N + 1)
    base = oracle.allreduce([x], order, 0x5, "SIMPLE", SMALL_BUFF["SIMPLE"], 4, "float32")[1][0]
    for in_place in (False, True):
        for direct in (False, True):
            for sched, seed in ((0, 0), (1, 3)):
                rc, out, _, _ = oracle.allreduce([x], order, 0x5, "SIMPLE", SMALL_BUFF["SIMPLE"],
                                                 4, "float32", in_place=in_place, sched=sched,
                                                 seed=seed, direct=direct, direct_read=True)
                assert rc == oracle.OK
                np.testing.assert_array_equal(out[0], base)


def test_direct_read_needs_simple():
    x = np.ones((4, 64), dtype=np.float32)
    for proto in ("LL", "LL128"):
        assert oracle.allreduce([x], [0, 1, 2, 3], 1, proto, SMALL_BUFF[proto], 4, "float32",
                                direct_read=True)[0] == oracle.INVALID


def test_fifo_bytes_of_the_direct_variants():
    """FIFO bytes written per rank, per collective of M bytes: 2(N-1) M/N
    through the FIFO; (N-1) M/N with the direct all-gather (only the
    reduce-scatter half uses the FIFO); (N-2) M/N with direct read as well
    (the loop's opening send moves nothing)."""
    N, count = 4, 4 * 8192
    x = np.ones((N, count), dtype=np.float32)
    M = count * 4
    for kw, chunks in ((dict(), 2 * (N - 1)), (dict(direct=True), N - 1),
                       (dict(direct_read=True), 2 * (N - 1) - 1),
                       (dict(direct=True, direct_read=True), N - 2)):
        rc, _, st, _ = oracle.allreduce([x], [0, 1, 2, 3], 0x1, "SIMPLE", 65536, 4, "float32", **kw)
        assert rc == oracle.OK
        for r in range(N):
            assert st.wire_sent[r] == chunks * M // N, (kw, r)


def test_simulator_matches_closed_form_random():
    """The simulator and the closed form, derived independently, agree bit
    for bit on random launches: ring sizes 2-8 with random ring orders and
    per-channel rings, random masks, every protocol, dtype and operator,
    groups of ragged counts (zeros included), in place or not, and a random
    interleaving of the ranks."""
    from hypothesis import given, settings, strategies as st

    quantum = {"SIMPLE": 512, "LL": 256, "LL128": 2048}

    @settings(max_examples=60, deadline=None, derandomize=True)
    @given(N=st.integers(2, 8), seed=st.integers(0, 2 ** 32 - 1),
           mask=st.integers(1, 2 ** 12 - 1), proto=st.sampled_from(["SIMPLE", "LL", "LL128"]),
           units=st.integers(1, 8), cs=st.sampled_from([2, 4]),
           dtype=st.sampled_from(["int32", "float32", "bfloat16"]),
           op=st.sampled_from(["sum", "prod", "max", "min", "avg"]),
           counts=st.lists(st.integers(0, 5000), min_size=1, max_size=4),
           nrings=st.integers(1, 3), in_place=st.booleans(), sched=st.integers(0, 1))
    def check(N, seed, mask, proto, units, cs, dtype, op, counts, nrings, in_place, sched):
        rng = np.random.default_rng(seed)
        rings = [[int(v) for v in rng.permutation(N)] for _ in range(nrings)]
        buff = 8 * quantum[proto] * units
        if dtype == "int32":
            xs = [rng.integers(-2 ** 31, 2 ** 31, size=(N, c)).astype(np.int32) for c in counts]
        else:
            xs = [_draw(dtype, (N, c), int(rng.integers(1 << 30))) for c in counts]
        order = rings if nrings > 1 else rings[0]
        rc, out, _, _ = oracle.allreduce(xs, order, mask, proto, buff, cs, dtype, op=op,
                                         in_place=in_place, sched=sched, seed=seed)
        assert rc == oracle.OK
        want = cf.allreduce(xs, order, mask, proto, buff, cs, dtype, op=op)
        for w in range(len(xs)):
            for r in range(N):
                np.testing.assert_array_equal(out[w][r].view(np.uint8), want[w].view(np.uint8))

    check()
