"""LL flag generations [course 23, "LL：Data 与 Flag 同 Line": a test mode
wraps the flag at 0x100, and at cleanup steps the sender stamps the rest of
the slot with the current generation].  Pins of the oracle's line-level model
and of the simulator's wrap mode (no GPU)."""
import numpy as np
import pytest

import oracle
from oracle import closed_form as cf

CAP = 16  # lines per slot


def test_stale_generation_comes_round_without_cleanup():
    """Step 0 fills slot 0; the next 255 steps write one line each.  Step 256
    uses slot 0 again with flag (256+1) mod 256 = 1, the flag step 0 left in
    lines 1..15: an eager consumer takes a stale line."""
    sizes = [CAP] + [1] * 255
    assert oracle.ll_wrap(8, False, 8, CAP, sizes, 400) == ("corrupt", 256)


def test_zeroed_lines_match_flag_zero_without_cleanup():
    """Step 255 has flag 0, the value of lines never written since the FIFO
    was zeroed: slot 7 only ever held one-line steps before it."""
    sizes = [1] * 255 + [CAP]
    assert oracle.ll_wrap(8, False, 8, CAP, sizes, 300) == ("corrupt", 255)


@pytest.mark.parametrize("sizes", [[CAP] + [1] * 255, [1] * 255 + [CAP]])
def test_cleanup_prevents_both(sizes):
    assert oracle.ll_wrap(8, True, 8, CAP, sizes, 3000) == ("complete", -1)


def test_cleanup_with_random_sizes():
    rng = np.random.default_rng(0)
    for trial in range(20):
        sizes = list(rng.integers(1, CAP + 1, size=int(rng.integers(1, 600))))
        assert oracle.ll_wrap(8, True, 8, CAP, sizes, 2500) == ("complete", -1), trial


def test_some_random_sizes_corrupt_without_cleanup():
    """Without cleanup, random step sizes eventually hand a stale line over."""
    rng = np.random.default_rng(1)
    hits = 0
    for _ in range(20):
        sizes = list(rng.integers(1, CAP + 1, size=int(rng.integers(1, 600))))
        hits += oracle.ll_wrap(8, False, 8, CAP, sizes, 2500)[0] == "corrupt"
    assert hits > 0


def test_32_bit_flags_do_not_wrap_in_reach():
    assert oracle.ll_wrap(32, False, 8, CAP, [CAP] + [1] * 255, 3000) == ("complete", -1)


def test_model_rejects_bad_parameters():
    assert oracle.ll_wrap(16, True, 8, CAP, [1], 10)[0] == "invalid"
    assert oracle.ll_wrap(8, True, 128, CAP, [1], 10)[0] == "invalid"   # slots >= half period
    assert oracle.ll_wrap(8, True, 8, CAP, [CAP + 1], 10)[0] == "invalid"


@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_simulator_wrap_mode_matches_closed_form(dtype):
    """LL with 8-bit flags over more than 256 steps per connector: the result
    is that of the closed form (the flags carry no data)."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 20011)).astype(np.float32)
    if dtype == "bfloat16":
        x = (x.view(np.uint32) >> 16).astype(np.uint16)
    rc, out, st, _ = oracle.allreduce([x], [0, 2, 3, 1], 0x1, "LL", 8 * 512, 4, dtype,
                                      ll_wrap8=True, sched=1, seed=5)
    assert rc == oracle.OK
    assert st.units_run / 4 > 256  # units per rank: each advances its connectors
    want = cf.allreduce([x], [0, 2, 3, 1], 0x1, "LL", 8 * 512, 4, dtype)[0]
    for r in range(4):
        np.testing.assert_array_equal(out[0][r], want)
