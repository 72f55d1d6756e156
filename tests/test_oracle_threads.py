"""The oracle's channel-parallel mode (the CPU baseline's timing mode): its
outputs and statistics equal the sequential round-robin mode's, and the
threads it runs do not race (a ThreadSanitizer build of a small driver)."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _inputs(rng, dtype, N, count):
    if dtype == "int32":
        return rng.integers(-2 ** 31, 2 ** 31, size=(N, count)).astype(np.int32)
    x = rng.standard_normal((N, count)).astype(np.float32)
    if dtype == "bfloat16":
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    return x


@pytest.mark.parametrize("proto,buff", [("SIMPLE", 8 * 1024), ("LL", 8 * 512), ("LL128", 8 * 2048)])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
def test_threads_match_sequential(proto, buff, dtype):
    rng = np.random.default_rng(hash((proto, dtype)) % 2 ** 32)
    for N, mask, counts in ((4, 0xFFF, [20011]), (3, 0b101101010011, [3001, 17, 999]),
                            (8, 0xF0F0, [4097, 8])):
        order = [0] + [int(v) for v in rng.permutation(np.arange(1, N))]
        xs = [_inputs(rng, dtype, N, c) for c in counts]
        rc0, out0, st0, _ = oracle.allreduce(xs, order, mask, proto, buff, 4, dtype)
        for threads in (1, 3, 0):
            rc1, out1, st1, _ = oracle.allreduce(xs, order, mask, proto, buff, 4, dtype, threads=threads)
            assert rc0 == rc1 == oracle.OK
            for a, b in zip(out0, out1):
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
            assert st0.units_run == st1.units_run
            assert list(st0.wire_sent) == list(st1.wire_sent)
            assert list(st0.send_ops) == list(st1.send_ops)


def test_threads_report_a_deadlock():
    """A dropped receive head stalls every channel; the parallel mode reports it."""
    x = np.ones((4, 50000), dtype=np.float32)
    rc, _, st, _ = oracle.allreduce([x], [0, 1, 2, 3], 0xF, "SIMPLE", 8 * 1024, 4, "float32",
                                    drop_recv_head=True, threads=4)
    assert rc == oracle.DEADLOCK
    assert st.deadlock_rank >= 0 and st.deadlock_channel in (0, 1, 2, 3)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_threads_are_race_free_under_thread_sanitizer():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "tsan_check")
        cmd = ["g++", "-O1", "-g", "-std=c++17", "-fsanitize=thread", "-pthread", "-ffp-contract=off",
               "-I", os.path.join(ROOT, "oracle"), os.path.join(ROOT, "oracle", "ring_sim.cpp"),
               os.path.join(ROOT, "oracle", "tsan_check.cpp"), "-o", exe]
        b = subprocess.run(cmd, capture_output=True, text=True)
        if b.returncode != 0 and "tsan" in (b.stderr or "").lower():
            pytest.skip("ThreadSanitizer runtime not available: " + b.stderr[-200:])
        assert b.returncode == 0, b.stderr
        env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
        assert "OK" in r.stdout
