"""The structures of include/rar.h and their ctypes mirrors in the binding
have the same size and field offsets (checked with a C compiler; no GPU)."""
import ctypes
import os
import shutil
import subprocess
import tempfile

import pytest

from ring_all_reduce_channelmask_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

STRUCTS = {
    "rar_tuning_t": _lib.Tuning,
    "rar_oneshot_tuning_t": _lib.OneshotTuning,
    "rar_trace_rec_t": _lib.TraceRec,
    "rar_piece_t": _lib.Piece,
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_struct_layouts_match_the_header():
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "rar.h"', "int main(void) {"]
    for cname, py in STRUCTS.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    with tempfile.TemporaryDirectory() as tmp:
        src, exe = os.path.join(tmp, "l.c"), os.path.join(tmp, "l")
        open(src, "w").write("\n".join(lines) + "\n")
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    got = {}
    for line in out.splitlines():
        c, f, v = line.split()
        got[(c, f)] = int(v)
    for cname, py in STRUCTS.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)
