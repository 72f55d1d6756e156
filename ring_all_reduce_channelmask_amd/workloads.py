"""Seeded synthetic inputs and the workload shapes used by tests and the
benchmark.  This module holds no arithmetic of the method: it only draws
numbers.  Both the HIP path and the oracle receive the same arrays from here.

The workloads mirror the sizes the NCCL course pages measure (4 KiB,
512 KiB and 64 MiB messages over 4 ranks, 1/4/12 channels, all three
protocols), plus an 8-rank bf16/int32 case and a fused group of small
collectives over a sparse channel mask.  Raw representations: float32 and
int32 as themselves, bfloat16 as uint16 bit patterns.
"""
from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

MiB = 1 << 20
KiB = 1 << 10


@dataclass(frozen=True)
class Workload:
    key: str
    nranks: int
    ring_order: Tuple[int, ...]
    mask: int
    proto: str
    dtype: str
    counts: Tuple[int, ...]       # one entry per collective of the launch
    buff_size: int                # 0 = protocol default
    chunk_steps: int
    dist: str
    seed_base: Tuple[int, ...]
    note: str = ""

    @property
    def elem_size(self) -> int:
        return 2 if self.dtype == "bfloat16" else 4

    @property
    def message_bytes(self) -> int:
        return sum(self.counts) * self.elem_size


DEFAULT_BUFF = {"SIMPLE": 4 * MiB, "LL": 512 * KiB, "LL128": 4915200}

WORKLOADS = {
    "simple_4k": Workload("simple_4k", 4, (0, 1, 2, 3), 0x1, "SIMPLE", "float32", (1024,),
                          64 * KiB, 4, "int_pm8", (1,),
                          "4 ranks, 1 channel, Simple, fp32, 4 KiB/rank, integer-valued in [-8,8]"),
    "ll_512k": Workload("ll_512k", 4, (0, 2, 3, 1), 0xF, "LL", "float32", (131072,),
                        512 * KiB, 4, "uniform", (2,),
                        "4 ranks, 4 channels, LL, fp32, 512 KiB/rank, uniform [-1,1]"),
    "simple_64m": Workload("simple_64m", 4, (0, 2, 3, 1), 0xFFF, "SIMPLE", "float32",
                           (16 * MiB,), 4 * MiB, 4, "uniform", (3,),
                           "4 ranks, 12 channels, Simple 4 MiB buffer, fp32, 64 MiB/rank"),
    "ll128_64m": Workload("ll128_64m", 4, (0, 2, 3, 1), 0xFFF, "LL128", "float32",
                          (16 * MiB,), 4915200, 4, "uniform", (3,),
                          "4 ranks, 12 channels, LL128, fp32, 64 MiB/rank"),
    "bf16_n8": Workload("bf16_n8", 8, (0, 3, 1, 6, 2, 7, 5, 4), 0xFFFF, "SIMPLE", "bfloat16",
                        (32 * MiB,), 4 * MiB, 4, "normal", (4,),
                        "8 ranks, 16 channels, Simple, bf16 per-hop rounding, 64 MiB/rank"),
    "int32_n8": Workload("int32_n8", 8, (0, 3, 1, 6, 2, 7, 5, 4), 0xFFFF, "SIMPLE", "int32",
                         (32 * MiB,), 4 * MiB, 4, "int27", (4,),
                         "8 ranks, 16 channels, Simple, int32, 128 MiB/rank"),
    "ll_64m": Workload("ll_64m", 4, (0, 2, 3, 1), 0xFFF, "LL", "float32", (16 * MiB,),
                       512 * KiB, 4, "uniform", (3,),
                       "4 ranks, 12 channels, LL, fp32, 64 MiB/rank"),
    "fused_ll": Workload("fused_ll", 4, (0, 1, 2, 3), 0b101101010011, "LL", "bfloat16",
                         (7168,) * 104, 512 * KiB, 4, "normal_half", (5,),
                         "104 fused bf16 AllReduces of 7168 elements, sparse mask, LL"),
}


def _bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns using torch's cast (round to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def draw(dist: str, dtype: str, n: int, seed) -> np.ndarray:
    rng = np.random.default_rng(list(seed))
    if dist == "int_pm8":
        v = rng.integers(-8, 9, size=n).astype(np.float64)
    elif dist == "uniform":
        v = rng.uniform(-1.0, 1.0, size=n)
    elif dist == "normal":
        v = rng.standard_normal(size=n)
    elif dist == "normal_half":
        v = rng.normal(0.0, 0.5, size=n)
    elif dist == "int27":
        return rng.integers(-2 ** 27, 2 ** 27, size=n).astype(np.int32)
    elif dist == "int_full":
        return rng.integers(-2 ** 31, 2 ** 31, size=n).astype(np.int32)
    else:
        raise ValueError(dist)
    if dtype == "int32":
        return v.astype(np.int32)
    x32 = v.astype(np.float32)  # round to nearest even
    if dtype == "float32":
        return x32
    return _bf16_bits(x32)


def inputs_for(w: Workload, scale: float = 1.0) -> List[np.ndarray]:
    """Per collective, an [N, count] array of rank inputs.  ``scale`` < 1 shrinks
    every count (kept a positive integer) for fast tests; the shape of the
    launch (ranks, ring, channels, protocol, group size) is kept."""
    out = []
    for i, c in enumerate(w.counts):
        n = max(1, int(c * scale)) if scale != 1.0 else c
        rows = []
        for r in range(w.nranks):
            seed = w.seed_base + (r,) if len(w.counts) == 1 else w.seed_base + (r, i)
            rows.append(draw(w.dist, w.dtype, n, seed))
        out.append(np.stack(rows))
    return out
