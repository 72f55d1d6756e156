"""Helpers for GPU tests: move seeded numpy inputs to device tensors, run the
HIP path through the C ABI, bring results back as raw numpy arrays."""
import numpy as np


def to_device(x, dtype):
    import torch
    if dtype == "bfloat16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def to_host(t, dtype):
    import torch
    if dtype == "bfloat16":
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy()


def run_hip(comm, inputs, dtype, in_place=False, op="sum", scalars=None):
    """inputs: list over collectives of [N, count] arrays; ``scalars``: for
    premulsum, one array of N payload elements per collective.  Returns a
    list of [N, count] arrays (what every rank's receive buffer holds)."""
    import torch
    N = comm.nranks
    sends, recvs = [], []
    for x in inputs:
        s = [to_device(x[r], dtype) for r in range(N)]
        r_ = s if in_place else [torch.full_like(t, 0x7F if dtype != "float32" else float("nan"))
                                 for t in s]
        sends.append(s)
        recvs.append(r_)
    sc = scalars if scalars is not None else [None] * len(inputs)
    if len(inputs) == 1:
        comm.allreduce(sends[0], recvs[0], op=op, scalars=sc[0])
    else:
        with comm.group():
            for s, r_, k in zip(sends, recvs, sc):
                comm.allreduce(s, r_, op=op, scalars=k)
    torch.cuda.synchronize()
    assert comm.async_error() == 0, "watchdog fired"
    return [np.stack([to_host(t, dtype) for t in r_]) for r_ in recvs]


def assert_bits_equal(got, want, what=""):
    g = np.ascontiguousarray(got).view(np.uint8)
    w = np.ascontiguousarray(want).view(np.uint8)
    if g.shape != w.shape or not np.array_equal(g, w):
        gg = np.ascontiguousarray(got).reshape(-1)
        ww = np.ascontiguousarray(want).reshape(-1)
        bad = np.nonzero(gg.view(np.uint8 if gg.dtype.itemsize == 1 else
                                 {2: np.uint16, 4: np.uint32}[gg.dtype.itemsize]) !=
                         ww.view({1: np.uint8, 2: np.uint16, 4: np.uint32}[ww.dtype.itemsize]))[0]
        raise AssertionError(f"{what}: {bad.size} of {gg.size} elements differ; first at "
                             f"{bad[:8].tolist()}: got {gg[bad[:4]]} want {ww[bad[:4]]}")
