"""Ring AllReduce on one MI355X hosting N virtual ranks (HIP, gfx950).

Thin Python binding of librar.so: every byte the collective moves is moved by
the HIP kernel; this module only marshals pointers, sizes and the stream.
torch supplies device memory (tensors) and streams.

    comm = Comm(4, [0, 2, 3, 1], mask=0xFFF, proto="SIMPLE")
    comm.allreduce(sends, recvs)          # lists of N CUDA tensors
    with comm.group():                    # fused works, one launch
        for s, r in pairs:
            comm.allreduce(s, r)
"""
import contextlib
import ctypes

from . import _lib
from ._lib import RarError  # noqa: F401

__all__ = ["Comm", "ring_allreduce", "ring_allreduce_noalloc", "oneshot_allreduce", "ring_info", "graph_text", "plan_pieces", "RarError"]


def _dtype_name(t):
    import torch
    m = {torch.float32: "float32", torch.bfloat16: "bfloat16", torch.int32: "int32"}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _ptr_array(tensors):
    arr = (ctypes.c_void_p * len(tensors))()
    for i, t in enumerate(tensors):
        arr[i] = t.data_ptr()
    return arr


def _check_tensors(sends, recvs, nranks):
    if len(sends) != nranks or len(recvs) != nranks:
        raise ValueError(f"need {nranks} send and {nranks} recv tensors")
    n = sends[0].numel()
    dt = sends[0].dtype
    for t in list(sends) + list(recvs):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")
        if t.numel() != n or t.dtype != dt:
            raise ValueError("all tensors need the same size and dtype")
    return n, _dtype_name(sends[0])


def _scalar_buffer(scalars, dtype, nranks):
    """PreMulSum scalars as a host array of payload-type elements: numbers
    are converted (bfloat16 rounded to nearest even); a numpy uint16 array
    for bfloat16 is taken as bit patterns."""
    import numpy as np
    if scalars is None or len(scalars) != nranks:
        raise ValueError(f"premulsum needs {nranks} scalars")
    if dtype == "bfloat16":
        a = np.asarray(scalars)
        if a.dtype != np.uint16:
            import torch
            a = torch.tensor(np.asarray(scalars, dtype=np.float32)).to(torch.bfloat16) \
                .view(torch.int16).numpy().view(np.uint16)
    else:
        a = np.asarray(scalars, dtype=np.float32 if dtype == "float32" else np.int32)
    return np.ascontiguousarray(a)


def _stream_handle(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class Comm:
    """A communicator: N virtual ranks on the current device, a ring (or one
    ring per channel: ``ring_order`` a list of rings, channel id c running
    ring c mod len(rings)), a channel mask and a protocol; owns the FIFOs
    between ring neighbours."""

    def __init__(self, nranks, ring_order, mask, proto="SIMPLE", buff_size=0, chunk_steps=0,
                 lanes=0, waves=0, timeout_us=0, debug_flags=0, launch_mode=0, placement=0,
                 slices_per_chunk=0, direct=0, deal_works=0, strict_scope=0, waves_by_size=0):
        lib = _lib.load()
        rings = [list(r) for r in ring_order] if len(ring_order) and \
            isinstance(ring_order[0], (list, tuple)) else [list(ring_order)]
        if any(len(r) != nranks for r in rings):
            raise ValueError("every ring must list every rank once")
        self.nranks = nranks
        self.rings = rings
        self.ring_order = rings[0]
        self.mask = mask
        self.proto = proto
        flat = [r for ring in rings for r in ring]
        order = (ctypes.c_int * len(flat))(*flat)
        tune = _lib.Tuning(lanes, waves, timeout_us, debug_flags, launch_mode, placement,
                           slices_per_chunk, direct, deal_works, strict_scope, waves_by_size)
        h = ctypes.c_void_p()
        _lib.check(lib.rar_comm_create_rings(ctypes.byref(h), nranks, len(rings), order, mask,
                                             _lib.PROTO[proto], buff_size, chunk_steps,
                                             ctypes.byref(tune)))
        self._h = h

    @property
    def handle(self):
        return self._h

    def allreduce(self, sends, recvs=None, stream=None, op="sum", scalars=None):
        """Reduce over ranks with ``op`` (sum, prod, max, min, avg, or
        premulsum with one scalar per rank); ``recvs=None`` runs in place."""
        recvs = sends if recvs is None else recvs
        n, dt = _check_tensors(sends, recvs, self.nranks)
        lib = _lib.load()
        if op == "premulsum":
            buf = _scalar_buffer(scalars, dt, self.nranks)
            _lib.check(lib.rar_allreduce_premul(self._h, _ptr_array(sends), _ptr_array(recvs), n,
                                                _lib.DTYPE[dt], buf.ctypes.data,
                                                _stream_handle(stream)))
            return
        _lib.check(lib.rar_allreduce(self._h, _ptr_array(sends), _ptr_array(recvs), n,
                                     _lib.DTYPE[dt], _lib.RED[op], _stream_handle(stream)))

    @contextlib.contextmanager
    def group(self, stream=None):
        """Queue the body's AllReduces and launch them as one fused launch
        when the body ends normally.  If the body raises, the partly queued
        group is dropped (nothing is launched) and the exception propagates."""
        lib = _lib.load()
        _lib.check(lib.rar_group_start(self._h))
        try:
            yield self
        except BaseException:
            lib.rar_group_discard(self._h)
            raise
        _lib.check(lib.rar_group_end(self._h, _stream_handle(stream)))

    def async_error(self):
        return _lib.load().rar_comm_get_async_error(self._h)

    def shape(self):
        c, p, w, g = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        _lib.check(_lib.load().rar_comm_shape(self._h, ctypes.byref(c), ctypes.byref(p),
                                              ctypes.byref(w), ctypes.byref(g)))
        return dict(channels=c.value, lanes=p.value, waves=w.value, grid=g.value)

    def graph(self):
        """The rings as GRAPH lines, each followed by its channel's geometry."""
        return _text(lambda buf, cap, n: _lib.load().rar_comm_graph_text(self._h, buf, cap, n))

    def query_state(self):
        s = self.shape()
        cap = self.nranks * s["channels"] * s["lanes"] * 2
        out = (ctypes.c_int64 * cap)()
        written = ctypes.c_size_t()
        _lib.check(_lib.load().rar_comm_query_state(self._h, out, cap, ctypes.byref(written)))
        return list(out[:written.value])

    def read_trace(self):
        """Timeline of the last launch (needs debug_flags bit 1): a list of
        dicts, one per Simple slice or LL/LL128 step of every workgroup."""
        s = self.shape()
        cap = s["grid"] * 4096
        out = (_lib.TraceRec * cap)()
        written = ctypes.c_size_t()
        _lib.check(_lib.load().rar_comm_read_trace(self._h, out, cap, ctypes.byref(written)))
        names = [f for f, _ in _lib.TraceRec._fields_]
        return [{f: getattr(r, f) for f in names} for r in out[:written.value]]

    def close(self):
        if getattr(self, "_h", None):
            _lib.load().rar_comm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def ring_allreduce(sends, recvs, ring_order, proto="SIMPLE", nchannels=1, buff_size=0,
                   chunk_steps=0, stream=None, op="sum"):
    """The pages' problem statement as one call (communicator cached inside)."""
    nranks = len(sends)
    n, dt = _check_tensors(sends, recvs, nranks)
    lib = _lib.load()
    order = (ctypes.c_int * nranks)(*ring_order)
    _lib.check(lib.ring_allreduce(_ptr_array(sends), _ptr_array(recvs), nranks, n,
                                  _lib.DTYPE[dt], _lib.RED[op], order, _lib.PROTO[proto], nchannels,
                                  buff_size, chunk_steps, _stream_handle(stream)))


def ring_allreduce_cache_release():
    """Destroy the communicators ring_allreduce has cached (after their last
    launches): frees their device memory, and clears one that a watchdog
    abort left refusing calls."""
    _lib.check(_lib.load().ring_allreduce_cache_release())


def ring_allreduce_noalloc(sends, recvs, ring_order, proto="SIMPLE", nchannels=1, buff_size=0,
                           chunk_steps=0, stream=None, op="sum"):
    """ring_allreduce with its device state in the library's static array:
    no device allocation (see include/rar.h for the size limit)."""
    nranks = len(sends)
    n, dt = _check_tensors(sends, recvs, nranks)
    order = (ctypes.c_int * nranks)(*ring_order)
    _lib.check(_lib.load().ring_allreduce_noalloc(
        _ptr_array(sends), _ptr_array(recvs), nranks, n, _lib.DTYPE[dt], _lib.RED[op], order,
        _lib.PROTO[proto], nchannels, buff_size, chunk_steps, _stream_handle(stream)))


def oneshot_allreduce(sends, recvs=None, workgroups=0, waves=0, unroll=0, stream=None, op="sum",
                      scalars=None):
    """One-shot AllReduce of N equally sized device tensors (one per virtual
    rank): every output gets the fold of all inputs in rank order.
    ``recvs=None`` runs in place."""
    recvs = sends if recvs is None else recvs
    nranks = len(sends)
    n, dt = _check_tensors(sends, recvs, nranks)
    tune = _lib.OneshotTuning(workgroups, waves, unroll, 0)
    if op == "premulsum":
        buf = _scalar_buffer(scalars, dt, nranks)
        _lib.check(_lib.load().rar_oneshot_allreduce_premul(
            _ptr_array(sends), _ptr_array(recvs), nranks, n, _lib.DTYPE[dt], buf.ctypes.data,
            ctypes.byref(tune), _stream_handle(stream)))
        return
    _lib.check(_lib.load().rar_oneshot_allreduce(_ptr_array(sends), _ptr_array(recvs), nranks, n,
                                                 _lib.DTYPE[dt], _lib.RED[op], ctypes.byref(tune),
                                                 _stream_handle(stream)))


def ring_info(ring_order):
    """(index, prev, next) per user rank, as the library computes them."""
    n = len(ring_order)
    idx, prv, nxt = (ctypes.c_int * n)(), (ctypes.c_int * n)(), (ctypes.c_int * n)()
    _lib.check(_lib.load().rar_ring_info(n, (ctypes.c_int * n)(*ring_order), idx, prv, nxt))
    return list(idx), list(prv), list(nxt)


def _text(call):
    """A text result: ask for its length, then fetch it."""
    n = ctypes.c_size_t()
    _lib.check(call(None, 0, ctypes.byref(n)))
    buf = ctypes.create_string_buffer(n.value + 1)
    _lib.check(call(buf, n.value + 1, ctypes.byref(n)))
    return buf.value.decode()


def graph_text(nranks, rings, mask):
    """GRAPH lines of a ring layout: one "Channel cc/CC : r0 r1 ..." line per
    set bit of mask; `rings` is one ring order or a list of them."""
    rings = [list(r) for r in rings] if len(rings) and isinstance(rings[0], (list, tuple)) \
        else [list(rings)]
    flat = [r for ring in rings for r in ring]
    arr = (ctypes.c_int * len(flat))(*flat)
    return _text(lambda buf, cap, n: _lib.load().rar_graph_text(nranks, len(rings), arr, mask, buf,
                                                                cap, n))


def plan_pieces(nranks, mask, proto, buff_size, chunk_steps, dtype, counts):
    """The library's channel split: (pieces as dicts, chunk maximum)."""
    counts = list(counts)
    cap = 64 * (len(counts) + 1)
    arr = (_lib.Piece * cap)()
    npieces, cmax = ctypes.c_int(), ctypes.c_int64()
    carr = (ctypes.c_size_t * len(counts))(*counts)
    _lib.check(_lib.load().rar_plan_pieces(nranks, mask, _lib.PROTO[proto], buff_size,
                                           chunk_steps, _lib.DTYPE[dtype], len(counts), carr,
                                           arr, cap, ctypes.byref(npieces), ctypes.byref(cmax)))
    assert npieces.value <= cap
    return ([dict(channel=p.channel, channel_id=p.channel_id, work=p.work,
                  grid_offset=p.grid_offset, channel_count=p.channel_count,
                  chunk_count=p.chunk_count) for p in arr[:npieces.value]], cmax.value)
