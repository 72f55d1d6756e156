"""ctypes declarations for librar.so (the C ABI in include/rar.h).

Argument marshalling only.  torch is imported first so that the process has
one HIP runtime (torch's), which librar.so then shares.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "librar.so")

SUCCESS, INVALID_ARGUMENT, UNSUPPORTED, HIP_ERROR, INTERNAL_ERROR, ABORTED = range(6)
DEBUG_DROP_RECV_HEAD, DEBUG_TRACE, DEBUG_LL_FLAG_WRAP8 = 1, 2, 4
PROTO = {"LL": 0, "LL128": 1, "SIMPLE": 2}
DTYPE = {"int32": 0, "float32": 1, "bfloat16": 2}
SUM = 0
RED = {"sum": 0, "prod": 1, "max": 2, "min": 3, "avg": 4, "premulsum": 5}


class Tuning(ctypes.Structure):
    _fields_ = [("lanes_per_channel", ctypes.c_int), ("waves_per_lane", ctypes.c_int),
                ("spin_timeout_us", ctypes.c_int), ("debug_flags", ctypes.c_int),
                ("launch_mode", ctypes.c_int), ("placement", ctypes.c_int),
                ("slices_per_chunk", ctypes.c_int), ("direct", ctypes.c_int),
                ("deal_works", ctypes.c_int), ("strict_scope", ctypes.c_int),
                ("waves_by_size", ctypes.c_int)]


class OneshotTuning(ctypes.Structure):
    _fields_ = [("workgroups", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("unroll", ctypes.c_int32), ("pad", ctypes.c_int32)]


class TraceRec(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("channel_id", ctypes.c_int32),
                ("lane", ctypes.c_int32), ("op", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("nelem", ctypes.c_uint32), ("t_begin", ctypes.c_uint64),
                ("wait_ticks", ctypes.c_uint32), ("data_ticks", ctypes.c_uint32),
                ("recv_step", ctypes.c_uint64), ("waves", ctypes.c_int32), ("pad", ctypes.c_int32)]


class Piece(ctypes.Structure):
    _fields_ = [("channel", ctypes.c_int32), ("channel_id", ctypes.c_int32),
                ("work", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("grid_offset", ctypes.c_int64), ("channel_count", ctypes.c_int64),
                ("chunk_count", ctypes.c_int64)]


class RarError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


_lib = None

# (name, restype, argtypes) of every entry point in include/rar.h
_c = ctypes
_vpp = _c.POINTER(_c.c_void_p)
_ip = _c.POINTER(_c.c_int)
SIGNATURES = [
    ("rar_comm_create", _c.c_int, [_c.POINTER(_c.c_void_p), _c.c_int, _ip, _c.c_uint64, _c.c_int,
                                   _c.c_size_t, _c.c_int, _c.POINTER(Tuning)]),
    ("rar_comm_create_rings", _c.c_int, [_c.POINTER(_c.c_void_p), _c.c_int, _c.c_int, _ip,
                                         _c.c_uint64, _c.c_int, _c.c_size_t, _c.c_int,
                                         _c.POINTER(Tuning)]),
    ("rar_allreduce", _c.c_int, [_c.c_void_p, _vpp, _vpp, _c.c_size_t, _c.c_int, _c.c_int,
                                 _c.c_void_p]),
    ("rar_allreduce_premul", _c.c_int, [_c.c_void_p, _vpp, _vpp, _c.c_size_t, _c.c_int,
                                        _c.c_void_p, _c.c_void_p]),
    ("rar_group_start", _c.c_int, [_c.c_void_p]),
    ("rar_group_end", _c.c_int, [_c.c_void_p, _c.c_void_p]),
    ("rar_group_discard", _c.c_int, [_c.c_void_p]),
    ("rar_comm_destroy", _c.c_int, [_c.c_void_p]),
    ("ring_allreduce", _c.c_int, [_vpp, _vpp, _c.c_int, _c.c_size_t, _c.c_int, _c.c_int, _ip,
                                  _c.c_int, _c.c_int, _c.c_size_t, _c.c_int, _c.c_void_p]),
    ("ring_allreduce_cache_release", _c.c_int, []),
    ("ring_allreduce_noalloc", _c.c_int, [_vpp, _vpp, _c.c_int, _c.c_size_t, _c.c_int, _c.c_int,
                                          _ip, _c.c_int, _c.c_int, _c.c_size_t, _c.c_int,
                                          _c.c_void_p]),
    ("rar_oneshot_allreduce", _c.c_int, [_vpp, _vpp, _c.c_int, _c.c_size_t, _c.c_int, _c.c_int,
                                         _c.POINTER(OneshotTuning), _c.c_void_p]),
    ("rar_oneshot_allreduce_premul", _c.c_int, [_vpp, _vpp, _c.c_int, _c.c_size_t, _c.c_int,
                                                _c.c_void_p, _c.POINTER(OneshotTuning),
                                                _c.c_void_p]),
    ("rar_comm_get_async_error", _c.c_int, [_c.c_void_p]),
    ("rar_comm_query_state", _c.c_int, [_c.c_void_p, _c.POINTER(_c.c_int64), _c.c_size_t,
                                        _c.POINTER(_c.c_size_t)]),
    ("rar_comm_shape", _c.c_int, [_c.c_void_p, _ip, _ip, _ip, _ip]),
    ("rar_comm_graph_text", _c.c_int, [_c.c_void_p, _c.c_char_p, _c.c_size_t,
                                       _c.POINTER(_c.c_size_t)]),
    ("rar_comm_read_trace", _c.c_int, [_c.c_void_p, _c.POINTER(TraceRec), _c.c_size_t,
                                       _c.POINTER(_c.c_size_t)]),
    ("rar_ring_info", _c.c_int, [_c.c_int, _ip, _ip, _ip, _ip]),
    ("rar_graph_text", _c.c_int, [_c.c_int, _c.c_int, _ip, _c.c_uint64, _c.c_char_p, _c.c_size_t,
                                  _c.POINTER(_c.c_size_t)]),
    ("rar_plan_pieces", _c.c_int, [_c.c_int, _c.c_uint64, _c.c_int, _c.c_size_t, _c.c_int,
                                   _c.c_int, _c.c_int, _c.POINTER(_c.c_size_t),
                                   _c.POINTER(Piece), _c.c_int, _ip, _c.POINTER(_c.c_int64)]),
    ("rar_get_error_string", _c.c_char_p, [_c.c_int]),
    ("rar_get_last_error", _c.c_char_p, []),
]


def load():
    """Load librar.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- one HIP runtime per process: torch's
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python ring_all_reduce_channelmask_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(code):
    if code != SUCCESS:
        lib = load()
        detail = lib.rar_get_last_error().decode()
        name = lib.rar_get_error_string(code).decode()
        raise RarError(code, f"{name}: {detail}")
