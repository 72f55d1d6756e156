"""Closed form of the ring AllReduce result -- TEST INFRASTRUCTURE ONLY.

No FIFOs, steps or scheduling: for every element it states which ring
position owns the element's chunk and folds the N inputs in the order the
ring visits them, rounding to the payload type after every addition.

The chunk that owns an element follows the channel split and the runRing
chunking [C12 "runRing 的数据切分", "多 channel 如何并行"]; the fold order
follows the primitive sequence [C12 "源码步骤一：初始 send" .. "源码步骤三：
融合边界"]: the rank at ring position c+1 sends its own input, every following
rank adds its input and forwards, and the owner at position c adds last.  The
all-gather half copies that value unchanged to every rank [C12 "源码步骤四",
"源码步骤五"], so all ranks end with the same bits.

Written independently of ``ring_sim.cpp``: nothing is shared between them.
"""
import numpy as np

_PROTO_SLOTS = 8


def _div_up(a, b):
    return -(-a // b)


def _align_up(a, b):
    return _div_up(a, b) * b


def _elem_size(dtype):
    return 2 if dtype == "bfloat16" else 4


def chunk_max(proto, buff_size, chunk_steps, dtype):
    """Largest chunk in elements for a protocol and FIFO size [C23 "Buffer 到
    Chunk 的实测公式", "LL：Data 与 Flag 同 Line", "LL128：15/16 Payload"]."""
    es = _elem_size(dtype)
    step = buff_size // _PROTO_SLOTS
    if proto == "SIMPLE":
        return (step // es) * chunk_steps
    if proto == "LL":
        return (step // 2) // es  # 16-byte line = 8 payload bytes + two flags
    return ((step // 128) * 120) // es  # 128-byte line = 15 payload words + flag


def owner_positions(counts, nranks, nchannels, cmax, dtype, with_channel=False):
    """For each collective of the launch, an int array giving the ring position
    that owns each element (the chunk index of the element); with
    ``with_channel``, also the dense channel index of each element."""
    vec = 16 // _elem_size(dtype)
    starts, total = [], 0
    for c in counts:
        s = _align_up(total, vec)
        starts.append(s)
        total = s + c
    owners = [np.full(c, -1, dtype=np.int64) for c in counts]
    chans = [np.full(c, -1, dtype=np.int64) for c in counts]
    if total == 0:
        return (owners, chans) if with_channel else owners
    per_ch = _align_up(_div_up(total, nchannels), vec)
    for n in range(nchannels):
        lo, hi = n * per_ch, min((n + 1) * per_ch, total)
        for w, c in enumerate(counts):
            a, b = max(lo, starts[w]), min(hi, starts[w] + c)
            if a >= b:
                continue
            grid_off, ch_count = a - starts[w], b - a
            loop_count = nranks * cmax
            elem_off = 0
            while elem_off < ch_count:
                rem = ch_count - elem_off
                cc = cmax if rem >= loop_count else _align_up(_div_up(rem, nranks), vec)
                for chunk in range(nranks):
                    first = chunk * cc
                    nel = max(0, min(cc, rem - first))
                    if nel:
                        base = grid_off + elem_off + first
                        owners[w][base:base + nel] = chunk
                        chans[w][base:base + nel] = n
                elem_off += loop_count
    for o in owners:
        assert (o >= 0).all()
    return (owners, chans) if with_channel else owners


def _round_bf16(v64):
    """Round binary64 values to the nearest bfloat16 (ties to even), returned
    as uint16 bit patterns.  Spacing is 2^(e-8) for |v| in [2^(e-1), 2^e),
    never finer than 2^-133 (the subnormal spacing)."""
    v64 = np.asarray(v64, dtype=np.float64)
    a = np.abs(v64)
    _, e = np.frexp(a)
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(a / q) * q
    r = np.where(a == 0, 0.0, r)
    r = np.copysign(r, v64)
    with np.errstate(over="ignore"):
        f = r.astype(np.float32)  # exact unless it overflows to inf
    f = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.float32(np.inf), v64), f)
    bits = f.astype(np.float32).view(np.uint32)
    return (bits >> 16).astype(np.uint16)


def _to_f64(x, dtype):
    if dtype == "bfloat16":
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _hop(acc, x, dtype, op="sum"):
    """One reduction of the ring (the partial ``acc`` with a rank's input
    ``x``), rounded to the payload type.  max / min keep ``acc`` unless ``x``
    is strictly larger / smaller; avg adds (its division is the post-op)."""
    if op in ("max", "min"):
        a, b = _to_f64(acc, dtype), _to_f64(x, dtype)
        if dtype == "int32":
            a, b = acc.astype(np.int64), x.astype(np.int64)
        take = b > a if op == "max" else b < a
        return np.where(take, x, acc).astype(acc.dtype)
    if dtype == "int32":
        au, xu = acc.astype(np.int32).view(np.uint32), x.astype(np.int32).view(np.uint32)
        if op == "prod":
            # low 32 bits of the product
            return ((au.astype(np.uint64) * xu.astype(np.uint64)) & 0xFFFFFFFF) \
                .astype(np.uint32).view(np.int32)
        return (au + xu).view(np.int32)  # two's-complement wrap modulo 2^32
    a, b = _to_f64(acc, dtype), _to_f64(x, dtype)
    s = a * b if op == "prod" else a + b  # exact in binary64 for fp32 / bf16 operands
    if dtype == "float32":
        return s.astype(np.float32)
    return _round_bf16(s)


def _premul(s, x, dtype):
    """PreMulSum's scaling of a rank's input: s * x rounded once to the
    payload type (int32: low 32 bits)."""
    if dtype == "int32":
        su = np.asarray(s).astype(np.int32).view(np.uint32).astype(np.uint64)
        xu = x.astype(np.int32).view(np.uint32).astype(np.uint64)
        return ((su * xu) & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
    p = _to_f64(np.asarray(s), dtype) * _to_f64(x, dtype)  # exact in binary64
    if dtype == "float32":
        return p.astype(np.float32)
    return _round_bf16(p)


def _post_div(v, nranks, dtype):
    """avg's post-op: the owner's final sum divided by N, rounded once
    (int32: truncated toward zero)."""
    if dtype == "int32":
        q = np.abs(v.astype(np.int64)) // nranks
        return np.where(v < 0, -q, q).astype(np.int32)
    q = _to_f64(v, dtype) / nranks
    if dtype == "float32":
        return q.astype(np.float32)
    return _round_bf16(q)


def allreduce(inputs, ring_order, mask, proto, buff_size, chunk_steps, dtype, op="sum",
              scalars=None):
    """Expected output of every rank.

    ``inputs``: list over collectives of arrays [N, count] (int32 / float32 /
    uint16 bfloat16 bits).  Returns a list of [count] arrays, the value every
    rank must hold.
    """
    if isinstance(inputs, np.ndarray):
        inputs = [inputs]
    if op == "premulsum":
        # every rank's input enters the fold already scaled by its scalar;
        # then the fold is the sum's
        sc = np.asarray(scalars).reshape(len(inputs), -1)
        inputs = [np.stack([_premul(sc[w, r], x[r], dtype) for r in range(x.shape[0])])
                  for w, x in enumerate(inputs)]
        op = "sum"
    # one ring, or one per channel id (channel c runs ring c mod len(rings))
    rings = [list(r) for r in ring_order] if isinstance(ring_order[0], (list, tuple)) \
        else [list(ring_order)]
    N = len(rings[0])
    ids = [b for b in range(64) if (mask >> b) & 1]
    nch = len(ids)
    # rank_at[n, p]: user rank at ring position p of dense channel n, positions
    # counted from user rank 0 along that channel's ring
    rank_at = np.zeros((nch, N), dtype=np.int64)
    for n, cid in enumerate(ids):
        ring = rings[cid % len(rings)]
        pos0 = ring.index(0)
        rank_at[n] = [ring[(p + pos0) % N] for p in range(N)]
    cmax = chunk_max(proto, buff_size, chunk_steps, dtype)
    counts = [int(x.shape[1]) for x in inputs]
    owners, chans = owner_positions(counts, N, nch, cmax, dtype, with_channel=True)
    results = []
    for x, own, ch in zip(inputs, owners, chans):
        cols = np.arange(x.shape[1])
        acc = x[rank_at[ch, (own + 1) % N], cols]
        for k in range(2, N + 1):
            acc = _hop(acc, x[rank_at[ch, (own + k) % N], cols], dtype, op)
        if op == "avg":
            acc = _post_div(acc, N, dtype)
        results.append(acc)
    return results
