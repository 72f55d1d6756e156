/*
 * ring_sim.cpp -- CPU oracle: a plain, sequential simulator of the N-rank ring
 * AllReduce state machine (connectors with head/tail credit over FIFO slots,
 * the LL and LL128 line formats, the runRing schedule and the channel split).
 *
 * TEST INFRASTRUCTURE ONLY (see ring_sim.h).  It is deliberately slow and
 * direct so that every step can be checked against the two course pages it
 * follows:
 *   [C12] NCCL 专家课程 12 "Ring AllReduce 逐步推导、真实 Ring 与 Channel 并行"
 *   [C23] NCCL 专家课程 23 "Device Kernel、Primitives、Step/Credit 与 LL Flag"
 *
 * Readings taken where the pages leave a step open are marked READING.
 */
#include "ring_sim.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <random>
#include <thread>
#include <vector>

namespace {

size_t elem_size(int dtype) { return dtype == ORC_BFLOAT16 ? 2 : 4; }
int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align_up(int64_t a, int64_t b) { return div_up(a, b) * b; }

/* ---------------------------------------------------------------------------
 * Arithmetic of one reduction hop.  The partial sum travels between ranks in
 * the payload type, so it is rounded to that type after every addition
 * (READING: per-hop rounding for bf16).  Floating sums are formed exactly in
 * binary64 (two fp32 or two bf16 values differ by at most ~2^280 in scale, so
 * the binary64 sum is either exact or its second rounding is innocuous) and
 * then rounded once to the payload type.  int32 wraps modulo 2^32.
 * ------------------------------------------------------------------------- */
double bf16_to_double(uint16_t b) {
  uint32_t bits = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &bits, 4);
  return (double)f;
}

uint16_t bf16_round(double v) {
  if (std::isnan(v)) return 0x7FC0;
  const uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  const double a = std::fabs(v);
  if (a == 0.0) return sign;
  if (std::isinf(a)) return (uint16_t)(sign | 0x7F80);
  int e = 0;
  std::frexp(a, &e);  // a = m * 2^e with m in [0.5, 1)
  // bf16 keeps 8 significant bits; below 2^-126 the spacing stays 2^-133.
  const int q_exp = std::max(e, -125) - 8;
  const double q = std::ldexp(1.0, q_exp);
  const double r = std::nearbyint(a / q) * q;  // ties to even (default mode)
  if (r >= std::ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
  const float f = (float)r;  // exact: r has at most 8 significant bits
  uint32_t bits;
  std::memcpy(&bits, &f, 4);
  return (uint16_t)(sign | (uint16_t)(bits >> 16));
}

/* One reduction of the partial `a` with the own input `b`.  Floating
 * operands are taken exactly as binary64; a product of two fp32 (48
 * significant bits) or two bf16 values is exact there, so every result below
 * is rounded to the payload type once (or, for the sum, with an innocuous
 * second rounding, as above). */
double combine(int red, double acc, double x) {
  switch (red) {
    case ORC_RED_PROD: return acc * x;
    case ORC_RED_MAX: return x > acc ? x : acc;
    case ORC_RED_MIN: return x < acc ? x : acc;
    default: return acc + x;  // SUM, AVG
  }
}

void reduce_elem(int dtype, int red, const uint8_t* a, const uint8_t* b, uint8_t* out) {
  if (dtype == ORC_INT32) {
    int32_t x, y;
    std::memcpy(&x, a, 4);
    std::memcpy(&y, b, 4);
    uint32_t r;
    if (red == ORC_RED_PROD) r = (uint32_t)x * (uint32_t)y;  // low 32 bits
    else if (red == ORC_RED_MAX) r = (uint32_t)(y > x ? y : x);
    else if (red == ORC_RED_MIN) r = (uint32_t)(y < x ? y : x);
    else r = (uint32_t)x + (uint32_t)y;
    std::memcpy(out, &r, 4);
  } else if (dtype == ORC_FLOAT32) {
    float x, y;
    std::memcpy(&x, a, 4);
    std::memcpy(&y, b, 4);
    const float r = (float)combine(red, (double)x, (double)y);
    std::memcpy(out, &r, 4);
  } else {
    uint16_t x, y;
    std::memcpy(&x, a, 2);
    std::memcpy(&y, b, 2);
    const double dx = bf16_to_double(x), dy = bf16_to_double(y);
    uint16_t r;
    if (red == ORC_RED_MAX) r = dy > dx ? y : x;  // max / min pick an operand's bits
    else if (red == ORC_RED_MIN) r = dy < dx ? y : x;
    else r = bf16_round(combine(red, dx, dy));
    std::memcpy(out, &r, 2);
  }
}

/* PreMulSum's scaling of one own input: s * x rounded once to the payload
 * type (the product of two fp32 or two bf16 values is exact in binary64). */
void premul_elem(int dtype, const uint8_t* s, const uint8_t* x, uint8_t* out) {
  if (dtype == ORC_INT32) {
    uint32_t a, b;
    std::memcpy(&a, s, 4);
    std::memcpy(&b, x, 4);
    const uint32_t r = a * b;  // low 32 bits
    std::memcpy(out, &r, 4);
  } else if (dtype == ORC_FLOAT32) {
    float a, b;
    std::memcpy(&a, s, 4);
    std::memcpy(&b, x, 4);
    const float r = (float)((double)a * (double)b);
    std::memcpy(out, &r, 4);
  } else {
    uint16_t a, b;
    std::memcpy(&a, s, 2);
    std::memcpy(&b, x, 2);
    const uint16_t r = bf16_round(bf16_to_double(a) * bf16_to_double(b));
    std::memcpy(out, &r, 2);
  }
}

/* The AVG post-op: the owner's final sum divided by N, rounded once to the
 * payload type (int32: the wrapped sum, truncated toward zero).  binary64
 * holds the quotient to 53 bits, and 53 >= 2*24 + 2, so rounding it again to
 * fp32 or bf16 equals rounding the exact quotient. */
void post_div(int dtype, int nranks, uint8_t* v) {
  if (dtype == ORC_INT32) {
    int32_t x;
    std::memcpy(&x, v, 4);
    const int32_t q = (int32_t)((int64_t)x / nranks);  // C division truncates toward zero
    std::memcpy(v, &q, 4);
  } else if (dtype == ORC_FLOAT32) {
    float x;
    std::memcpy(&x, v, 4);
    const float q = (float)((double)x / (double)nranks);
    std::memcpy(v, &q, 4);
  } else {
    uint16_t x;
    std::memcpy(&x, v, 2);
    const uint16_t q = bf16_round(bf16_to_double(x) / (double)nranks);
    std::memcpy(v, &q, 2);
  }
}

/* ---------------------------------------------------------------------------
 * Protocol geometry [C23 "Buffer 到 Chunk 的实测公式", "LL：Data 与 Flag 同
 * Line", "LL128：15/16 Payload"].
 *   Simple: a step is buffSize/NCCL_STEPS bytes of payload, a chunk is
 *           chunkSteps steps.
 *   LL:     a step is buffSize/NCCL_STEPS bytes of 16-byte lines, half of
 *           which is payload; READING: a chunk is one step of payload.
 *   LL128:  a step is buffSize/NCCL_STEPS bytes of 128-byte lines carrying
 *           120 payload bytes each; READING: a chunk is one step of payload.
 * ------------------------------------------------------------------------- */
constexpr int kSlicesPerChunk = 2;  // READING: SlicePerChunk = 2, StepPerSlice = chunkSteps/2

int64_t chunk_max_elems(int proto, size_t buff_size, int chunk_steps, size_t es, int slots) {
  const int64_t step_bytes = (int64_t)(buff_size / (size_t)slots);
  if (proto == ORC_PROTO_SIMPLE) return (step_bytes / (int64_t)es) * chunk_steps;
  if (proto == ORC_PROTO_LL) return (step_bytes / 16) * 8 / (int64_t)es;
  return (step_bytes / 128) * 120 / (int64_t)es;
}

bool valid_params(int nranks, uint64_t mask, int proto, size_t buff_size, int chunk_steps,
                  int dtype, int slots) {
  if (nranks < 2 || nranks > 64) return false;
  if (mask == 0) return false;
  if (dtype != ORC_INT32 && dtype != ORC_FLOAT32 && dtype != ORC_BFLOAT16) return false;
  if (slots < 1 || slots > 64) return false;
  if (proto == ORC_PROTO_SIMPLE) {
    if (chunk_steps != 2 && chunk_steps != 4 && chunk_steps != 8) return false;
    if (slots % (chunk_steps / 2) != 0) return false;
    // a slice is rounded up to 16 elements; 64-byte steps keep it inside its slots
    if (buff_size == 0 || buff_size % ((size_t)slots * 64) != 0) return false;
  } else if (proto == ORC_PROTO_LL) {
    if (buff_size == 0 || buff_size % ((size_t)slots * 32) != 0) return false;
  } else if (proto == ORC_PROTO_LL128) {
    if (buff_size == 0 || buff_size % ((size_t)slots * 256) != 0) return false;
  } else {
    return false;
  }
  return true;
}

/* Channel split, READING of the pages' ncclCollCbdPart [C23 "Ring AllReduce
 * 到 Primitive"; C12 "多 channel 如何并行"]: the collectives of the launch are
 * laid end to end (each starting 16-byte aligned) and the stream is cut into
 * one contiguous, 16-byte aligned range per active channel, in channel order.
 * Every (collective, channel) overlap becomes a piece that runs runRing on its
 * own. */
std::vector<orc_piece> make_pieces(int nranks, uint64_t mask, int proto, size_t buff_size,
                                   int chunk_steps, int dtype, int nworks, const size_t* counts,
                                   int slots, int64_t* chunk_max_out) {
  (void)nranks;
  const int64_t es = (int64_t)elem_size(dtype);
  const int64_t vec = 16 / es;
  std::vector<int64_t> start(nworks);
  int64_t total = 0;
  for (int w = 0; w < nworks; ++w) {
    start[w] = align_up(total, vec);
    total = start[w] + (int64_t)counts[w];
  }
  std::vector<int> ids;
  for (int b = 0; b < 64; ++b)
    if (mask & (1ull << b)) ids.push_back(b);
  const int nch = (int)ids.size();
  const int64_t chunk_max = chunk_max_elems(proto, buff_size, chunk_steps, (size_t)es, slots);
  if (chunk_max_out) *chunk_max_out = chunk_max;
  std::vector<orc_piece> out;
  if (total == 0) return out;
  const int64_t per_channel = align_up(div_up(total, nch), vec);
  for (int n = 0; n < nch; ++n) {
    const int64_t lo = (int64_t)n * per_channel;
    const int64_t hi = std::min<int64_t>(lo + per_channel, total);
    for (int w = 0; w < nworks; ++w) {
      const int64_t a = std::max(lo, start[w]);
      const int64_t b = std::min(hi, start[w] + (int64_t)counts[w]);
      if (a >= b) continue;
      orc_piece p;
      p.channel = n;
      p.channel_id = ids[n];
      p.work = w;
      p.pad = 0;
      p.grid_offset = a - start[w];
      p.channel_count = b - a;
      p.chunk_count = chunk_max;
      out.push_back(p);
    }
  }
  return out;
}

/* ---------------------------------------------------------------------------
 * The collective simulator.
 * ------------------------------------------------------------------------- */
struct Unit {
  int op;
  int work;
  int chunk;
  int loop;
  int first_of_call;  // first slice of a primitive call (counts the call once)
  int raw_recv;       // the loop's first receive: its data is the previous rank's raw input
  int64_t offset;     // element offset of this unit in the collective's buffers
  int64_t nelem;      // elements moved by this unit (may be 0)
  int64_t call_offset, call_nelem;
};

struct Conn {
  std::vector<uint8_t> fifo;  // `slots` slots of step_bytes each
  uint64_t head = 0;          // consumer progress (credit back to the sender)
  uint64_t tail = 0;          // producer progress (Simple only)
};

struct Agent {
  int rank = 0, n = 0;
  std::vector<Unit> prog;
  size_t pc = 0;
  uint64_t send_step = 0, recv_step = 0;
};

struct Sim {
  int N = 0, C = 0, proto = 0, dtype = 0, slots = 8, chunk_steps = 4;
  int64_t es = 4, step_bytes = 0, sps = 1;
  bool drop_head = false;
  uint64_t ll_period = 1ull << 32;
  int red = ORC_RED_SUM;
  const uint8_t* scalars = nullptr;  // PreMulSum: [work * N + rank] payload-type scalars
  bool direct = false;  // Simple: all-gather half writes into the next rank's receive buffer
  bool direct_read = false;  // Simple: the loop's first receive reads the previous send buffer
  // Ring of each active channel: entry [n * N + rank] for dense channel n.
  // Channel id c follows ring c mod nrings [C12 "为什么 channels 会重复":
  // the base rings are duplicated onto the following channels].
  std::vector<int> index, prev, next;
  std::vector<Conn> conn;  // conn[rank * C + n]: FIFO that `rank` receives on, channel n
  const void* const* sendbufs = nullptr;
  void* const* recvbufs = nullptr;
  orc_stats* stats = nullptr;
  orc_call* log = nullptr;
  int64_t log_cap = 0;
  std::vector<int> channel_ids;

  int64_t lines_for(int64_t nelem) const {
    const int64_t bytes = nelem * es;
    if (proto == ORC_PROTO_LL) return div_up(bytes, 8);
    if (proto == ORC_PROTO_LL128) return div_up(bytes, 120);
    return 0;
  }
  // LL line flag of a step: step+1 modulo the flag period (2^32, or 2^8 in
  // the wrap test mode) [C23 "LL：Data 与 Flag 同 Line"].
  uint32_t ll_flag(uint64_t step) const { return (uint32_t)((step + 1) % ll_period); }
  bool ll_cleanup(uint64_t step) const {
    const uint64_t half = ll_period / 2;
    return (step + 1) % half >= half - (uint64_t)slots;
  }

  uint8_t* slot(Conn& c, uint64_t step) { return c.fifo.data() + (step % (uint64_t)slots) * step_bytes; }

  /* A receiver may consume step `step` of an LL / LL128 connector once every
   * line it needs carries the flag of that step [C23 "LL：Data 与 Flag 同
   * Line": both 32-bit flags equal step+1; "LL128": flag word equals step+1]. */
  bool lines_ready(Conn& c, uint64_t step, int64_t nlines) {
    uint8_t* s = slot(c, step);
    for (int64_t j = 0; j < nlines; ++j) {
      if (proto == ORC_PROTO_LL) {
        uint32_t f1, f2;
        std::memcpy(&f1, s + 16 * j + 4, 4);
        std::memcpy(&f2, s + 16 * j + 12, 4);
        const uint32_t want = ll_flag(step);
        if (f1 != want || f2 != want) return false;
      } else {
        uint64_t f;
        std::memcpy(&f, s + 128 * j + 120, 8);
        if (f != step + 1) return false;
      }
    }
    return true;
  }

  void read_payload(Conn& c, uint64_t step, int64_t nelem, std::vector<uint8_t>& out) {
    const int64_t bytes = nelem * es;
    out.assign((size_t)bytes, 0);
    uint8_t* s = slot(c, step);
    if (proto == ORC_PROTO_SIMPLE) {
      std::memcpy(out.data(), s, (size_t)bytes);
    } else if (proto == ORC_PROTO_LL) {
      for (int64_t b = 0; b < bytes; ++b) {
        const int64_t line = b / 8, within = b % 8;
        // data1 holds payload bytes 0..3 of the line, data2 bytes 4..7
        const int64_t pos = 16 * line + (within < 4 ? within : 8 + (within - 4));
        out[(size_t)b] = s[pos];
      }
    } else {
      for (int64_t b = 0; b < bytes; ++b) {
        const int64_t line = b / 120, within = b % 120;
        out[(size_t)b] = s[128 * line + within];
      }
    }
  }

  void write_payload(Conn& c, uint64_t step, const std::vector<uint8_t>& val) {
    const int64_t bytes = (int64_t)val.size();
    uint8_t* s = slot(c, step);
    if (proto == ORC_PROTO_SIMPLE) {
      std::memcpy(s, val.data(), (size_t)bytes);
      return;
    }
    const int64_t nlines = proto == ORC_PROTO_LL ? div_up(bytes, 8) : div_up(bytes, 120);
    for (int64_t j = 0; j < nlines; ++j) {
      if (proto == ORC_PROTO_LL) {
        uint8_t line[16];
        std::memset(line, 0, 16);
        for (int k = 0; k < 8; ++k) {
          const int64_t b = 8 * j + k;
          if (b < bytes) line[k < 4 ? k : 8 + (k - 4)] = val[(size_t)b];
        }
        const uint32_t flag = ll_flag(step);
        std::memcpy(line + 4, &flag, 4);
        std::memcpy(line + 12, &flag, 4);
        std::memcpy(s + 16 * j, line, 16);
      } else {
        uint8_t line[128];
        std::memset(line, 0, 128);
        for (int k = 0; k < 120; ++k) {
          const int64_t b = 120 * j + k;
          if (b < bytes) line[k] = val[(size_t)b];
        }
        const uint64_t flag = step + 1;
        std::memcpy(line + 120, &flag, 8);
        std::memcpy(s + 128 * j, line, 128);
      }
    }
    // LL cleanup: in the last NCCL_STEPS steps of each half of the flag period
    // the rest of the slot takes the current flag, so no line keeps a
    // generation old enough to come round again.
    if (proto == ORC_PROTO_LL && ll_cleanup(step)) {
      const uint32_t flag = ll_flag(step);
      for (int64_t j = nlines; j < step_bytes / 16; ++j) {
        std::memset(s + 16 * j, 0, 16);
        std::memcpy(s + 16 * j + 4, &flag, 4);
        std::memcpy(s + 16 * j + 12, &flag, 4);
      }
    }
  }

  /* One unit = one slice (Simple) or one step (LL, LL128) of a primitive call:
   * wait -> reduce/copy -> publish [C23 "Primitive API 是模板组合", "Simple 的
   * Credit 与 Step", "发布顺序与 Fence"].  Returns false when a wait fails. */
  bool try_unit(Agent& ag) { return try_unit(ag, stats); }
  // `st`: where this unit's counts go (each thread of the channel-parallel
  // mode has its own, merged at the end)
  bool try_unit(Agent& ag, orc_stats* st) {
    const Unit& u = ag.prog[ag.pc];
    const bool recv = u.op != ORC_OP_SEND;
    const bool send = u.op != ORC_OP_RECV;
    // Direct variants [C23 "发布顺序与 Fence"]: directRecvReduceCopySend and
    // directRecvCopySend put their result straight into the next rank's
    // receive buffer (no FIFO slot, so no send credit to wait for);
    // directRecvCopySend and directRecv find their input already in their own
    // receive buffer.  Steps still advance on both sides.
    const bool direct_send =
        direct && (u.op == ORC_OP_RECV_REDUCE_COPY_SEND || u.op == ORC_OP_RECV_COPY_SEND);
    const bool direct_recv = direct && (u.op == ORC_OP_RECV_COPY_SEND || u.op == ORC_OP_RECV);
    // Direct read: the loop's opening send leaves its data where it is, and
    // the next rank's first receive reads it from this rank's send buffer.
    const bool skip_send = direct_read && u.op == ORC_OP_SEND;
    const bool read_prev = direct_read && u.raw_recv;
    Conn& rc = conn[(size_t)ag.rank * C + ag.n];
    const int nxt = next[(size_t)ag.n * N + ag.rank];
    Conn& sc = conn[(size_t)nxt * C + ag.n];
    const uint64_t adv = (uint64_t)sps;
    // sender wait: head + NCCL_STEPS >= step + StepPerSlice
    if (send && !direct_send && !skip_send && !(sc.head + (uint64_t)slots >= ag.send_step + adv))
      return false;
    // receiver wait: tail >= step + StepPerSlice (Simple) or line flags (LL, LL128)
    if (recv) {
      if (proto == ORC_PROTO_SIMPLE) {
        if (!(rc.tail >= ag.recv_step + adv)) return false;
      } else if (!lines_ready(rc, ag.recv_step, lines_for(u.nelem))) {
        return false;
      }
    }
    const uint8_t* src =
        (const uint8_t*)sendbufs[(size_t)u.work * N + ag.rank] + u.offset * es;
    uint8_t* dst = (uint8_t*)recvbufs[(size_t)u.work * N + ag.rank] + u.offset * es;
    uint8_t* next_dst = (uint8_t*)recvbufs[(size_t)u.work * N + nxt] + u.offset * es;
    std::vector<uint8_t> got;
    if (recv && read_prev) {
      const int prv = prev[(size_t)ag.n * N + ag.rank];
      const uint8_t* prev_src = (const uint8_t*)sendbufs[(size_t)u.work * N + prv] + u.offset * es;
      got.assign(prev_src, prev_src + u.nelem * es);
      if (red == ORC_RED_PREMULSUM)  // the raw input enters the fold here, with its owner's scalar
        for (int64_t i = 0; i < u.nelem; ++i)
          premul_elem(dtype, scalars + ((size_t)u.work * N + prv) * es, got.data() + i * es,
                      got.data() + i * es);
    } else if (recv && direct_recv) got.assign(dst, dst + u.nelem * es);
    else if (recv) read_payload(rc, ag.recv_step, u.nelem, got);
    std::vector<uint8_t> val((size_t)(u.nelem * es));
    const uint8_t* my_scalar = scalars ? scalars + ((size_t)u.work * N + ag.rank) * es : nullptr;
    for (int64_t i = 0; i < u.nelem; ++i) {
      uint8_t* v = val.data() + i * es;
      // the rank's own input as it enters the fold (PreMulSum: scaled)
      uint8_t own[8];
      std::memcpy(own, src + i * es, (size_t)es);
      if (red == ORC_RED_PREMULSUM) premul_elem(dtype, my_scalar, own, own);
      switch (u.op) {
        case ORC_OP_SEND:
          std::memcpy(v, own, (size_t)es);
          break;
        case ORC_OP_RECV_REDUCE_SEND:
        case ORC_OP_RECV_REDUCE_COPY_SEND:
          reduce_elem(dtype, red == ORC_RED_PREMULSUM ? ORC_RED_SUM : red, got.data() + i * es, own, v);
          if (u.op == ORC_OP_RECV_REDUCE_COPY_SEND && red == ORC_RED_AVG) post_div(dtype, N, v);
          break;
        default:
          std::memcpy(v, got.data() + i * es, (size_t)es);
          break;
      }
    }
    if (u.op == ORC_OP_RECV_REDUCE_COPY_SEND ||
        ((u.op == ORC_OP_RECV_COPY_SEND || u.op == ORC_OP_RECV) && !direct_recv)) {
      if (u.nelem > 0) std::memcpy(dst, val.data(), val.size());
    }
    if (send && direct_send) {
      if (u.nelem > 0) std::memcpy(next_dst, val.data(), val.size());
    } else if (send && !skip_send) {
      write_payload(sc, ag.send_step, val);
    }
    // publish: receiver frees the slots (head), sender announces data (tail)
    if (recv) {
      ag.recv_step += adv;
      if (!drop_head) rc.head = ag.recv_step;
    }
    if (send) {
      ag.send_step += adv;
      if (proto == ORC_PROTO_SIMPLE) sc.tail = ag.send_step;
    }
    if (st) {
      st->units_run++;
      if (u.first_of_call) {
        if (send) st->send_ops[ag.rank]++;
        if (recv) st->recv_ops[ag.rank]++;
      }
      if (send) {
        st->payload_sent[ag.rank] += u.nelem * es;
        if (proto == ORC_PROTO_SIMPLE) {
          if (!direct_send && !skip_send) st->wire_sent[ag.rank] += u.nelem * es;  // FIFO bytes
        }
        else if (proto == ORC_PROTO_LL) st->wire_sent[ag.rank] += lines_for(u.nelem) * 16;
        else st->wire_sent[ag.rank] += lines_for(u.nelem) * 128;
      }
      if (u.first_of_call && log && st->calls_recorded < log_cap) {
        orc_call& c = log[st->calls_recorded++];
        c.rank = ag.rank;
        c.channel_id = channel_ids[ag.n];
        c.work = u.work;
        c.op = u.op;
        c.chunk = u.chunk;
        c.loop = u.loop;
        c.offset = u.call_offset;
        c.nelem = u.call_nelem;
      }
    }
    return true;
  }
};

/* Expand runRing for one (rank, channel) into units [C12 "runRing 的数据切
 * 分", "源码步骤一..五"; C23 "Slice Size"]. */
void build_program(Agent& ag, const Sim& sim, const std::vector<orc_piece>& pieces) {
  const int N = sim.N;
  std::vector<int> ops(2 * N - 1), chunks(2 * N - 1);
  orc_ring_schedule(N, sim.index[(size_t)ag.n * N + ag.rank], ops.data(), chunks.data());
  const int64_t vec = 16 / sim.es;
  const int64_t step_elems = sim.step_bytes / sim.es;
  for (const orc_piece& p : pieces) {
    if (p.channel != ag.n) continue;
    const int64_t loop_count = (int64_t)N * p.chunk_count;
    int loop = 0;
    for (int64_t elem_off = 0; elem_off < p.channel_count; elem_off += loop_count, ++loop) {
      const int64_t rem = p.channel_count - elem_off;
      int64_t cc = p.chunk_count;
      if (rem < loop_count) cc = align_up(div_up(rem, N), vec);  // tail loop re-chunking
      for (int k = 0; k < 2 * N - 1; ++k) {
        const int c = chunks[k];
        const int64_t chunk_off = (int64_t)c * cc;
        const int64_t nelem = std::max<int64_t>(0, std::min<int64_t>(cc, rem - chunk_off));
        const int64_t offset = p.grid_offset + elem_off + chunk_off;
        if (sim.proto == ORC_PROTO_SIMPLE) {
          // sliceSize = max(divUp(nelem, 16*SlicePerChunk)*16, stepSize*StepPerSlice/32)
          const int64_t slice =
              std::max<int64_t>(div_up(nelem, 16 * kSlicesPerChunk) * 16, step_elems * sim.sps / 32);
          for (int s = 0; s < kSlicesPerChunk; ++s) {
            const int64_t soff = (int64_t)s * slice;
            const int64_t sn = std::max<int64_t>(0, std::min<int64_t>(slice, nelem - soff));
            Unit u{ops[k], p.work, c, loop, s == 0, k == 1, offset + soff, sn, offset, nelem};
            ag.prog.push_back(u);
          }
        } else {
          Unit u{ops[k], p.work, c, loop, 1, k == 1, offset, nelem, offset, nelem};
          ag.prog.push_back(u);
        }
      }
    }
  }
}

}  // namespace

extern "C" {

uint16_t orc_bf16_round(double v) { return bf16_round(v); }

int orc_ring_setup(int nranks, const int* ring_order, int* index, int* prev, int* next) {
  if (nranks < 2 || nranks > 64 || !ring_order) return ORC_INVALID;
  std::vector<int> seen(nranks, 0), nx(nranks, -1);
  for (int i = 0; i < nranks; ++i) {
    const int r = ring_order[i];
    if (r < 0 || r >= nranks || seen[r]) return ORC_INVALID;
    seen[r] = 1;
  }
  for (int i = 0; i < nranks; ++i) nx[ring_order[i]] = ring_order[(i + 1) % nranks];
  // Walk `next` N times from every rank: each walk must visit every rank once
  // and come back to its start [C12 "Graph 如何变成完整 ring"].
  for (int start = 0; start < nranks; ++start) {
    std::vector<int> visited(nranks, 0);
    int cur = start;
    for (int i = 0; i < nranks; ++i) {
      if (visited[cur]) return ORC_INVALID;
      visited[cur] = 1;
      cur = nx[cur];
    }
    if (cur != start) return ORC_INVALID;
  }
  // ring index = distance of the rank from user rank 0 along the ring
  // [C12 "ring index 如何计算"].
  int ix_zero = 0;
  for (int i = 0; i < nranks; ++i)
    if (ring_order[i] == 0) ix_zero = i;
  for (int i = 0; i < nranks; ++i) {
    const int r = ring_order[i];
    if (index) index[r] = (i - ix_zero + nranks) % nranks;
    if (next) next[r] = ring_order[(i + 1) % nranks];
    if (prev) prev[r] = ring_order[(i - 1 + nranks) % nranks];
  }
  return ORC_OK;
}

int orc_ring_schedule(int nranks, int ring_index, int* ops, int* chunks) {
  if (nranks < 2 || ring_index < 0 || ring_index >= nranks) return -1;
  auto mod = [nranks](int x) { return ((x % nranks) + nranks) % nranks; };
  int k = 0;
  // reduce-scatter half: send the chunk i-1, then add-and-forward i-2 .. i-(N-1)
  ops[k] = ORC_OP_SEND;
  chunks[k++] = mod(ring_index - 1);
  for (int j = 2; j < nranks; ++j) {
    ops[k] = ORC_OP_RECV_REDUCE_SEND;
    chunks[k++] = mod(ring_index - j);
  }
  // fused boundary: the final add of the own chunk i, written out and forwarded
  ops[k] = ORC_OP_RECV_REDUCE_COPY_SEND;
  chunks[k++] = ring_index;
  // all-gather half: copy-and-forward i-1 .. i-(N-2), then receive i+1
  for (int j = 1; j < nranks - 1; ++j) {
    ops[k] = ORC_OP_RECV_COPY_SEND;
    chunks[k++] = mod(ring_index - j);
  }
  ops[k] = ORC_OP_RECV;
  chunks[k++] = mod(ring_index + 1);
  return k;
}

int orc_geometry(int nranks, uint64_t channel_mask, int proto, size_t buff_size, int chunk_steps,
                 int dtype, int nworks, const size_t* counts, orc_piece* pieces, int max_pieces,
                 int64_t* chunk_max_out) {
  if (!valid_params(nranks, channel_mask, proto, buff_size, chunk_steps, dtype, 8)) return -1;
  if (nworks < 1 || !counts) return -1;
  std::vector<orc_piece> ps = make_pieces(nranks, channel_mask, proto, buff_size, chunk_steps,
                                          dtype, nworks, counts, 8, chunk_max_out);
  const int n = (int)std::min<size_t>(ps.size(), (size_t)std::max(max_pieces, 0));
  for (int i = 0; i < n; ++i) pieces[i] = ps[i];
  return (int)ps.size();
}

int orc_allreduce(int nranks, const int* ring_order, uint64_t channel_mask, int proto,
                  size_t buff_size, int chunk_steps, int dtype, int nworks, const size_t* counts,
                  const void* const* sendbufs, void* const* recvbufs, int slots, int sched,
                  uint64_t seed, int options, orc_stats* stats, orc_call* call_log,
                  int64_t call_log_cap) {
  return orc_allreduce_rings(nranks, 1, ring_order, channel_mask, proto, buff_size, chunk_steps,
                             dtype, nworks, counts, sendbufs, recvbufs, slots, sched, seed, options,
                             stats, call_log, call_log_cap);
}

int orc_allreduce_rings(int nranks, int nrings, const int* ring_orders, uint64_t channel_mask,
                        int proto, size_t buff_size, int chunk_steps, int dtype, int nworks,
                        const size_t* counts, const void* const* sendbufs, void* const* recvbufs,
                        int slots, int sched, uint64_t seed, int options, orc_stats* stats,
                        orc_call* call_log, int64_t call_log_cap) {
  if (((options >> ORC_OPT_RED_SHIFT) & 15) == ORC_RED_PREMULSUM) return ORC_INVALID;  // needs scalars
  return orc_allreduce_premul(nranks, nrings, ring_orders, channel_mask, proto, buff_size,
                              chunk_steps, dtype, nworks, counts, sendbufs, recvbufs, nullptr, slots,
                              sched, seed, options, stats, call_log, call_log_cap);
}

int orc_allreduce_premul(int nranks, int nrings, const int* ring_orders, uint64_t channel_mask,
                         int proto, size_t buff_size, int chunk_steps, int dtype, int nworks,
                         const size_t* counts, const void* const* sendbufs, void* const* recvbufs,
                         const void* scalars, int slots, int sched, uint64_t seed, int options,
                         orc_stats* stats, orc_call* call_log, int64_t call_log_cap) {
  if (!valid_params(nranks, channel_mask, proto, buff_size, chunk_steps, dtype, slots))
    return ORC_INVALID;
  if (nworks < 1 || !counts || !sendbufs || !recvbufs) return ORC_INVALID;
  Sim sim;
  sim.N = nranks;
  sim.proto = proto;
  sim.dtype = dtype;
  sim.slots = slots;
  sim.chunk_steps = chunk_steps;
  sim.es = (int64_t)elem_size(dtype);
  sim.step_bytes = (int64_t)(buff_size / (size_t)slots);
  sim.sps = proto == ORC_PROTO_SIMPLE ? chunk_steps / 2 : 1;
  sim.drop_head = (options & ORC_OPT_DROP_RECV_HEAD) != 0;
  sim.direct = (options & ORC_OPT_DIRECT) != 0;
  sim.direct_read = (options & ORC_OPT_DIRECT_READ) != 0;
  if ((sim.direct || sim.direct_read) && proto != ORC_PROTO_SIMPLE) return ORC_INVALID;
  sim.red = scalars ? ORC_RED_PREMULSUM : (options >> ORC_OPT_RED_SHIFT) & 15;
  sim.scalars = (const uint8_t*)scalars;
  if (options & ORC_OPT_LL_WRAP8) sim.ll_period = 256;
  if ((uint64_t)slots >= sim.ll_period / 2) return ORC_INVALID;
  if (sim.red > ORC_RED_PREMULSUM) return ORC_INVALID;
  sim.sendbufs = sendbufs;
  sim.recvbufs = recvbufs;
  sim.stats = stats;
  sim.log = call_log;
  sim.log_cap = call_log ? call_log_cap : 0;
  if (nrings < 1 || !ring_orders) return ORC_INVALID;
  for (int b = 0; b < 64; ++b)
    if (channel_mask & (1ull << b)) sim.channel_ids.push_back(b);
  sim.C = (int)sim.channel_ids.size();
  sim.index.assign((size_t)sim.C * nranks, 0);
  sim.prev.assign((size_t)sim.C * nranks, 0);
  sim.next.assign((size_t)sim.C * nranks, 0);
  for (int n = 0; n < sim.C; ++n) {
    const int* order = ring_orders + (size_t)(sim.channel_ids[n] % nrings) * nranks;
    const size_t at = (size_t)n * nranks;
    if (orc_ring_setup(nranks, order, &sim.index[at], &sim.prev[at], &sim.next[at]) != ORC_OK)
      return ORC_INVALID;
  }
  if (stats) {
    std::memset(stats, 0, sizeof(*stats));
    stats->deadlock_rank = -1;
    stats->deadlock_channel = -1;
  }
  std::vector<orc_piece> pieces = make_pieces(nranks, channel_mask, proto, buff_size, chunk_steps,
                                              dtype, nworks, counts, slots, nullptr);
  sim.conn.resize((size_t)nranks * sim.C);
  for (Conn& c : sim.conn) c.fifo.assign(buff_size, 0);
  std::vector<Agent> agents((size_t)nranks * sim.C);
  for (int r = 0; r < nranks; ++r)
    for (int n = 0; n < sim.C; ++n) {
      Agent& ag = agents[(size_t)r * sim.C + n];
      ag.rank = r;
      ag.n = n;
      build_program(ag, sim, pieces);
    }
  auto report_deadlock = [&]() {
    if (!stats) return;
    for (Agent& ag : agents)
      if (ag.pc < ag.prog.size()) {
        stats->deadlock_rank = ag.rank;
        stats->deadlock_channel = sim.channel_ids[ag.n];
        stats->deadlock_send_step = (int64_t)ag.send_step;
        stats->deadlock_recv_step = (int64_t)ag.recv_step;
        return;
      }
  };
  if (sched == 2) {
    // Channel-parallel: channels share no connector, no agent and no output
    // element, so each thread runs whole channels (n = t, t + T, ...) with
    // the round-robin schedule below restricted to that channel's agents,
    // counting into its own statistics.  The results are those of any other
    // interleaving.
    if (call_log) return ORC_INVALID;
    const int hw = (int)std::thread::hardware_concurrency();
    int T = seed ? (int)seed : (hw > 0 ? hw : 1);
    if (T > sim.C) T = sim.C;
    std::vector<orc_stats> tstats((size_t)T);
    std::vector<int> rcode((size_t)T, ORC_OK);
    std::vector<int> stuck((size_t)T, -1);  // an agent index of a deadlocked channel
    auto run_channels = [&](int t) {
      orc_stats* st = stats ? &tstats[(size_t)t] : nullptr;
      if (st) std::memset(st, 0, sizeof(*st));
      for (int n = t; n < sim.C; n += T) {
        while (true) {
          bool progress = false, all_done = true;
          for (int r = 0; r < nranks; ++r) {
            Agent& ag = agents[(size_t)r * sim.C + n];
            while (ag.pc < ag.prog.size() && sim.try_unit(ag, st)) {
              ++ag.pc;
              progress = true;
            }
            if (ag.pc < ag.prog.size()) all_done = false;
          }
          if (all_done) break;
          if (!progress) {
            rcode[(size_t)t] = ORC_DEADLOCK;
            for (int r = 0; r < nranks; ++r)
              if (agents[(size_t)r * sim.C + n].pc < agents[(size_t)r * sim.C + n].prog.size()) {
                stuck[(size_t)t] = r * sim.C + n;
                break;
              }
            return;
          }
        }
      }
    };
    std::vector<std::thread> pool;
    for (int t = 1; t < T; ++t) pool.emplace_back(run_channels, t);
    run_channels(0);
    for (std::thread& th : pool) th.join();
    if (stats) {
      for (const orc_stats& ts : tstats) {
        stats->units_run += ts.units_run;
        for (int r = 0; r < 64; ++r) {
          stats->send_ops[r] += ts.send_ops[r];
          stats->recv_ops[r] += ts.recv_ops[r];
          stats->payload_sent[r] += ts.payload_sent[r];
          stats->wire_sent[r] += ts.wire_sent[r];
        }
      }
    }
    for (int t = 0; t < T; ++t)
      if (rcode[(size_t)t] != ORC_OK) {
        if (stats && stuck[(size_t)t] >= 0) {
          const Agent& ag = agents[(size_t)stuck[(size_t)t]];
          stats->deadlock_rank = ag.rank;
          stats->deadlock_channel = sim.channel_ids[ag.n];
          stats->deadlock_send_step = (int64_t)ag.send_step;
          stats->deadlock_recv_step = (int64_t)ag.recv_step;
        }
        return rcode[(size_t)t];
      }
  } else if (sched == 0) {
    // Deterministic: visit agents round robin; each runs until it blocks.
    while (true) {
      bool progress = false, all_done = true;
      for (Agent& ag : agents) {
        while (ag.pc < ag.prog.size() && sim.try_unit(ag)) {
          ++ag.pc;
          progress = true;
        }
        if (ag.pc < ag.prog.size()) all_done = false;
      }
      if (all_done) break;
      if (!progress) {
        report_deadlock();
        return ORC_DEADLOCK;
      }
    }
  } else {
    // Seeded random interleaving: one unit of one randomly chosen agent at a time.
    std::mt19937_64 rng(seed);
    std::vector<size_t> order(agents.size());
    for (size_t i = 0; i < order.size(); ++i) order[i] = i;
    while (true) {
      std::shuffle(order.begin(), order.end(), rng);
      bool any_left = false, ran = false;
      for (size_t i : order) {
        Agent& ag = agents[i];
        if (ag.pc >= ag.prog.size()) continue;
        any_left = true;
        if (sim.try_unit(ag)) {
          ++ag.pc;
          ran = true;
          break;
        }
      }
      if (!any_left) break;
      if (!ran) {
        report_deadlock();
        return ORC_DEADLOCK;
      }
    }
  }
  return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Single-connector fault model [C23 "状态机故障注入"].  The producer and the
 * consumer are explicit micro-step machines; the scheduler always lets the
 * consumer move first when it can, which is the interleaving that exposes an
 * early publication.  Payload words are tagged with their step so that any
 * stale or torn read is detected.
 * ------------------------------------------------------------------------- */
namespace {

uint32_t tag32(int64_t step, int64_t word) {
  uint32_t x = (uint32_t)(step * 0x9E3779B1u) ^ (uint32_t)(word * 0x85EBCA77u) ^ 0xA5A5A5A5u;
  return x ? x : 1u;  // never equal to the zero-initialised FIFO
}

}  // namespace

int orc_stream_fault(int proto, int fault, int slots, int nsteps, int64_t* steps_done,
                     int64_t* consumed, int64_t* bad_step) {
  if (slots < 1 || slots > 64 || nsteps < 1) return ORC_INVALID;
  const int kLines = 4;  // lines (LL, LL128) or 32-bit words (Simple) per step
  // FIFO storage: per slot, per line: up to 16 u64 words (LL uses 4 u32 = 2 u64).
  std::vector<uint32_t> simple((size_t)slots * kLines, 0);
  std::vector<uint32_t> ll((size_t)slots * kLines * 4, 0);        // data1 flag1 data2 flag2
  std::vector<uint64_t> ll128((size_t)slots * kLines * 16, 0);    // 15 data words + flag
  uint64_t head = 0, tail = 0;
  int64_t p = 0, c = 0;      // producer / consumer step
  int pph = 0, cph = 0;      // micro-phase within the step
  int64_t first_bad = -1;
  const bool const_flag = fault == 4;
  auto ll_flag = [&](int64_t step) -> uint32_t { return const_flag ? 1u : (uint32_t)(step + 1); };

  // Producer micro-phases per step.
  //   Simple: 0 wait credit, 1 write payload, 2 publish tail  (fault 2: 1<->2)
  //   LL:     0 wait credit, 1..kLines write line j
  //   LL128:  0 wait credit, then per line: data, flag         (fault 6: flag, data)
  auto producer_phases = [&]() {
    if (proto == ORC_PROTO_SIMPLE) return 3;
    if (proto == ORC_PROTO_LL) return 1 + kLines;
    return 1 + 2 * kLines;
  };
  auto producer_step = [&]() -> bool {  // returns false if blocked
    if (pph == 0) {
      if (!(head + (uint64_t)slots >= (uint64_t)p + 1)) return false;  // credit
    } else if (proto == ORC_PROTO_SIMPLE) {
      const bool write_payload = (fault == 2) ? (pph == 2) : (pph == 1);
      if (write_payload) {
        for (int w = 0; w < kLines; ++w) simple[(size_t)(p % slots) * kLines + w] = tag32(p, w);
      } else {
        tail = (uint64_t)p + 1;
      }
    } else if (proto == ORC_PROTO_LL) {
      const int j = pph - 1;
      uint32_t* line = &ll[((size_t)(p % slots) * kLines + j) * 4];
      line[0] = tag32(p, 2 * j);
      line[1] = ll_flag(p);
      line[2] = tag32(p, 2 * j + 1);
      if (fault != 3) line[3] = ll_flag(p);
    } else {
      const int j = (pph - 1) / 2;
      const bool first = ((pph - 1) % 2) == 0;
      const bool is_flag = (fault == 6) ? first : !first;
      uint64_t* line = &ll128[((size_t)(p % slots) * kLines + j) * 16];
      if (is_flag) {
        if (fault != 5) line[15] = (uint64_t)p + 1;
      } else {
        for (int w = 0; w < 15; ++w) line[w] = tag32(p, 15 * j + w);
      }
    }
    if (++pph == producer_phases()) {
      pph = 0;
      ++p;
    }
    return true;
  };
  // Consumer micro-phases per step: 0 wait/poll, 1 read and check, 2 publish head.
  auto consumer_step = [&]() -> bool {
    if (cph == 0) {
      if (proto == ORC_PROTO_SIMPLE) {
        if (!(tail >= (uint64_t)c + 1)) return false;
      } else if (proto == ORC_PROTO_LL) {
        for (int j = 0; j < kLines; ++j) {
          const uint32_t* line = &ll[((size_t)(c % slots) * kLines + j) * 4];
          if (line[1] != ll_flag(c) || line[3] != ll_flag(c)) return false;
        }
      } else {
        for (int j = 0; j < kLines; ++j) {
          const uint64_t* line = &ll128[((size_t)(c % slots) * kLines + j) * 16];
          if (line[15] != (uint64_t)c + 1) return false;
        }
      }
    } else if (cph == 1) {
      bool ok = true;
      for (int j = 0; j < kLines; ++j) {
        if (proto == ORC_PROTO_SIMPLE) {
          ok = ok && simple[(size_t)(c % slots) * kLines + j] == tag32(c, j);
        } else if (proto == ORC_PROTO_LL) {
          const uint32_t* line = &ll[((size_t)(c % slots) * kLines + j) * 4];
          ok = ok && line[0] == tag32(c, 2 * j) && line[2] == tag32(c, 2 * j + 1);
        } else {
          const uint64_t* line = &ll128[((size_t)(c % slots) * kLines + j) * 16];
          for (int w = 0; w < 15; ++w) ok = ok && line[w] == tag32(c, 15 * j + w);
        }
      }
      if (!ok && first_bad < 0) first_bad = c;
    } else {
      if (fault != 1) head = (uint64_t)c + 1;
    }
    if (++cph == 3) {
      cph = 0;
      ++c;
    }
    return true;
  };
  int rc = ORC_OK;
  while (c < nsteps) {
    if (first_bad >= 0) {
      rc = ORC_CORRUPT;
      break;
    }
    if (consumer_step()) continue;
    if (p < nsteps && producer_step()) continue;
    rc = ORC_DEADLOCK;
    break;
  }
  if (rc == ORC_OK && first_bad >= 0) rc = ORC_CORRUPT;
  if (steps_done) *steps_done = p;
  if (consumed) *consumed = c;
  if (bad_step) *bad_step = first_bad;
  return rc;
}

int orc_ll_wrap(int flag_bits, int cleanup, int slots, int cap, int nsizes, const int* lines_of,
                int nsteps, int64_t* bad_step) {
  if ((flag_bits != 8 && flag_bits != 32) || slots < 1 || cap < 1 || nsizes < 1 || !lines_of ||
      nsteps < 1)
    return ORC_INVALID;
  const uint64_t period = 1ull << flag_bits, half = period / 2;
  if ((uint64_t)slots >= half) return ORC_INVALID;
  for (int i = 0; i < nsizes; ++i)
    if (lines_of[i] < 1 || lines_of[i] > cap) return ORC_INVALID;
  // line = {payload tag, flag}; both halves of an LL line carry the same flag
  struct Line {
    uint32_t tag = 0, flag = 0;
  };
  std::vector<Line> fifo((size_t)slots * cap);
  auto flag_of = [&](int64_t k) { return (uint32_t)(((uint64_t)k + 1) % period); };
  auto tag_of = [&](int64_t k, int j) { return tag32(k, j) | 1u; };  // never 0: zero lines are stale
  auto lines = [&](int64_t k) { return lines_of[k % nsizes]; };
  auto is_cleanup = [&](int64_t k) { return ((uint64_t)k + 1) % half >= half - (uint64_t)slots; };
  int64_t p = 0, c = 0;  // producer step, consumer step
  int pj = 0, cj = 0;    // next line to write / to take
  uint64_t head = 0;
  *bad_step = -1;
  while (c < nsteps) {
    // consumer first: take every line that looks ready
    bool moved = false;
    while (c < nsteps && cj < lines(c)) {
      const Line& l = fifo[(size_t)(c % slots) * cap + cj];
      if (l.flag != flag_of(c)) break;
      if (l.tag != tag_of(c, cj)) {
        *bad_step = c;
        return ORC_CORRUPT;
      }
      ++cj;
      moved = true;
    }
    if (c < nsteps && cj == lines(c)) {  // step consumed: hand the slot back
      ++c;
      cj = 0;
      head = (uint64_t)c;
      continue;
    }
    if (moved) continue;
    // producer: one line (or the whole cleanup tail) per turn
    if (p >= nsteps || head + (uint64_t)slots < (uint64_t)p + 1) return ORC_DEADLOCK;
    Line* slot = &fifo[(size_t)(p % slots) * cap];
    slot[pj].tag = tag_of(p, pj);
    slot[pj].flag = flag_of(p);
    if (++pj == lines(p)) {
      if (cleanup && is_cleanup(p))
        for (int j = lines(p); j < cap; ++j) slot[j] = Line{0, flag_of(p)};
      ++p;
      pj = 0;
    }
  }
  return ORC_OK;
}

}  // extern "C"
