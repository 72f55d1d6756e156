/*
 * tsan_check.cpp -- TEST INFRASTRUCTURE ONLY: a driver that runs the
 * oracle's channel-parallel mode (sched 2) on small collectives and checks
 * that it gives the bytes of the sequential round-robin mode (sched 0).
 * The CPU test suite builds it with -fsanitize=thread and runs it, so that a
 * data race between the channel threads fails the test.  Exit status 0 when
 * every case matches, 1 otherwise.
 */
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "ring_sim.h"

static int run_case(int nranks, uint64_t mask, int proto, size_t buff, int dtype, size_t count,
                    int nworks, int options, int threads, unsigned seed) {
  const size_t es = dtype == ORC_BFLOAT16 ? 2 : 4;
  std::mt19937 rng(seed);
  std::vector<int> order(nranks);
  for (int r = 0; r < nranks; ++r) order[r] = r;
  std::shuffle(order.begin() + 1, order.end(), rng);
  std::vector<size_t> counts(nworks);
  std::vector<std::vector<uint8_t>> in((size_t)nworks * nranks), out_a(in.size()), out_b(in.size());
  std::vector<const void*> sp(in.size());
  std::vector<void*> ra(in.size()), rb(in.size());
  for (int w = 0; w < nworks; ++w) {
    counts[w] = count + (size_t)w * 37;
    for (int r = 0; r < nranks; ++r) {
      const size_t i = (size_t)w * nranks + r;
      in[i].resize(counts[w] * es);
      for (size_t b = 0; b < in[i].size(); b += 2) {
        // small integer-valued payloads of every type (bf16 / fp32 / int32)
        const int v = (int)(rng() % 17) - 8;
        if (dtype == ORC_BFLOAT16) {
          const float f = (float)v;
          uint32_t u;
          std::memcpy(&u, &f, 4);
          const uint16_t h = (uint16_t)(u >> 16);
          std::memcpy(&in[i][b], &h, 2);
        } else if (b % 4 == 0) {
          const float f = (float)v;
          if (dtype == ORC_FLOAT32) std::memcpy(&in[i][b], &f, 4);
          else std::memcpy(&in[i][b], &v, 4);
        }
      }
      out_a[i].assign(in[i].size(), 0);
      out_b[i].assign(in[i].size(), 0xAB);
      sp[i] = in[i].data();
      ra[i] = out_a[i].data();
      rb[i] = out_b[i].data();
    }
  }
  orc_stats sa, sb;
  const int ca = orc_allreduce(nranks, order.data(), mask, proto, buff, 4, dtype, nworks, counts.data(),
                               sp.data(), ra.data(), 8, 0, 0, options, &sa, nullptr, 0);
  const int cb = orc_allreduce(nranks, order.data(), mask, proto, buff, 4, dtype, nworks, counts.data(),
                               sp.data(), rb.data(), 8, 2, (uint64_t)threads, options, &sb, nullptr, 0);
  if (ca != ORC_OK || cb != ORC_OK) {
    std::printf("case N=%d mask=%llx proto=%d: rc %d / %d\n", nranks, (unsigned long long)mask, proto, ca, cb);
    return 1;
  }
  for (size_t i = 0; i < in.size(); ++i)
    if (out_a[i] != out_b[i]) {
      std::printf("case N=%d mask=%llx proto=%d: outputs differ\n", nranks, (unsigned long long)mask, proto);
      return 1;
    }
  if (sa.units_run != sb.units_run || std::memcmp(sa.wire_sent, sb.wire_sent, sizeof(sa.wire_sent)) != 0) {
    std::printf("case N=%d mask=%llx proto=%d: statistics differ\n", nranks, (unsigned long long)mask, proto);
    return 1;
  }
  return 0;
}

int main() {
  int bad = 0;
  unsigned seed = 1;
  // protocol, buffer: Simple, LL, LL128 at small buffers so that chunks loop
  const int protos[3] = {ORC_PROTO_SIMPLE, ORC_PROTO_LL, ORC_PROTO_LL128};
  const size_t buffs[3] = {8 * 1024, 8 * 512, 8 * 2048};
  for (int p = 0; p < 3; ++p)
    for (int dtype = 0; dtype < 3; ++dtype) {
      bad |= run_case(4, 0xFFF, protos[p], buffs[p], dtype, 9001, 1, 0, 4, seed++);
      bad |= run_case(3, 0b101101010011, protos[p], buffs[p], dtype, 3001, 5, 0, 3, seed++);
      bad |= run_case(8, 0xF0F, protos[p], buffs[p], dtype, 4097, 2, 0, 8, seed++);
    }
  // direct variants and an operator other than the sum
  bad |= run_case(4, 0xFF, ORC_PROTO_SIMPLE, 8 * 1024, ORC_FLOAT32, 7777, 2, ORC_OPT_DIRECT | ORC_OPT_DIRECT_READ, 4, seed++);
  bad |= run_case(5, 0x3F, ORC_PROTO_LL, 8 * 512, ORC_INT32, 3333, 1, ORC_RED_MAX << ORC_OPT_RED_SHIFT, 6, seed++);
  std::printf(bad ? "MISMATCH\n" : "OK\n");
  return bad;
}
