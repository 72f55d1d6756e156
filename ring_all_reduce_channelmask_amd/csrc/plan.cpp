// plan.cpp -- host planner (see plan.h).
#include "plan.h"

#include <algorithm>
#include <cstdio>

namespace rar {
namespace {

int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align_up(int64_t a, int64_t b) { return div_up(a, b) * b; }

}  // namespace

bool build_ring(int nranks, const int* ring_order, RingInfo* out, std::string* err) {
  if (nranks < 2 || nranks > kMaxRanks) {
    *err = "nranks must be in [2, 64]";
    return false;
  }
  if (!ring_order) {
    *err = "ring_order is NULL";
    return false;
  }
  std::vector<int> next(nranks, -1), count(nranks, 0);
  for (int i = 0; i < nranks; ++i) {
    const int r = ring_order[i];
    if (r < 0 || r >= nranks) {
      *err = "ring_order holds a rank outside [0, nranks)";
      return false;
    }
    if (count[r]++) {
      *err = "ring_order lists a rank twice";
      return false;
    }
  }
  for (int i = 0; i < nranks; ++i) next[ring_order[i]] = ring_order[(i + 1) % nranks];
  // walk the ring N times from rank 0: it must visit all ranks and loop back
  std::vector<int> seen(nranks, 0);
  int cur = 0;
  for (int i = 0; i < nranks; ++i) {
    seen[cur] = 1;
    cur = next[cur];
  }
  if (cur != 0 || std::count(seen.begin(), seen.end(), 1) != nranks) {
    *err = "ring does not loop back";
    return false;
  }
  out->index.assign(nranks, 0);
  out->prev.assign(nranks, 0);
  out->next = next;
  // ring index: number of hops from rank 0 along next
  int r = 0;
  for (int hops = 0; hops < nranks; ++hops) {
    out->index[r] = hops;
    out->prev[next[r]] = r;
    r = next[r];
  }
  return true;
}

int64_t elem_size(int dtype) { return dtype == 2 ? 2 : 4; }

int64_t chunk_max_elems(int proto, size_t buff_size, int chunk_steps, int64_t es) {
  const int64_t step = (int64_t)buff_size / kSteps;
  switch (proto) {
    case kSimple:
      return step / es * chunk_steps;
    case kLL:
      return step / 2 / es;
    default:
      return step / 128 * 120 / es;
  }
}

size_t default_buff_size(int proto) {
  switch (proto) {
    case kSimple:
      return 4u << 20;
    case kLL:
      return 512u << 10;
    default:
      return 4915200u;  // 640 threads x 120 words x 8 bytes x 8 steps -> 576000-byte chunks
  }
}

bool check_shape(int nranks, uint64_t mask, int proto, size_t buff_size, int chunk_steps,
                 std::string* err) {
  if (nranks < 2 || nranks > kMaxRanks) {
    *err = "nranks must be in [2, 64]";
    return false;
  }
  if (mask == 0) {
    *err = "channel_mask is empty";
    return false;
  }
  if (proto != kSimple && proto != kLL && proto != kLL128) {
    *err = "unknown protocol";
    return false;
  }
  // Simple: slices are rounded up to 16 elements, so a step must hold a
  // multiple of 16 elements of every dtype (64-byte steps).  LL: a step's
  // payload is a multiple of 16 bytes.  LL128: an even number of lines per
  // step, so that a 576000-style chunk stays 16-byte aligned.
  const size_t quantum = proto == kSimple ? 512 : proto == kLL ? 256 : 2048;
  if (buff_size == 0 || buff_size % quantum != 0) {
    *err = "buff_size must be a positive multiple of " + std::to_string(quantum) +
           " for this protocol";
    return false;
  }
  if (buff_size > (size_t(1) << 31)) {
    *err = "buff_size above 2 GiB";
    return false;
  }
  if (proto == kSimple && chunk_steps != 2 && chunk_steps != 4) {
    *err = "chunk_steps must be 2 or 4 (a chunk of all 8 slots deadlocks the ring)";
    return false;
  }
  return true;
}

std::vector<Piece> split_channels(uint64_t mask, int proto, size_t buff_size, int chunk_steps,
                                  int64_t es, const std::vector<size_t>& counts) {
  const int64_t vec = 16 / es;
  std::vector<int> ids;
  for (int b = 0; b < kMaxChannels; ++b)
    if ((mask >> b) & 1ull) ids.push_back(b);
  const int64_t nch = (int64_t)ids.size();
  std::vector<int64_t> first(counts.size());
  int64_t end = 0;
  for (size_t w = 0; w < counts.size(); ++w) {
    first[w] = align_up(end, vec);
    end = first[w] + (int64_t)counts[w];
  }
  std::vector<Piece> pieces;
  if (end == 0 || nch == 0) return pieces;
  const int64_t cmax = chunk_max_elems(proto, buff_size, chunk_steps, es);
  const int64_t span = align_up(div_up(end, nch), vec);
  for (int64_t n = 0; n < nch; ++n) {
    const int64_t lo = n * span, hi = std::min(end, lo + span);
    for (size_t w = 0; w < counts.size(); ++w) {
      const int64_t a = std::max(lo, first[w]);
      const int64_t b = std::min(hi, first[w] + (int64_t)counts[w]);
      if (b <= a) continue;
      pieces.push_back(Piece{(int)n, ids[n], (int)w, a - first[w], b - a, cmax});
    }
  }
  return pieces;
}

int work_waves(const Piece& p, int n_waves, const WaveSizing& sz) {
  if (!sz.on) return n_waves;
  // the chunk of the piece's first call: the protocol maximum, or the tail
  // loop's re-chunked size when the piece is shorter than one loop
  const int64_t vec = 16 / sz.es;
  const int64_t loop = (int64_t)sz.nranks * p.chunk_count;
  const int64_t cc = p.channel_count < loop ? align_up(div_up(p.channel_count, sz.nranks), vec) : p.chunk_count;
  const int64_t bytes = div_up(cc * sz.es, sz.split_lanes);
  // bytes one wave moves per pass: Simple 64 lanes x 16 bytes x the vectors
  // reduceCopy keeps in flight (16 for 4-byte payloads, 4 for bf16); LL 64
  // lanes x 4 lines x 8 payload bytes; LL128 groups of 8 lines x 120 bytes,
  // 4 groups per pass for 4-byte payloads and 3 for bf16
  const int64_t simple_pass = sz.es == 2 ? 4096 : 16384;
  const int64_t ll128_pass = 960 * (sz.es == 2 ? 3 : 4);
  const int64_t pass = sz.proto == kSimple ? simple_pass : sz.proto == kLL ? 2048 : ll128_pass;
  return (int)std::max<int64_t>(1, std::min<int64_t>(n_waves, div_up(bytes, pass)));
}

BatchPlan encode_batches(const std::vector<Piece>& pieces, int n_channels, int n_waves,
                         const WaveSizing& sizing) {
  BatchPlan plan;
  plan.batches.push_back(DevBatch{0, 0, 0});  // sentinel: next_jump 0 means "no next"
  plan.first_batch.assign(kMaxChannels, 0);
  for (int n = 0; n < n_channels; ++n) {
    std::vector<const Piece*> mine;
    for (const Piece& p : pieces)
      if (p.channel == n) mine.push_back(&p);
    if (mine.empty()) continue;
    const int channel_id = mine.front()->channel_id;
    uint32_t prev_batch = 0;
    for (size_t k = 0; k < mine.size(); k += kBatchWorks) {
      const size_t cnt = std::min<size_t>(kBatchWorks, mine.size() - k);
      DevBatch b;
      b.next_jump = 0;
      b.offset_base = (uint32_t)plan.works.size();
      b.offset_bitset = cnt == 64 ? ~0ull : ((1ull << cnt) - 1);
      for (size_t i = 0; i < cnt; ++i) {
        const Piece& p = *mine[k + i];
        DevWork w{};
        w.grid_offset = p.grid_offset;
        w.channel_count = p.channel_count;
        w.chunk_count = p.chunk_count;
        w.buf_index = (uint32_t)p.work;
        w.n_waves = (uint16_t)work_waves(p, n_waves, sizing);
        plan.works.push_back(w);
      }
      const uint32_t idx = (uint32_t)plan.batches.size();
      plan.batches.push_back(b);
      if (prev_batch)
        plan.batches[prev_batch].next_jump = idx;
      else
        plan.first_batch[channel_id] = idx;
      prev_batch = idx;
    }
  }
  return plan;
}

std::vector<uint32_t> make_wg_map(int nranks, int n_channels, int n_lanes, bool spread) {
  constexpr int kXcds = 8;
  const int pipes = n_channels * n_lanes;
  if (!spread) {
    std::vector<uint32_t> map(wg_grid_size(nranks, pipes));
    for (size_t g = 0; g < map.size(); ++g) map[g] = wg_entry((uint32_t)g, nranks, n_lanes, pipes);
    return map;
  }
  std::vector<std::vector<uint32_t>> per_xcd(kXcds);
  for (int q = 0; q < pipes; ++q) {
    const int n = q / n_lanes, lane = q % n_lanes;
    for (int r = 0; r < nranks; ++r)
      per_xcd[(q + r) % kXcds].push_back((uint32_t)r | ((uint32_t)n << 8) |
                                                         ((uint32_t)lane << 16));
  }
  size_t depth = 0;
  for (auto& v : per_xcd) depth = std::max(depth, v.size());
  std::vector<uint32_t> map(depth * kXcds, kIdleWg);
  for (int x = 0; x < kXcds; ++x)
    for (size_t k = 0; k < per_xcd[x].size(); ++k) map[k * kXcds + x] = per_xcd[x][k];
  return map;
}

bool graph_lines(int nranks, int nrings, const int* orders, uint64_t mask,
                 std::vector<std::string>* lines, std::string* err) {
  if (nrings < 1 || nrings > kMaxChannels) {
    *err = "nrings must be in [1, 64]";
    return false;
  }
  if (!orders) {
    *err = "ring_orders is NULL";
    return false;
  }
  if (mask == 0) {
    *err = "channel mask selects no channel";
    return false;
  }
  std::vector<RingInfo> rings(nrings);
  for (int k = 0; k < nrings; ++k)
    if (!build_ring(nranks, orders + (size_t)k * nranks, &rings[k], err)) return false;
  const int space = 64 - __builtin_clzll(mask);
  lines->clear();
  for (int c = 0; c < 64; ++c) {
    if (!((mask >> c) & 1)) continue;
    const RingInfo& ring = rings[c % nrings];
    char head[32];
    snprintf(head, sizeof head, "Channel %02d/%02d :", c, space);
    std::string line = head;
    int cur = 0;
    for (int i = 0; i < nranks; ++i) {
      line += " " + std::to_string(cur);
      cur = ring.next[cur];
    }
    lines->push_back(line);
  }
  return true;
}

int64_t lane_step_bytes(int proto, size_t buff_size, int lanes) {
  // LL128 lanes take an even number of 128-byte lines; Simple lanes take
  // whole 128-byte cache lines of every slice, so a lane's slot steps are
  // cache-line multiples too
  const int64_t unit = proto == kLL128 ? 256 : proto == kSimple ? 128 : 16;
  const int64_t step_units = div_up((int64_t)buff_size / kSteps, unit);
  return unit * div_up(step_units, lanes);
}

int auto_lanes(int nranks, int n_channels, int cus) {
  // as many lanes as keep every workgroup on its own CU (measured on MI355X:
  // 5 lanes x 12 channels x 4 ranks = 240 workgroups beats 4 lanes = 192)
  return std::max(1, std::min(cus / (nranks * n_channels), kMaxLanes));
}

}  // namespace rar
