// plan.h -- host planner of one ring AllReduce launch.
//
// Computes, on the host and before any launch: the ring position of every
// rank, the active channels, the channel split of the launch into
// (collective, channel) pieces, the encoding of those pieces into work
// batches, and the workgroup -> (rank, channel, lane) map of the grid.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "rar_device.h"

namespace rar {

struct RingInfo {
  std::vector<int> index, prev, next;
};

// Ring set-up [NCCL 专家课程 12, "Graph 如何变成完整 ring" and "ring index 如何
// 计算"]: ring_order lists user ranks along next.  Returns false (with a
// message) unless every rank appears exactly once and the walk loops back.
bool build_ring(int nranks, const int* ring_order, RingInfo* out, std::string* err);

// GRAPH lines of a ring layout [NCCL 专家课程 12, "Graph 如何变成完整 ring" (a
// channel's ring is recomputed from the connector graph) and "GRAPH 重建：N=2 /
// N=3 / N=4" (the lines)]: one line "Channel cc/CC : r0 r1 ..." per set bit c
// of mask, in increasing c, CC = highest set bit + 1; channel c runs ring
// c mod nrings of `orders` (nranks ints each), printed from rank 0 along next.
// Returns false (with a message) for a bad nranks, nrings, mask or ring.
bool graph_lines(int nranks, int nrings, const int* orders, uint64_t mask,
                 std::vector<std::string>* lines, std::string* err);

int64_t elem_size(int dtype);

// Largest chunk in elements [NCCL 专家课程 23, "Buffer 到 Chunk 的实测公式";
// LL and LL128 sections]: Simple = chunkSteps steps of buff/8 bytes; LL and
// LL128 = one step of payload (8 of every 16, 120 of every 128 bytes).
int64_t chunk_max_elems(int proto, size_t buff_size, int chunk_steps, int64_t es);

// Parameter checks shared by every entry point.
bool check_shape(int nranks, uint64_t mask, int proto, size_t buff_size, int chunk_steps,
                 std::string* err);

size_t default_buff_size(int proto);

struct Piece {
  int channel;     // dense index n
  int channel_id;  // n-th set bit of the mask
  int work;
  int64_t grid_offset, channel_count, chunk_count;
};

// Channel split of the launch: the collectives are laid end to end, each
// starting 16-byte aligned, and the element stream is cut into one
// contiguous 16-byte aligned range per active channel, in channel order.
std::vector<Piece> split_channels(uint64_t mask, int proto, size_t buff_size, int chunk_steps,
                                  int64_t es, const std::vector<size_t>& counts);

struct BatchPlan {
  std::vector<DevBatch> batches;       // batches[0] is an unused sentinel
  std::vector<DevWork> works;
  std::vector<uint32_t> first_batch;   // per channel id, 64 entries (0 = no work)
};

// Pack each channel's pieces, in order, into batches of at most kBatchWorks
// works (1024 bytes), chained by next_jump.  Every work runs on n_waves
// waves, or, with `sizing`, on the waves its per-call data fills (see
// work_waves).
struct WaveSizing {
  bool on = false;
  int nranks = 0;
  int proto = 0;
  int64_t es = 4;
  int split_lanes = 1;  // workgroups that split one call (1 when works are dealt)
};
BatchPlan encode_batches(const std::vector<Piece>& pieces, int n_channels, int n_waves,
                         const WaveSizing& sizing = WaveSizing());

// Waves for a piece: the bytes one workgroup moves per call of the piece
// (its first call's chunk, split over the workgroups of the channel) over
// the bytes a wave moves per pass, rounded up, within [1, n_waves].
int work_waves(const Piece& p, int n_waves, const WaveSizing& sizing);


// Workgroup map: the N ranks of one (channel, lane) pipeline are placed on
// the same XCD (workgroups are dispatched to the 8 XCDs round robin by
// blockIdx), so their FIFO traffic stays in one L2.  Idle slots pad the grid.
// With `spread`, the ranks of a pipeline go to different XCDs instead (each
// connector then crosses L2s; used to test that path).
std::vector<uint32_t> make_wg_map(int nranks, int n_channels, int n_lanes, bool spread = false);

// Bytes of one slot of one lane's FIFO.  A channel's step is split among its
// lanes in whole 16-byte vectors (Simple), 16-byte lines (LL) or 128-byte
// lines (LL128); every lane owns 8 such slots, so the lanes of a channel never
// touch each other's FIFO bytes.
int64_t lane_step_bytes(int proto, size_t buff_size, int lanes);

// Default lanes per channel: fill about one workgroup per CU.
int auto_lanes(int nranks, int n_channels, int cus);

}  // namespace rar
