// Host planner: how one all-reduce message is split over channels, chunks,
// ring loops and rank-chunks, and the order programs the kernels run.
#pragma once

#include <cstdint>
#include <vector>

#include "common.h"
#include "topology.h"

namespace emu {

struct Range {
  uint64_t offset;
  uint64_t count;
};

// Channel ranges: ceil(count/unit) units dealt over nch channels, the first
// (units % nch) channels one unit more; offsets clipped to count.
std::vector<Range> channel_ranges(uint64_t count, uint64_t unit, int nch);
// Chunks of at most chunk_count elements inside one channel range.
std::vector<Range> tree_chunks(const Range& ch, uint64_t chunk_count);
// Ring loops of nranks*chunk_count elements inside one channel range, each
// cut into nranks rank-chunks (block k is the one whose fold starts at k).
std::vector<std::vector<Range>> ring_loops(const Range& ch, int nranks, uint64_t chunk_count,
                                           uint64_t unit);

// Fused mode: tiles of at most tile_elems elements, each inside one variant
// segment (ring: one rank-chunk; tree: one node-level tree).
void build_fused_tiles(const Topology& topo, Algo algo, uint64_t count, uint64_t unit,
                       uint64_t chunk_count, uint64_t tile_elems, std::vector<Tile>* out);

// Fused tree program for one channel tree (see TreeProgram in common.h).
// Returns EMU_SUCCESS or EMU_ERR_INTERNAL (register stack too deep, or the
// self-check of the program against the fold definition failed).
int compile_tree_program(const ChannelTopology& ch, uint8_t perm[kMaxRanks],
                         uint8_t instr[kMaxRanks], int* nregs, bool* pure_fold);

// Stepwise ring: loop table (nranks blocks per loop) and tasks (loop, slice).
void build_ring_tasks(const Topology& topo, uint64_t count, uint64_t unit, uint64_t chunk_count,
                      uint64_t slice_elems, std::vector<RingLoopBlock>* loops,
                      std::vector<RingTask>* tasks);

// Stepwise tree: about target_tasks contiguous pieces of the message, each
// inside one run of channels that share a node-level tree and cut at
// slice-cell boundaries, and the per-(channel, rank) tree table.
void build_tree_tasks(const Topology& topo, uint64_t count, uint64_t unit, uint64_t slice_elems,
                      uint64_t target_tasks, std::vector<TreeTask>* tasks,
                      std::vector<TreeNode>* nodes);

}  // namespace emu
