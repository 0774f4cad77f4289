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

// Fused tree program for one channel tree (the kProgram encoding of
// common.h: input order perm, per-input register instruction instr).
// Returns EMU_SUCCESS or EMU_ERR_INTERNAL (register stack too deep, or the
// self-check of the program against the fold definition failed).
int compile_tree_program(const ChannelTopology& ch, uint8_t perm[kMaxRanks],
                         uint8_t instr[kMaxRanks], int* nregs, bool* pure_fold);

// Fused orders of a communicator: the mode, the order rows, the pointer
// permutation of kRotate, and each channel's variant base (the tile variant
// of ring block k in channel c is base[c] + k; of a tree tile, base[c]).
struct FusedOrders {
  int mode = kRotate;
  std::vector<uint32_t> rows;               // [nrows][kRowLen]
  uint8_t rotate_perm[kMaxRanks] = {};      // kRotate: pointer j is rank rotate_perm[j]
  std::vector<uint32_t> base;               // per channel
};
int build_fused_orders(const Topology& topo, Algo algo, FusedOrders* out);

// Fused mode: tiles of at most tile_elems elements, each inside one variant
// segment (ring: one rank-chunk of one ring order; tree: one tree).
void build_fused_tiles(const Topology& topo, Algo algo, const FusedOrders& orders, uint64_t count,
                       uint64_t unit, uint64_t chunk_count, uint64_t tile_elems, std::vector<Tile>* out);

// Reduce-scatter / all-gather, fused: tiles over the input positions
// (reduce-scatter: block r of every input, folded in channel c's ring order
// from the position after r's) or the output positions (all-gather: block k
// of every output, copied from rank k).  `block` elements per block.
void build_fused_coll_tiles(const Topology& topo, Coll coll, const FusedOrders& ring_orders, uint64_t block,
                            uint64_t unit, uint64_t tile_elems, std::vector<Tile>* out);

// Reduce-scatter / all-gather, stepwise: per channel range of a block and
// chunk, one loop of nranks step-schedule blocks; step block k is data block
// order[k-1] (so that position p finishes, or starts from, its own rank's
// block).  Loop table, tasks and ring orders as for build_ring_tasks.
void build_ring_coll_tasks(const Topology& topo, uint64_t block, uint64_t unit, uint64_t chunk_count,
                           uint64_t slice_elems, std::vector<RingLoopBlock>* loops, std::vector<RingTask>* tasks,
                           std::vector<uint32_t>* orders);

// Stepwise ring: loop table (nranks blocks per loop), tasks (loop, slice,
// ring order) and the ring order table ([nrings][kMaxRanks]).
void build_ring_tasks(const Topology& topo, uint64_t count, uint64_t unit, uint64_t chunk_count,
                      uint64_t slice_elems, std::vector<RingLoopBlock>* loops,
                      std::vector<RingTask>* tasks, std::vector<uint32_t>* orders);

// Stepwise ring across workgroups: per channel, the range [first, end) of
// its loops in build_ring_tasks' loop table ([nch][2]).
std::vector<uint32_t> ring_channel_loops(const Topology& topo, uint64_t count, uint64_t unit, uint64_t chunk_count);

// Stepwise tree: about target_tasks contiguous pieces of the message, each
// inside one run of channels with the same tree records and cut at
// slice-cell boundaries, and the per-(channel, rank) tree table.  Pieces
// hold at least min_cells slice cells where the segments allow (fewer,
// longer pieces).
void build_tree_tasks(const Topology& topo, uint64_t count, uint64_t unit, uint64_t slice_elems,
                      uint64_t target_tasks, std::vector<TreeTask>* tasks,
                      std::vector<TreeNode>* nodes, uint64_t min_cells = 1);

}  // namespace emu
