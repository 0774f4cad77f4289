// Layouts shared by the host planner and the HIP kernels.  Plain structs,
// no HIP types, so the host planner also builds with a plain C++ compiler.
#pragma once

#include <cstdint>

#include "../../include/emu_comm.h"

namespace emu {

constexpr int kMaxRanks = EMU_MAX_RANKS;
constexpr int kMaxChannels = EMU_MAX_CHANNELS;
constexpr int kVecBytes = 16;        // one 128-bit access per lane
constexpr int kMaxRegs = 8;          // register stack of the fused tree program

enum class Algo : int { Ring = EMU_ALGO_RING, Tree = EMU_ALGO_TREE };
enum class DType : int { I32 = EMU_INT32, I64 = EMU_INT64, F32 = EMU_FLOAT32,
                         F16 = EMU_FLOAT16, BF16 = EMU_BFLOAT16 };
enum class Op : int { Sum = EMU_SUM, Max = EMU_MAX };

inline int elem_size(DType t) {
  switch (t) {
    case DType::I32: case DType::F32: return 4;
    case DType::I64: return 8;
    case DType::F16: case DType::BF16: return 2;
  }
  return 0;
}

// Collectives on the ring schedule: the all-reduce, and its two halves run
// standalone (reduce-scatter: rank r keeps the reduction of block r;
// all-gather: block k of every output is rank k's input).
enum Coll : int { kAllReduce = 0, kReduceScatter = 1, kAllGather = 2 };

// A contiguous element range evaluated with one order ("variant"): bits
// 0..7 the start k of the fold (rank-chunk index), bits 8..15 the row of the
// order table (FusedMode), bits 16..23 the block owner (reduce-scatter: the
// output rank; all-gather: the source rank).  A tile never straddles two
// variants.
struct Tile {
  uint64_t start;     // first element
  uint32_t nelem;     // elements in the tile
  uint32_t variant;
};
static_assert(sizeof(Tile) == 16, "tile layout");

// Fused modes.
//  kRotate:  input j is rank (k + j) mod N of the send-pointer array, which
//            the host passes already permuted into the one order every
//            channel shares; a plain left fold.
//  kFold:    input j is rank rows[row][k + j] & 0xFF; a plain left fold.
//  kProgram: input j is rank rows[row][j] & 0xFF, consumed by the register
//            program in bits 8..15 of the entry: it goes to register
//            d = (w >> 1) & 7, loaded if bit 0 of w is clear, folded in
//            (R[d] = R[d] op x) if set; then (w >> 4) cascaded register
//            folds R[d-1] = R[d-1] op R[d], R[d-2] = R[d-2] op R[d-1], ...
//            The result ends in R[0].
enum FusedMode : int { kRotate = 0, kFold = 1, kProgram = 2 };
constexpr int kRowLen = 2 * kMaxRanks;   // a ring row holds its order twice: k + j needs no wrap

struct FusedArgs {
  const void* send[kMaxRanks];
  void* recv[kMaxRanks];
  uint64_t block_bytes;       // reduce-scatter / all-gather: bytes per block
  uint32_t ntiles;
  uint32_t nranks;
  uint32_t xcd_runs;          // nonzero: each XCD takes a contiguous run of tiles
};

// Stepwise ring: one task = slice q of every rank-chunk of one ring loop.
struct RingLoopBlock {
  uint64_t offset;
  uint32_t nelem;
  uint32_t first_cell;   // offset / slice elements: the block's first slice-size cell
};
struct RingTask {
  uint32_t loop;      // index into the loop table (nranks blocks per loop)
  uint32_t slice;     // slice index inside each block
  uint32_t ring;      // the loop's ring order: row of the order table
  uint32_t nslices;   // tasks of the loop (slice = 0 .. nslices - 1)
};

// Stepwise tree: one task = a run of consecutive slices of the message that
// all use one tree (channels with identical records).
struct TreeTask {
  uint64_t start;     // first element
  uint32_t nelem;     // elements covered
  uint32_t channel;   // a channel of the task's tree
};
// Tree record of one rank in one channel, plus its distance from the root.
struct alignas(8) TreeNode {   // 8-byte aligned: one scalar load per record
  int8_t up;
  int8_t down[3];
  int8_t depth;
  int8_t pad[3];
};
static_assert(sizeof(TreeNode) == 8, "tree node layout");

struct StepArgs {
  const void* send[kMaxRanks];
  void* recv[kMaxRanks];
  const void* tasks;          // RingTask* or TreeTask*
  const void* table;          // RingLoopBlock* (ring) or TreeNode* (tree, [nch][nranks])
  const uint32_t* orders;     // ring: [rings][kMaxRanks], position p -> rank
  uint64_t count;             // elements per rank
  uint64_t block;             // reduce-scatter / all-gather: elements per block
  uint32_t ntasks;
  uint32_t nranks;
  uint32_t group;             // lanes per virtual rank
  uint32_t height;            // tree: max depth over the channel trees
};

}  // namespace emu
