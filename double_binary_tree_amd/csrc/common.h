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

// A contiguous element range evaluated with one order program ("variant"):
// for the ring, the rank whose block it is (the fold starts there); for the
// tree, the index of the node-level tree (0 or 1) of its channel.  A tile
// never straddles two variants.
struct Tile {
  uint64_t start;     // first element
  uint32_t nelem;     // elements in the tile
  uint32_t variant;
};
static_assert(sizeof(Tile) == 16, "tile layout");

// Fused tree program.  Inputs are consumed in the order perm[0..N); input j
// goes to register d = (instr >> 1) & 7: loaded if bit 0 is clear, folded
// in (R[d] = R[d] op x) if set; then (instr >> 4) cascaded register folds
// R[d-1] = R[d-1] op R[d], R[d-2] = R[d-2] op R[d-1], ...  The result ends
// in R[0].
struct TreeProgram {
  uint8_t perm[2][kMaxRanks];
  uint8_t instr[2][kMaxRanks];
  uint8_t pure_fold[2];       // 1: plain left fold (all inputs folded into R[0])
  uint8_t nregs[2];
};

struct FusedArgs {
  const void* send[kMaxRanks];
  void* recv[kMaxRanks];
  const Tile* tiles;
  uint32_t ntiles;
  uint32_t nranks;
  TreeProgram prog;
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
};

// Stepwise tree: one task = a run of consecutive slices of the message that
// all use one node-level tree.
struct TreeTask {
  uint64_t start;     // first element
  uint32_t nelem;     // elements covered
  uint32_t channel;   // a channel of the task's node-level tree
};
// Tree record of one rank in one channel, plus its distance from the root.
struct TreeNode {
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
  uint64_t count;             // elements per rank
  uint32_t ntasks;
  uint32_t nranks;
  uint32_t group;             // lanes per virtual rank
  uint32_t height;            // tree: max depth over the channel trees
};

}  // namespace emu
