// Fused collectives: one pass over HBM.  All-reduce: each lane owns one
// 16-byte vector position of the message; it reads that position from every
// rank's send buffer once, evaluates the element in the schedule's own
// order, and writes the result to every rank's receive buffer (2*N*S bytes
// in total, no LDS).  Reduce-scatter evaluates the same way but writes only
// the owner of the block; all-gather copies one input to every output.
//
// Orders (see the oracle and the pages):
//  * ring: rank-chunk k of a channel whose ring visits ranks o_0, o_1, ...
//    is folded x_{o_k}, x_{o_{k+1}}, ..., x_{o_{k-1}} (the block's journey
//    through the reduce-scatter steps of page "all-reduce 每张卡要发多少数据?
//    ring 和 tree 有什么区别?", Figure 1);
//  * tree: the expression of the channel's tree (reduce-up of page "NCCL
//    专家课程 13", section "runTreeSplit 如何流水"), compiled on the host into
//    a register program; a chain is a plain fold from the leaf up.
// The three ways to name the order are the FusedMode values: a rotation of
// host-permuted pointers when every channel shares one order, else rows of
// a small order table.  Tiles never straddle two orders, so all control
// flow below is uniform (scalar) and only the element positions are per lane.
#include "device_ops.h"

namespace emu {

// Lanes per tile (a tile is one vector per lane of every rank: 2 KiB per
// rank).  Measured on MI355X against 256 and 512 lanes (3 alternating
// rounds): 8 ranks f32 1.4-2.5% faster than 256 from 16 to 256 MiB per
// rank, 16 and 32 ranks within 0.3%; 512 lanes won only at 16 MiB per rank
// and lost 1-2% elsewhere.
#ifndef EMU_FUSED_THREADS
#define EMU_FUSED_THREADS 128
#endif
constexpr int kFusedThreads = EMU_FUSED_THREADS;
#ifndef EMU_FUSED_VPT
#define EMU_FUSED_VPT 1
#endif
constexpr int kVpt = EMU_FUSED_VPT;      // vectors per lane in a full tile
constexpr uint32_t kXcds = 8;            // accelerator complex dies of the chip
// Ranks whose loads a lane issues back to back before the first fold, a
// launch-time choice: 8 up to 8 ranks, 16 above.  With 16, the ranks past
// the last whole batch are folded in one more phase (fold_rest).  Measured
// on MI355X (3 alternating rounds): 16 at 16 and 32 ranks ran 0.4-2.5%
// faster on the 16- and 32-rank workloads than 8 (f32 max within 0.3%), 32
// was 1-4% slower on the tree programs; at 15 ranks one phase of 15 loads
// ran 3.1% faster than phases of 8, 4, 2 and 1 (tree, 32 MiB bf16; ring
// 1.5%).  Up to 8 ranks the batch of 8 keeps the kernel at 44-48 VGPRs.
constexpr int kBatchSmall = 8, kBatchLarge = 16;

// The register stack is indexed with the (wave-uniform) level of the
// program; the compiler keeps it in VGPRs and indexes it relatively.
template <typename R>
__device__ __forceinline__ void reg_fold_in(u32x4 (&g)[kMaxRegs], int d, bool fold, u32x4 x) {
  g[d] = fold ? R::op(g[d], x) : x;
}

template <typename R>
__device__ __forceinline__ void reg_fold_down(u32x4 (&g)[kMaxRegs], int d) {
  g[d] = R::op(g[d], g[d + 1]);
}

// Entry j of the order: the rank whose buffer input j comes from (bits
// 0..7) and, for kProgram, its register instruction (bits 8..15).
template <int MODE>
__device__ __forceinline__ uint32_t order_entry(const FusedArgs& a, const uint32_t* __restrict__ rows,
                                                uint32_t variant, uint32_t j) {
  if (MODE == kRotate) {
    const uint32_t r = (variant & 0xFF) + j;
    return r >= a.nranks ? r - a.nranks : r;
  }
  return rows[((variant >> 8) & 0xFF) * kRowLen + (variant & 0xFF) + j];
}

// Register stack size: the program mode's stack; the fold modes need none.
template <int MODE>
constexpr int stack_regs() { return MODE == kProgram ? kMaxRegs : 1; }

template <typename R, int MODE, int V>
__device__ __forceinline__ void consume(uint32_t entry, uint32_t j, const u32x4 (&x)[V],
                                        u32x4 (&acc)[V], u32x4 (&g)[stack_regs<MODE>()]) {
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const u32x4 val = R::pre(x[v]);
    if constexpr (MODE == kProgram) {
      const uint32_t w = entry >> 8;
      const int d = (w >> 1) & 7;
      static_assert(MODE != kProgram || V == 1, "program mode evaluates one position at a time");
      reg_fold_in<R>(g, d, (w & 1) != 0, val);
      const int pops = (int)(w >> 4);
      for (int p = 1; p <= pops; ++p) reg_fold_down<R>(g, d - p);
    } else {
      acc[v] = j == 0 ? val : R::op(acc[v], val);
    }
  }
}

// Fold inputs j .. j+B-1 at V whole-vector positions (byte offsets boff +
// v*stride).  The B*V loads are unconditional and issued back to back.
template <typename R, int MODE, int V, int B>
__device__ __forceinline__ void fold_batch(const FusedArgs& a, const uint32_t* __restrict__ rows, uint32_t variant,
                                           uint32_t j, uint64_t boff, uint32_t stride, u32x4 (&acc)[V],
                                           u32x4 (&g)[stack_regs<MODE>()]) {
  uint32_t e[B];
  const void* src[B];
#pragma unroll
  for (int i = 0; i < B; ++i) e[i] = order_entry<MODE>(a, rows, variant, j + i);
#pragma unroll
  for (int i = 0; i < B; ++i) src[i] = a.send[e[i] & 0xFF];
  u32x4 x[B][V];
#pragma unroll
  for (int i = 0; i < B; ++i)
#pragma unroll
    for (int v = 0; v < V; ++v) x[i][v] = ld_vec(src[i], boff + (uint64_t)v * stride);
  // Keep every load of the batch ahead of the first fold.
#ifndef EMU_SCHED_BARRIER
#define EMU_SCHED_BARRIER 1
#endif
#if EMU_SCHED_BARRIER
  __builtin_amdgcn_sched_barrier(0);
#endif
#pragma unroll
  for (int i = 0; i < B; ++i) consume<R, MODE, V>(e[i], j + i, x[i], acc, g);
}

// Fold the last r (1 <= r < B) inputs j .. j+r-1 in one phase: B loads
// issued back to back before the first fold, of which entries r .. B-1 pass
// an out-of-range offset to a raw buffer view (the hardware returns zeros
// without a memory access) and are not folded.  So a rank count that is not
// a multiple of the batch costs one memory round trip more, not one per
// power of two in its remainder; and no load sits under a branch (the
// merges would copy every loaded register).  The views are based at the
// first active lane's offset (uniform); every lane's offset lies at or
// above it, within the tile.
template <typename R, int MODE, int V, int B>
__device__ __forceinline__ void fold_rest(const FusedArgs& a, const uint32_t* __restrict__ rows, uint32_t variant,
                                          uint32_t j, uint32_t r, uint64_t boff, uint32_t stride, u32x4 (&acc)[V],
                                          u32x4 (&g)[stack_regs<MODE>()]) {
  const uint64_t wbase = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(boff >> 32)) << 32) |
                         (uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)boff);
  const uint32_t loff = (uint32_t)(boff - wbase);
  uint32_t e[B];
  u32x4 x[B][V];
#pragma unroll
  for (int i = 0; i < B; ++i) {
    const bool live = (uint32_t)i < r;
    e[i] = order_entry<MODE>(a, rows, variant, j + (live ? (uint32_t)i : 0u));
    const auto rs = buffer_view(static_cast<const char*>(a.send[e[i] & 0xFF]) + wbase);
#pragma unroll
    for (int v = 0; v < V; ++v) x[i][v] = ld_buf(rs, live ? loff + (uint32_t)v * stride : kNoLoad);
  }
#if EMU_SCHED_BARRIER
  __builtin_amdgcn_sched_barrier(0);
#endif
#pragma unroll
  for (int i = 0; i < B; ++i)
    if ((uint32_t)i < r) consume<R, MODE, V>(e[i], j + i, x[i], acc, g);
}

// Evaluate V whole-vector positions.
template <typename R, int MODE, int V, int B>
__device__ __forceinline__ void evaluate(const FusedArgs& a, const uint32_t* __restrict__ rows, uint32_t variant,
                                         uint64_t boff, uint32_t stride, u32x4 (&out)[V]) {
  const uint32_t n = a.nranks;
  u32x4 acc[V];
  u32x4 g[stack_regs<MODE>()];
#pragma unroll
  for (int i = 0; i < stack_regs<MODE>(); ++i) g[i] = u32x4{0, 0, 0, 0};
  uint32_t j = 0;
  static_assert(B == kBatchSmall || B == kBatchLarge, "the load batch is 8 or 16");
  for (; j + B <= n; j += B) fold_batch<R, MODE, V, B>(a, rows, variant, j, boff, stride, acc, g);
  if constexpr (B == kBatchLarge) {
    if (j < n) fold_rest<R, MODE, V, B>(a, rows, variant, j, n - j, boff, stride, acc, g);
  } else {
    // Up to 8 ranks the remainder (below 8 ranks only) is folded 4, 2 and 1
    // inputs at a time: the one-phase remainder shifted the 8-rank kernel's
    // code and measured 0.8% slower there.
    for (; j + 4 <= n; j += 4) fold_batch<R, MODE, V, 4>(a, rows, variant, j, boff, stride, acc, g);
    if (j + 2 <= n) { fold_batch<R, MODE, V, 2>(a, rows, variant, j, boff, stride, acc, g); j += 2; }
    if (j < n) fold_batch<R, MODE, V, 1>(a, rows, variant, j, boff, stride, acc, g);
  }
#pragma unroll
  for (int v = 0; v < V; ++v) out[v] = R::post(MODE == kProgram ? g[0] : acc[v]);
}

// The one partial vector at the end of the message: `nbytes` valid bytes,
// one rank at a time, 16-bit accesses.  Reduce-scatter writes only the
// block owner's output, `shift` bytes lower; all-gather copies from the
// block owner's input, `shift` bytes lower.
template <typename R, int MODE, int COLL>
__device__ __forceinline__ void partial_vector(const FusedArgs& a, const uint32_t* __restrict__ rows,
                                               uint32_t variant, uint64_t boff, int nbytes) {
  const uint32_t owner = variant >> 16;
  const uint64_t shift = COLL == kAllReduce ? 0 : (uint64_t)owner * a.block_bytes;
  u32x4 res;
  if constexpr (COLL == kAllGather) {
    res = ld_part(a.send[owner], boff - shift, nbytes);
  } else {
    u32x4 acc[1];
    u32x4 g[stack_regs<MODE>()];
#pragma unroll
    for (int i = 0; i < stack_regs<MODE>(); ++i) g[i] = u32x4{0, 0, 0, 0};
    for (uint32_t j = 0; j < a.nranks; ++j) {
      const uint32_t e = order_entry<MODE>(a, rows, variant, j);
      const u32x4 x[1] = {ld_part(a.send[e & 0xFF], boff, nbytes)};
      consume<R, MODE, 1>(e, j, x, acc, g);
    }
    res = R::post(MODE == kProgram ? g[0] : acc[0]);
  }
  if constexpr (COLL == kReduceScatter) {
    st_part(a.recv[owner], boff - shift, nbytes, res);
  } else {
    for (uint32_t r = 0; r < a.nranks; ++r) st_part(a.recv[r], boff, nbytes, res);
  }
}

// Write V results to every rank.
template <int V>
__device__ __forceinline__ void store_all(const FusedArgs& a, uint64_t boff, uint32_t stride, const u32x4 (&res)[V]) {
  const uint32_t n = a.nranks;
  uint32_t r = 0;
  for (; r < n; ++r)
#pragma unroll
    for (int v = 0; v < V; ++v) st_vec(a.recv[r], boff + (uint64_t)v * stride, res[v]);
}

// V whole-vector positions (byte offsets boff + v*stride) of one tile: the
// all-reduce folds every rank's input there and writes every rank's output;
// reduce-scatter folds the same way and writes only the block owner's
// output, one block lower; all-gather copies the block owner's input (one
// block lower) to every rank's output.
template <typename R, int MODE, int COLL, int V, int B>
__device__ __forceinline__ void do_positions(const FusedArgs& a, const uint32_t* __restrict__ rows,
                                             uint32_t variant, uint64_t boff, uint32_t stride) {
  const uint32_t owner = variant >> 16;
  const uint64_t shift = COLL == kAllReduce ? 0 : (uint64_t)owner * a.block_bytes;
  if constexpr (COLL == kAllGather) {
    u32x4 x[V];
#pragma unroll
    for (int v = 0; v < V; ++v) x[v] = ld_vec(a.send[owner], boff - shift + (uint64_t)v * stride);
    store_all<V>(a, boff, stride, x);
  } else {
    u32x4 res[V];
    evaluate<R, MODE, V, B>(a, rows, variant, boff, stride, res);
    if constexpr (COLL == kReduceScatter) {
#pragma unroll
      for (int v = 0; v < V; ++v) st_vec(a.recv[owner], boff - shift + (uint64_t)v * stride, res[v]);
    } else {
      store_all<V>(a, boff, stride, res);
    }
  }
}

// A tile holds kFusedThreads * kVpt vectors; lane l owns vectors l,
// l + kFusedThreads, ... (each group of 64 lanes touches 1 KiB contiguous
// per rank).  Tiles
// are laid on the input positions (all-reduce, reduce-scatter) or the
// output positions (all-gather): the side with N accesses per position.
// The tile table and the order rows come as their own read-only arguments
// so that the (uniform) loads from them go through the scalar unit.
template <typename R, int MODE, int ESZ, int COLL, int B>
__global__ __launch_bounds__(kFusedThreads) void fused_collective(const FusedArgs a, const Tile* __restrict__ tiles,
                                                                  const uint32_t* __restrict__ rows) {
  constexpr uint32_t unit = kVecBytes / ESZ;
  constexpr uint32_t stride = kFusedThreads * kVecBytes;   // bytes between a lane's vectors
  // Workgroups are dealt to the chip's 8 XCDs in turn.  With xcd_runs each
  // XCD takes a contiguous run of tiles instead of every eighth one, so the
  // workgroups running at once spread over 8 distant parts of the buffers.
  uint32_t vb = blockIdx.x;
  if (a.xcd_runs && gridDim.x % kXcds == 0) vb = (blockIdx.x % kXcds) * (gridDim.x / kXcds) + blockIdx.x / kXcds;
  for (uint32_t t = vb; t < a.ntiles; t += gridDim.x) {
    const Tile tile = tiles[t];
    const uint64_t base = tile.start * ESZ;
    const uint32_t lane_off = threadIdx.x * kVecBytes;
    if (tile.nelem == kFusedThreads * kVpt * unit) {
      if constexpr (MODE == kProgram) {
        // The register stack is indexed dynamically; one position at a time
        // keeps it in VGPRs.
        for (int v = 0; v < kVpt; ++v)
          do_positions<R, MODE, COLL, 1, B>(a, rows, tile.variant, base + lane_off + (uint64_t)v * stride, 0);
      } else {
        do_positions<R, MODE, COLL, kVpt, B>(a, rows, tile.variant, base + lane_off, stride);
      }
      continue;
    }
    // A short tile (next to a segment boundary): vector by vector, each lane
    // keeping its position in the aligned tile-size cell, so that the wave
    // still touches whole cache lines; lanes outside the tile sit out.
    const uint64_t cell = tile.start / (kFusedThreads * kVpt * unit) * (kFusedThreads * kVpt * unit);
    const uint64_t end = tile.start + tile.nelem;
    for (int v = 0; v < kVpt; ++v) {
      const uint64_t pos = cell + (uint64_t)(threadIdx.x + v * kFusedThreads) * unit;
      if (pos < tile.start || pos >= end) continue;
      const uint64_t boff = pos * ESZ;
      if (end - pos >= unit)
        do_positions<R, MODE, COLL, 1, B>(a, rows, tile.variant, boff, 0);
      else
        partial_vector<R, MODE, COLL>(a, rows, tile.variant, boff, (int)((end - pos) * ESZ));
    }
  }
}

template <DType T, Op O, int MODE, int COLL, int B = kBatchSmall>
static hipError_t launch_b(const FusedArgs& a, const Tile* tiles, const uint32_t* rows, int grid,
                           hipStream_t stream) {
  hipLaunchKernelGGL((fused_collective<Red<T, O>, MODE, Unit<T>::esz, COLL, B>), dim3(grid), dim3(kFusedThreads),
                     0, stream, a, tiles, rows);
  return hipGetLastError();
}

// The load batch by rank count (the all-gather is a copy: one load per lane).
template <DType T, Op O, int MODE, int COLL>
static hipError_t launch_one(const FusedArgs& a, const Tile* tiles, const uint32_t* rows, int grid,
                             hipStream_t stream) {
  if constexpr (COLL != kAllGather) {
    if (a.nranks > kBatchSmall) return launch_b<T, O, MODE, COLL, kBatchLarge>(a, tiles, rows, grid, stream);
  }
  return launch_b<T, O, MODE, COLL>(a, tiles, rows, grid, stream);
}

template <DType T, Op O>
static hipError_t launch_mode(Coll coll, int mode, const FusedArgs& a, const Tile* tiles, const uint32_t* rows,
                              int grid, hipStream_t stream) {
  if (coll == kReduceScatter)   // ring orders only: no register programs
    return mode == kRotate ? launch_one<T, O, kRotate, kReduceScatter>(a, tiles, rows, grid, stream)
                           : launch_one<T, O, kFold, kReduceScatter>(a, tiles, rows, grid, stream);
  switch (mode) {
    case kRotate: return launch_one<T, O, kRotate, kAllReduce>(a, tiles, rows, grid, stream);
    case kFold: return launch_one<T, O, kFold, kAllReduce>(a, tiles, rows, grid, stream);
    default: return launch_one<T, O, kProgram, kAllReduce>(a, tiles, rows, grid, stream);
  }
}

template <DType T>
static hipError_t launch_op(Coll coll, Op op, int mode, const FusedArgs& a, const Tile* tiles, const uint32_t* rows,
                            int grid, hipStream_t stream) {
  return op == Op::Sum ? launch_mode<T, Op::Sum>(coll, mode, a, tiles, rows, grid, stream)
                       : launch_mode<T, Op::Max>(coll, mode, a, tiles, rows, grid, stream);
}

hipError_t launch_fused(Coll coll, DType t, Op op, int mode, const FusedArgs& a, const Tile* tiles,
                        const uint32_t* rows, int grid, hipStream_t stream) {
  if (coll == kAllGather) {
    // a copy: only the element size matters
    switch (elem_size(t)) {
      case 2: return launch_one<DType::F16, Op::Sum, kRotate, kAllGather>(a, tiles, rows, grid, stream);
      case 4: return launch_one<DType::I32, Op::Sum, kRotate, kAllGather>(a, tiles, rows, grid, stream);
      case 8: return launch_one<DType::I64, Op::Sum, kRotate, kAllGather>(a, tiles, rows, grid, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (t) {
    case DType::I32: return launch_op<DType::I32>(coll, op, mode, a, tiles, rows, grid, stream);
    case DType::I64: return launch_op<DType::I64>(coll, op, mode, a, tiles, rows, grid, stream);
    case DType::F32: return launch_op<DType::F32>(coll, op, mode, a, tiles, rows, grid, stream);
    case DType::F16: return launch_op<DType::F16>(coll, op, mode, a, tiles, rows, grid, stream);
    case DType::BF16: return launch_op<DType::BF16>(coll, op, mode, a, tiles, rows, grid, stream);
  }
  return hipErrorInvalidValue;
}

int fused_tile_vectors() { return kFusedThreads * kVpt; }

}  // namespace emu
