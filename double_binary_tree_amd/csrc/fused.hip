// Fused all-reduce: one pass over HBM.  Each lane owns one 16-byte vector
// position of the message; it reads that position from every rank's send
// buffer once, evaluates the element in the schedule's own order, and writes
// the result to every rank's receive buffer.  2*N*S bytes in total, no LDS.
//
// Orders (see the oracle and the pages):
//  * ring: a rank-chunk k is folded x_k, x_{k+1}, ..., x_{k-1} (the block's
//    journey through the reduce-scatter steps of page "all-reduce 每张卡要发
//    多少数据? ring 和 tree 有什么区别?", Figure 1);
//  * tree: the expression of the channel's tree (reduce-up of page "NCCL
//    专家课程 13", section "runTreeSplit 如何流水"), compiled on the host into
//    a register program; a chain is a plain fold from the leaf up.
// Tiles never straddle two orders, so all control flow below is uniform
// (scalar) and only the element positions are per lane.
#include "device_ops.h"

namespace emu {

enum FusedMode : int { kRingFold = 0, kTreeFold = 1, kTreeProgram = 2 };

constexpr int kFusedThreads = 256;
constexpr int kBatch = 8;   // loads issued back to back before they are folded

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

// Input j of the order program: the rank whose buffer it comes from.
template <int MODE>
__device__ __forceinline__ uint32_t input_rank(const FusedArgs& a, uint32_t variant, uint32_t j) {
  if (MODE == kRingFold) {
    const uint32_t r = variant + j;
    return r >= a.nranks ? r - a.nranks : r;
  }
  return a.prog.perm[variant][j];
}

template <bool FULL>
__device__ __forceinline__ u32x4 load_input(const void* p, uint64_t boff, int nbytes) {
  return FULL ? ld_vec(p, boff) : ld_part(p, boff, nbytes);
}

// Fold inputs j .. j+B-1 into the accumulator / register stack.  The B loads
// are unconditional and issued back to back; the folds then consume them in
// order.
template <typename R, int MODE, bool FULL, int B>
__device__ __forceinline__ void fold_batch(const FusedArgs& a, uint32_t variant, uint32_t j, uint64_t boff,
                                           int nbytes, u32x4& acc, u32x4 (&g)[kMaxRegs]) {
  u32x4 x[B];
#pragma unroll
  for (int i = 0; i < B; ++i) x[i] = load_input<FULL>(a.send[input_rank<MODE>(a, variant, j + i)], boff, nbytes);
#pragma unroll
  for (int i = 0; i < B; ++i) {
    const u32x4 v = R::pre(x[i]);
    if (MODE == kTreeProgram) {
      const uint32_t w = a.prog.instr[variant][j + i];
      const int d = (w >> 1) & 7;
      reg_fold_in<R>(g, d, (w & 1) != 0, v);
      const int pops = (int)(w >> 4);
      for (int p = 1; p <= pops; ++p) reg_fold_down<R>(g, d - p);
    } else {
      acc = R::op(acc, v);
    }
  }
}

// Evaluate one vector position.  FULL: all 16 bytes valid; otherwise
// `nbytes` valid bytes (only the very last vector of the message).
template <typename R, int MODE, bool FULL>
__device__ __forceinline__ u32x4 evaluate(const FusedArgs& a, uint32_t variant, uint64_t boff,
                                          int nbytes) {
  const uint32_t n = a.nranks;
  u32x4 acc;
  u32x4 g[kMaxRegs];
  uint32_t j = 0;
  if (MODE == kTreeProgram) {
#pragma unroll
    for (int i = 0; i < kMaxRegs; ++i) g[i] = u32x4{0, 0, 0, 0};
    acc = u32x4{0, 0, 0, 0};
  } else {
    // the fold starts with its first input as is
    acc = R::pre(load_input<FULL>(a.send[input_rank<MODE>(a, variant, 0)], boff, nbytes));
    j = 1;
  }
  if (FULL) {
    for (; j + kBatch <= n; j += kBatch) fold_batch<R, MODE, FULL, kBatch>(a, variant, j, boff, nbytes, acc, g);
    if (j + 4 <= n) { fold_batch<R, MODE, FULL, 4>(a, variant, j, boff, nbytes, acc, g); j += 4; }
    if (j + 2 <= n) { fold_batch<R, MODE, FULL, 2>(a, variant, j, boff, nbytes, acc, g); j += 2; }
  }
  for (; j < n; ++j) fold_batch<R, MODE, FULL, 1>(a, variant, j, boff, nbytes, acc, g);
  if (MODE == kTreeProgram) acc = g[0];
  return R::post(acc);
}

// Write the result to every rank, stores issued in groups.
__device__ __forceinline__ void store_all(const FusedArgs& a, uint64_t boff, u32x4 v) {
  const uint32_t n = a.nranks;
  uint32_t r = 0;
  for (; r + kBatch <= n; r += kBatch) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) st_vec(a.recv[r + i], boff, v);
  }
  for (; r < n; ++r) st_vec(a.recv[r], boff, v);
}

template <typename R, int MODE, int ESZ>
__global__ __launch_bounds__(kFusedThreads) void fused_allreduce(const FusedArgs a) {
  constexpr int unit = kVecBytes / ESZ;
  for (uint32_t t = blockIdx.x; t < a.ntiles; t += gridDim.x) {
    const Tile tile = a.tiles[t];
    const uint32_t off = threadIdx.x * unit;
    if (off >= tile.nelem) continue;
    const uint32_t left = tile.nelem - off;
    const uint64_t boff = (tile.start + off) * ESZ;
    if (left >= (uint32_t)unit) {
      store_all(a, boff, evaluate<R, MODE, true>(a, tile.variant, boff, kVecBytes));
    } else {
      // The one partial vector at the end of the message: one rank at a
      // time, element-wise accesses.
      const int nbytes = (int)(left * ESZ);
      const u32x4 res = evaluate<R, MODE, false>(a, tile.variant, boff, nbytes);
      for (uint32_t r = 0; r < a.nranks; ++r) st_part(a.recv[r], boff, nbytes, res);
    }
  }
}

template <DType T, Op O, int MODE>
static hipError_t launch_one(const FusedArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((fused_allreduce<Red<T, O>, MODE, Unit<T>::esz>), dim3(grid), dim3(kFusedThreads),
                     0, stream, a);
  return hipGetLastError();
}

template <DType T, Op O>
static hipError_t launch_mode(int mode, const FusedArgs& a, int grid, hipStream_t stream) {
  switch (mode) {
    case kRingFold: return launch_one<T, O, kRingFold>(a, grid, stream);
    case kTreeFold: return launch_one<T, O, kTreeFold>(a, grid, stream);
    default: return launch_one<T, O, kTreeProgram>(a, grid, stream);
  }
}

template <DType T>
static hipError_t launch_op(Op op, int mode, const FusedArgs& a, int grid, hipStream_t stream) {
  return op == Op::Sum ? launch_mode<T, Op::Sum>(mode, a, grid, stream)
                       : launch_mode<T, Op::Max>(mode, a, grid, stream);
}

hipError_t launch_fused(DType t, Op op, int mode, const FusedArgs& a, int grid, hipStream_t stream) {
  switch (t) {
    case DType::I32: return launch_op<DType::I32>(op, mode, a, grid, stream);
    case DType::I64: return launch_op<DType::I64>(op, mode, a, grid, stream);
    case DType::F32: return launch_op<DType::F32>(op, mode, a, grid, stream);
    case DType::F16: return launch_op<DType::F16>(op, mode, a, grid, stream);
    case DType::BF16: return launch_op<DType::BF16>(op, mode, a, grid, stream);
  }
  return hipErrorInvalidValue;
}

int fused_threads() { return kFusedThreads; }

}  // namespace emu
