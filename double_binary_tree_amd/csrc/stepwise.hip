// Stepwise all-reduce: the ring steps and the tree hops executed one by one
// between virtual ranks, each a receive-reduce-copy through a step FIFO slot.
//
// One workgroup hosts every virtual rank of a slice of the message: rank r
// is a group of G lanes (G = 64, 32 or 16 so that N*G <= 1024), each lane
// owning one 16-byte vector of the slice.  A rank "sends" by writing its
// FIFO slot in LDS and the receiving rank reads it after the step barrier;
// slots are double-buffered by step parity, so a step's writes never meet
// the previous step's reads.  Only the ranks' own inputs and outputs touch
// HBM (2*N*S bytes, as for the fused pass); the partials that the pages move
// over links stay in LDS.
//
// Ring (page "all-reduce 每张卡要发多少数据? ring 和 tree 有什么区别?", Figure 1
// and section "手撕代码"; page "NCCL 内部机制：…", section "Ring：带宽友好…"):
//   step 0: rank r sends its block r;  steps 1..N-1: rank r receives block
//   (r-s) mod N, adds its own input, sends it on (the last of these writes
//   the finished block); then N-1 all-gather steps forward finished blocks.
// Tree (page "NCCL 专家课程 13", sections "runTreeSplit 如何流水" and "每种
// rank 的操作"): a rank at depth d reduces slice q at stage q + (H - d)
// (children's partials arrive from the previous stage) and, if not the root,
// broadcasts slice q at stage q + H + d; the root writes the result at its
// reduce stage.  Reduce-up and broadcast-down run concurrently on different
// slices, with separate slot sets, as the split thread groups of the pages do.
#include "device_ops.h"

namespace emu {

// LDS barrier for step hand-off: LDS writes are complete before the barrier;
// outstanding global loads (prefetches of the next step) stay in flight.
__device__ __forceinline__ void step_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// ---------------------------------------------------------------------------
// Ring.
template <typename R, int ESZ>
__global__ __launch_bounds__(1024) void step_ring(const StepArgs a) {
  constexpr int unit = kVecBytes / ESZ;
  extern __shared__ u32x4 fifo[];   // [2][N][G]
  const uint32_t n = a.nranks, g = a.group;
  const uint32_t r = threadIdx.x / g, p = threadIdx.x % g;
  const bool active = r < n;
  const uint32_t prev = active ? (r + n - 1) % n : 0;
  const RingLoopBlock* loops = static_cast<const RingLoopBlock*>(a.table);
  const RingTask* tasks = static_cast<const RingTask*>(a.tasks);
  auto slot = [&](uint32_t parity, uint32_t rank) -> u32x4& { return fifo[(parity * n + rank) * g + p]; };

  for (uint32_t t = blockIdx.x; t < a.ntasks; t += gridDim.x) {
    const RingTask task = tasks[t];
    const RingLoopBlock* blk = loops + (size_t)task.loop * n;
    const uint64_t in_block = ((uint64_t)task.slice * g + p) * unit;   // element offset inside a block
    // bytes of block b this lane owns (0 if the block is shorter)
    auto nbytes_of = [&](uint32_t b) -> int {
      const uint64_t len = blk[b].nelem;
      if (in_block >= len) return 0;
      const uint64_t left = len - in_block;
      return left >= (uint64_t)unit ? kVecBytes : (int)(left * ESZ);
    };
    auto boff_of = [&](uint32_t b) -> uint64_t { return (blk[b].offset + in_block) * ESZ; };

    if (n == 1) {
      const int nb = nbytes_of(0);
      if (active && nb) st_any(a.recv[0], boff_of(0), nb, ld_any(a.send[0], boff_of(0), nb));
      continue;
    }
    // step 0: send own block r
    u32x4 own = {0, 0, 0, 0};
    if (active) {
      const int nb = nbytes_of(r);
      if (nb) own = ld_any(a.send[r], boff_of(r), nb);
    }
    // prefetch the block of step 1
    u32x4 next = {0, 0, 0, 0};
    if (active) {
      const uint32_t b1 = (r + n - 1) % n;
      const int nb = nbytes_of(b1);
      if (nb) next = ld_any(a.send[r], boff_of(b1), nb);
    }
    if (active) slot(0, r) = R::pre(own);
    step_barrier();

    // reduce-scatter steps 1..N-1
    for (uint32_t s = 1; s < n; ++s) {
      const uint32_t b = (r + n - s) % n;
      u32x4 mine = next;
      if (active && s + 1 < n) {
        const uint32_t bn = (r + n - s - 1) % n;
        const int nb = nbytes_of(bn);
        if (nb) next = ld_any(a.send[r], boff_of(bn), nb);
      }
      if (active) {
        const u32x4 incoming = slot((s - 1) & 1, prev);
        const u32x4 res = R::op(R::pre(mine), incoming);
        if (s == n - 1) {
          const int nb = nbytes_of(b);
          if (nb) st_any(a.recv[r], boff_of(b), nb, R::post(res));
        }
        slot(s & 1, r) = res;
      }
      step_barrier();
    }
    // all-gather steps 1..N-1
    for (uint32_t j = 1; j < n; ++j) {
      const uint32_t b = (r + 1 + n - j) % n;
      if (active) {
        const u32x4 v = slot((n - 2 + j) & 1, prev);
        const int nb = nbytes_of(b);
        if (nb) st_any(a.recv[r], boff_of(b), nb, R::post(v));
        if (j + 1 < n) slot((n - 1 + j) & 1, r) = v;
      }
      step_barrier();
    }
  }
}

// ---------------------------------------------------------------------------
// Tree.
template <typename R, int ESZ>
__global__ __launch_bounds__(1024) void step_tree(const StepArgs a) {
  constexpr int unit = kVecBytes / ESZ;
  extern __shared__ u32x4 fifo[];   // up[2][N][G] then down[2][N][G]
  const uint32_t n = a.nranks, g = a.group;
  const uint32_t r = threadIdx.x / g, p = threadIdx.x % g;
  const bool active = r < n;
  const TreeTask* tasks = static_cast<const TreeTask*>(a.tasks);
  const TreeNode* nodes = static_cast<const TreeNode*>(a.table);
  const int H = (int)a.height;
  const uint32_t slice_elems = g * unit;
  auto up_slot = [&](int parity, uint32_t rank) -> u32x4& { return fifo[((uint32_t)parity * n + rank) * g + p]; };
  auto dn_slot = [&](int parity, uint32_t rank) -> u32x4& {
    return fifo[((2u + (uint32_t)parity) * n + rank) * g + p];
  };

  for (uint32_t t = blockIdx.x; t < a.ntasks; t += gridDim.x) {
    const TreeTask task = tasks[t];
    const TreeNode me = nodes[(size_t)task.channel * n + (active ? r : 0)];
    const int depth = me.depth;
    const bool is_root = me.up < 0;
    const bool has_children = me.down[0] >= 0;
    const int nslices = (int)((task.nelem + slice_elems - 1) / slice_elems);
    auto nbytes_of = [&](int q) -> int {
      const uint64_t off = (uint64_t)q * slice_elems + (uint64_t)p * unit;
      if (off >= task.nelem) return 0;
      const uint64_t left = task.nelem - off;
      return left >= (uint64_t)unit ? kVecBytes : (int)(left * ESZ);
    };
    auto boff_of = [&](int q) -> uint64_t {
      return (task.start + (uint64_t)q * slice_elems + (uint64_t)p * unit) * ESZ;
    };
    const int up_lag = H - depth;        // reduce slice q at stage q + up_lag
    const int dn_lag = H + depth;        // broadcast slice q at stage q + dn_lag
    const int nstages = nslices + 2 * H;

    // prefetch own input of the first reduce slice
    u32x4 next = {0, 0, 0, 0};
    if (active && nslices > 0) {
      const int nb = nbytes_of(0);
      if (nb) next = ld_any(a.send[r], boff_of(0), nb);
    }
    for (int st = 0; st < nstages; ++st) {
      const int cur = st & 1, prv = cur ^ 1;
      const int qu = st - up_lag;
      if (active && qu >= 0 && qu < nslices) {
        u32x4 acc = R::pre(next);
        if (qu + 1 < nslices) {
          const int nb = nbytes_of(qu + 1);
          if (nb) next = ld_any(a.send[r], boff_of(qu + 1), nb);
        }
#pragma unroll
        for (int s = 0; s < 3; ++s) {
          const int c = me.down[s];
          if (c >= 0) acc = R::op(acc, up_slot(prv, (uint32_t)c));
        }
        if (is_root) {
          const int nb = nbytes_of(qu);
          if (nb) st_any(a.recv[r], boff_of(qu), nb, R::post(acc));
          if (has_children) dn_slot(cur, r) = acc;
        } else {
          up_slot(cur, r) = acc;
        }
      }
      const int qd = st - dn_lag;
      if (active && !is_root && qd >= 0 && qd < nslices) {
        const u32x4 v = dn_slot(prv, (uint32_t)me.up);
        const int nb = nbytes_of(qd);
        if (nb) st_any(a.recv[r], boff_of(qd), nb, R::post(v));
        if (has_children) dn_slot(cur, r) = v;
      }
      step_barrier();
    }
  }
}

template <DType T, Op O>
static hipError_t launch_ring_t(const StepArgs& a, int grid, int block, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((step_ring<Red<T, O>, Unit<T>::esz>), dim3(grid), dim3(block), lds, s, a);
  return hipGetLastError();
}
template <DType T, Op O>
static hipError_t launch_tree_t(const StepArgs& a, int grid, int block, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((step_tree<Red<T, O>, Unit<T>::esz>), dim3(grid), dim3(block), lds, s, a);
  return hipGetLastError();
}

template <DType T>
static hipError_t launch_step_t(bool ring, Op op, const StepArgs& a, int grid, int block, size_t lds,
                                hipStream_t s) {
  if (ring)
    return op == Op::Sum ? launch_ring_t<T, Op::Sum>(a, grid, block, lds, s)
                         : launch_ring_t<T, Op::Max>(a, grid, block, lds, s);
  return op == Op::Sum ? launch_tree_t<T, Op::Sum>(a, grid, block, lds, s)
                       : launch_tree_t<T, Op::Max>(a, grid, block, lds, s);
}

hipError_t launch_stepwise(bool ring, DType t, Op op, const StepArgs& a, int grid, int block,
                           size_t lds, hipStream_t s) {
  switch (t) {
    case DType::I32: return launch_step_t<DType::I32>(ring, op, a, grid, block, lds, s);
    case DType::I64: return launch_step_t<DType::I64>(ring, op, a, grid, block, lds, s);
    case DType::F32: return launch_step_t<DType::F32>(ring, op, a, grid, block, lds, s);
    case DType::F16: return launch_step_t<DType::F16>(ring, op, a, grid, block, lds, s);
    case DType::BF16: return launch_step_t<DType::BF16>(ring, op, a, grid, block, lds, s);
  }
  return hipErrorInvalidValue;
}

// Resident workgroups per CU for the stepwise kernels at this block/LDS size.
int stepwise_occupancy(bool ring, DType t, Op op, int block, size_t lds) {
  int blocks = 0;
  hipError_t e = hipErrorInvalidValue;
#define EMU_OCC(T_)                                                                                 \
  if (t == T_) {                                                                                    \
    if (ring)                                                                                       \
      e = op == Op::Sum                                                                             \
              ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, step_ring<Red<T_, Op::Sum>, Unit<T_>::esz>, block, lds) \
              : hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, step_ring<Red<T_, Op::Max>, Unit<T_>::esz>, block, lds); \
    else                                                                                            \
      e = op == Op::Sum                                                                             \
              ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, step_tree<Red<T_, Op::Sum>, Unit<T_>::esz>, block, lds) \
              : hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, step_tree<Red<T_, Op::Max>, Unit<T_>::esz>, block, lds); \
  }
  EMU_OCC(DType::I32)
  EMU_OCC(DType::I64)
  EMU_OCC(DType::F32)
  EMU_OCC(DType::F16)
  EMU_OCC(DType::BF16)
#undef EMU_OCC
  return e == hipSuccess && blocks > 0 ? blocks : 1;
}

}  // namespace emu
