// Stepwise all-reduce with the LL (low-latency) protocol: the same ring
// steps and tree hops as stepwise.hip, but a virtual rank hands a step's
// data to the next one through flag-in-line FIFO lines instead of a slot
// plus a workgroup barrier.
//
// Protocol (page "NCCL 内部机制：…", section "LL：用更高的元数据比例换低延迟"):
// a FIFO line carries half data and half flag.  Here every 8-byte word is
// {4 data bytes, 4 flag bytes} and is written and read as one 8-byte LDS
// access (single-copy atomic for aligned 8-byte LDS words), so a reader that
// sees the flag it expects also sees the data written with it: no fence and
// no separate ready notice.  A lane's 16-byte vector travels as four such
// words.  The flag of a FIFO's k-th item is k + 1 (k counted from the call's
// start on the ring, from the task's start on the tree), so a reader never
// takes a stale line for a new one.  A FIFO has
// kLLSlots slots; the writer of item k waits until the reader has consumed
// item k - kLLSlots (the reader publishes how many it consumed), so no slot
// is overwritten before it is read.
//
// One wave is one virtual rank (64 lanes, one vector each), so N <= 16.
// Waves never meet at a workgroup barrier inside a task: each waits only for
// the lines it reads and the slots it writes.  Every rank runs its steps in
// the order of the stepwise schedule and every wait is for an item produced
// (or consumed) at an earlier step of that schedule, so the waits cannot
// form a cycle; every wait is nevertheless bounded (spin_limit polls, 2^22
// unless the host lowers it), and on expiry the workgroup abandons the call
// and records it in *status.  A wave that abandons stops working but still
// meets every workgroup barrier (the tree's task boundaries), so the
// workgroup always ends together.
//
// The pages split a tree CTA's threads 70/30 between reduce and broadcast
// for LL (section "runTreeSplit 如何流水").  A rank here is one wave, whose
// lanes execute together, so the split has no counterpart; the reduce-up
// and broadcast-down streams still progress independently through separate
// FIFOs.
#include <algorithm>

#include "device_ops.h"

namespace emu {

// Whether a poll that failed yields the SIMD for a moment (s_sleep) before
// the next one.
#ifndef EMU_LL_SLEEP
#define EMU_LL_SLEEP 1
#endif

constexpr uint32_t kLLSlots = 2;            // FIFO depth (>= 2: see the tree's stage argument)
constexpr uint32_t kLLWords = 4;            // 8-byte words per lane per item (one 16-byte vector)
constexpr uint32_t kG = 64;                 // lanes per rank

// One rank's FIFO in LDS: [kLLSlots][kLLWords][kG] words.
constexpr uint32_t kFifoWords = kLLSlots * kLLWords * kG;

__device__ __forceinline__ uint64_t lds_load64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ uint32_t lds_acquire32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_release32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Per-workgroup protocol state in LDS after the FIFOs: the abandon flag.
struct LLCtl {
  uint32_t* abandon;     // set once any wave's wait expired
  uint32_t* status;      // device word the host reads (emu_protocol_status)
  uint32_t spin_limit;   // polls before a wait is abandoned
};

// Poll until every lane's `ready()` holds.  Returns false if the wait
// expired or another wave abandoned the call (then the caller returns).
template <typename Ready>
__device__ __forceinline__ bool ll_wait(const LLCtl& ctl, Ready ready) {
  for (uint32_t it = 0;; ++it) {
    if (__all(ready())) return true;
    if (it >= ctl.spin_limit || lds_acquire32(ctl.abandon)) {
      lds_release32(ctl.abandon, 1u);
      __hip_atomic_store(ctl.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    if (EMU_LL_SLEEP) __builtin_amdgcn_s_sleep(1);
  }
}

// Write item `k` (counted from 0) of `fifo`: four words {data, flag k + 1}.
// The caller has made sure that the slot's previous item was consumed.
__device__ __forceinline__ void ll_write(uint64_t* fifo, uint32_t k, uint32_t p, const u32x4& x) {
  uint64_t* line = fifo + (k % kLLSlots) * kLLWords * kG + p;
  const uint64_t flag = (uint64_t)(k + 1) << 32;
  lds_store64(line + 0 * kG, flag | x.x);
  lds_store64(line + 1 * kG, flag | x.y);
  lds_store64(line + 2 * kG, flag | x.z);
  lds_store64(line + 3 * kG, flag | x.w);
}
// Write item k of a FIFO with one reader, after that reader has consumed
// item k - kLLSlots (`*consumed` >= k + 1 - kLLSlots).
__device__ __forceinline__ bool ll_send(const LLCtl& ctl, uint64_t* fifo, const uint32_t* consumed, uint32_t k,
                                        uint32_t p, const u32x4& x) {
  if (k >= kLLSlots && !ll_wait(ctl, [&] { return lds_acquire32(consumed) >= k + 1 - kLLSlots; })) return false;
  ll_write(fifo, k, p, x);
  return true;
}

// Read item `k` of `fifo` into x once all four of its words carry flag k + 1,
// then publish k + 1 as consumed (one lane, after every lane's read).
__device__ __forceinline__ bool ll_recv(const LLCtl& ctl, const uint64_t* fifo, uint32_t* consumed, uint32_t k,
                                        uint32_t p, u32x4& x) {
  const uint64_t* line = fifo + (k % kLLSlots) * kLLWords * kG + p;
  const uint32_t flag = k + 1;
  uint64_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
  const bool ok = ll_wait(ctl, [&] {
    w0 = lds_load64(line + 0 * kG);
    w1 = lds_load64(line + 1 * kG);
    w2 = lds_load64(line + 2 * kG);
    w3 = lds_load64(line + 3 * kG);
    return (uint32_t)(w0 >> 32) == flag && (uint32_t)(w1 >> 32) == flag && (uint32_t)(w2 >> 32) == flag &&
           (uint32_t)(w3 >> 32) == flag;
  });
  if (!ok) return false;
  x = u32x4{(uint32_t)w0, (uint32_t)w1, (uint32_t)w2, (uint32_t)w3};
  if (p == 0) lds_release32(consumed, flag);   // release: every lane's reads above come first
  return true;
}

// ---------------------------------------------------------------------------
// Ring.  Position r sends to r+1 through FIFO r; its k-th item of the call
// is consumed by r+1 as that rank's k-th receive (the ring's sends and
// receives pair up in order, task after task), so the counters run across
// tasks.  Steps of one task as in step_ring: step 0 sends block r; steps
// 1..N-1 receive block r-s, add the own input, send it on (the last writes
// the finished block); then N-1 all-gather steps forward finished blocks.
template <typename R, int ESZ>
__global__ __launch_bounds__(1024) void ll_ring(const StepArgs a, const RingTask* __restrict__ tasks,
                                                 const RingLoopBlock* __restrict__ loops,
                                                 const uint32_t* __restrict__ orders, uint32_t* status,
                                                 uint32_t spin_limit) {
  constexpr int unit = kVecBytes / ESZ;
  extern __shared__ uint64_t lds_words[];   // fifo [N][kFifoWords], consumed [N], abandon
  const uint32_t n = a.nranks;
  const uint32_t r = __builtin_amdgcn_readfirstlane(threadIdx.x / kG);   // ring position
  const uint32_t p = threadIdx.x % kG;
  const uint32_t prev = (r + n - 1) % n;
  uint64_t* const fifo = lds_words;
  uint32_t* const consumed = reinterpret_cast<uint32_t*>(lds_words + (size_t)n * kFifoWords);
  const LLCtl ctl{consumed + n, status, spin_limit};
  for (uint32_t e = threadIdx.x; e < n * kFifoWords; e += blockDim.x) fifo[e] = 0;
  if (threadIdx.x <= n) consumed[threadIdx.x] = 0;   // and the abandon flag
  __syncthreads();

  uint64_t* const my_fifo = fifo + (size_t)r * kFifoWords;
  const uint64_t* const in_fifo = fifo + (size_t)prev * kFifoWords;
  const uint64_t slice_elems = (uint64_t)kG * unit;
  uint32_t nsent = 0, nrecv = 0;
  for (uint32_t t = blockIdx.x; t < a.ntasks; t += gridDim.x) {
    const RingTask task = tasks[t];
    const uint32_t me = __builtin_amdgcn_readfirstlane(orders[(size_t)task.ring * kMaxRanks + r]);
    // block b of this task: its cell and [start, end) range (scalar loads)
    struct View { uint64_t cell, pos, start, end; };
    auto view_of = [&](uint32_t b) -> View {
      const RingLoopBlock d = loops[(size_t)task.loop * n + b];
      const uint64_t cell = ((uint64_t)d.first_cell + task.slice) * slice_elems;
      return {cell, cell + (uint64_t)p * unit, d.offset, d.offset + d.nelem};
    };
    auto nbytes_of = [&](const View& w) -> int {
      if (w.pos < w.start || w.pos >= w.end) return 0;
      const uint64_t left = w.end - w.pos;
      return left >= (uint64_t)unit ? kVecBytes : (int)(left * ESZ);
    };
    // Own input of block b: the whole vectors through a raw buffer view,
    // unconditionally (kNoLoad for a lane without one, or for every lane
    // when `live` is false), and a partial vector, only ever at a block's
    // end, by load_part once the value is needed.  Every step then refills
    // the same registers: a load under a condition would leave two values
    // to merge, and the merge copy would wait for the load before the step
    // could wait for its item.
    auto cell_of = [&](const View& w) { return static_cast<const char*>(a.send[me]) + w.cell * ESZ; };
    auto load = [&](uint32_t b, bool live) -> u32x4 {
      const View w = view_of(b);
      return ld_buf(buffer_view(cell_of(w)), live && nbytes_of(w) == kVecBytes ? p * kVecBytes : kNoLoad);
    };
    auto load_part = [&](uint32_t b, u32x4& x) {
      const View w = view_of(b);
      const int nb = nbytes_of(w);
      if (nb > 0 && nb < kVecBytes) x = ld_part(cell_of(w), p * kVecBytes, nb);
    };
    auto store = [&](uint32_t b, const u32x4& x) {
      const View w = view_of(b);
      if (w.start <= w.cell && w.cell + slice_elems <= w.end) {   // whole cell: no lane is out of range
        st_vec(a.recv[me], w.pos * ESZ, R::post(x));
        return;
      }
      const int nb = nbytes_of(w);
      if (nb) st_any(a.recv[me], w.pos * ESZ, nb, R::post(x));
    };
    auto send = [&](const u32x4& x) { return ll_send(ctl, my_fifo, &consumed[r], nsent++, p, x); };
    auto recv = [&](u32x4& x) { return ll_recv(ctl, in_fifo, &consumed[prev], nrecv++, p, x); };

    u32x4 own = load(r, true);
    load_part(r, own);
    if (n == 1) {   // one rank: no steps (and no FIFO traffic)
      store(0, R::pre(own));
      continue;
    }
    if (!send(R::pre(own))) return;
    // blocks counted down instead of taken modulo N: step s works on block
    // (r - s) mod N, all-gather step j on (r + 1 - j) mod N
    uint32_t b = r == 0 ? n - 1 : r - 1;
    own = load(b, true);   // step 1's own input, read while waiting
    for (uint32_t s = 1; s < n; ++s) {
      u32x4 y;
      if (!recv(y)) return;
      load_part(b, own);
      const u32x4 res = R::op(R::pre(own), y);
      const uint32_t bn = b == 0 ? n - 1 : b - 1;   // block of step s + 1
      own = load(bn, s + 1 < n);   // the next step's own input (none after the last)
      if (s == n - 1) store(b, res);
      if (!send(res)) return;
      b = bn;
    }
    uint32_t bg = r;
    for (uint32_t j = 1; j < n; ++j) {
      u32x4 x;
      if (!recv(x)) return;
      store(bg, x);
      bg = bg == 0 ? n - 1 : bg - 1;
      if (j + 1 < n && !send(x)) return;
    }
  }
}

// ---------------------------------------------------------------------------
// Tree.  Rank r writes its partial of each reduce slice to FIFO up[r] (read
// by its parent) and the result of each broadcast slice to FIFO down[r]
// (read by each of its children, each publishing its own consumed count);
// the stage of every operation is the stepwise tree's (reduce slice q at
// stage q + H - depth, broadcast at q + H + depth), and a rank runs its
// operations in stage order.  An item of up[c] written at stage s is read at
// stage s + 1, so with two slots the writer's wait is for a read at stage
// s - 1: earlier than its own, as every other wait.  The relations change
// with the channel's tree, so FIFOs and counters restart at every task
// (between two workgroup barriers).
template <typename R, int ESZ>
__global__ __launch_bounds__(1024) void ll_tree(const StepArgs a, const TreeTask* __restrict__ tasks,
                                                 const TreeNode* __restrict__ nodes, uint32_t* status,
                                                 uint32_t spin_limit) {
  constexpr int unit = kVecBytes / ESZ;
  // LDS: up FIFOs [N][kFifoWords], down FIFOs [N][kFifoWords], consumed-up
  // [N], consumed-down [N][3], abandon
  extern __shared__ uint64_t lds_words[];
  const uint32_t n = a.nranks;
  const uint32_t r = __builtin_amdgcn_readfirstlane(threadIdx.x / kG);
  const uint32_t p = threadIdx.x % kG;
  uint64_t* const up_fifo = lds_words;
  uint64_t* const dn_fifo = lds_words + (size_t)n * kFifoWords;
  uint32_t* const up_used = reinterpret_cast<uint32_t*>(lds_words + 2 * (size_t)n * kFifoWords);
  uint32_t* const dn_used = up_used + n;   // [N][3]: child slot j of rank i reads down[i]
  const LLCtl ctl{dn_used + 3 * n, status, spin_limit};
  if (threadIdx.x == 0) *ctl.abandon = 0;
  const int H = (int)a.height;
  const uint32_t slice_elems = kG * unit;

  for (uint32_t t = blockIdx.x; t < a.ntasks; t += gridDim.x) {
    // restart: every rank clears its own FIFOs and counters
    for (uint32_t e = p; e < kFifoWords; e += kG) {
      up_fifo[(size_t)r * kFifoWords + e] = 0;
      dn_fifo[(size_t)r * kFifoWords + e] = 0;
    }
    if (p == 0) up_used[r] = 0;
    if (p < 3) dn_used[3 * r + p] = 0;
    __syncthreads();
    if (lds_acquire32(ctl.abandon)) return;   // the whole workgroup, after the barrier

    const TreeTask task = tasks[t];
    const TreeNode rec = nodes[task.channel * n + r];
    const int up = rec.up, depth = rec.depth;
    const int down[3] = {rec.down[0], rec.down[1], rec.down[2]};
    const bool is_root = up < 0;
    const bool has_children = down[0] >= 0;
    // this rank's child slot in its parent's record
    int my_slot = 0;
    if (!is_root) {
      const TreeNode pr = nodes[task.channel * n + up];
      my_slot = pr.down[0] == (int)r ? 0 : pr.down[1] == (int)r ? 1 : 2;
    }
    const uint64_t first_cell = task.start / slice_elems;
    const uint64_t end = task.start + task.nelem;
    const int nslices = (int)((end + slice_elems - 1) / slice_elems - first_cell);
    auto pos_of = [&](int q) { return (first_cell + (uint64_t)q) * slice_elems + (uint64_t)p * unit; };
    auto nbytes_of = [&](int q) -> int {
      const uint64_t pos = pos_of(q);
      if (pos < task.start || pos >= end) return 0;
      const uint64_t left = end - pos;
      return left >= (uint64_t)unit ? kVecBytes : (int)(left * ESZ);
    };
    auto load = [&](int q) -> u32x4 {
      const char* const cell = static_cast<const char*>(a.send[r]) + (first_cell + (uint64_t)q) * slice_elems * ESZ;
      return ld_lane(cell, p * kVecBytes, nbytes_of(q));
    };
    auto store = [&](int q, const u32x4& x) {
      if (q > 0 && q + 1 < nslices) {   // inside the task: every lane holds a whole vector
        st_vec(a.recv[r], pos_of(q) * ESZ, R::post(x));
        return;
      }
      const int nb = nbytes_of(q);
      if (nb) st_any(a.recv[r], pos_of(q) * ESZ, nb, R::post(x));
    };
    // counters of this task: items written to up[r] and down[r], read from
    // each child's up FIFO and from the parent's down FIFO.  A write to
    // down[r] waits for the slowest of the children.
    uint32_t nup = 0, ndn = 0, nrecv_dn = 0;
    uint32_t nrecv_up[3] = {0, 0, 0};
    auto send_down = [&](const u32x4& x) -> bool {
      const uint32_t k = ndn++;
      if (k >= kLLSlots) {
        const bool ok = ll_wait(ctl, [&] {
          bool ready = true;
          for (int j = 0; j < 3; ++j)
            if (down[j] >= 0) ready = ready && lds_acquire32(&dn_used[3 * r + j]) >= k + 1 - kLLSlots;
          return ready;
        });
        if (!ok) return false;
      }
      ll_write(dn_fifo + (size_t)r * kFifoWords, k, p, x);
      return true;
    };
    const int up_lag = H - depth, dn_lag = H + depth;
    const int nstages = nslices + 2 * H;
    u32x4 own = {0, 0, 0, 0};   // the next reduce slice's own input, once loaded
    bool have_own = false;
    bool ok = true;   // false once a wait of this wave gave up: the wave then only meets the barriers
    for (int st = 0; st < nstages && ok; ++st) {
      const int qu = st - up_lag;
      if (qu >= 0 && qu < nslices) {
        u32x4 acc = have_own ? own : load(qu);
        have_own = false;
        acc = R::pre(acc);
        for (int j = 0; j < 3; ++j) {
          const int c = down[j];
          if (c < 0) continue;
          u32x4 y;
          if (!ll_recv(ctl, up_fifo + (size_t)c * kFifoWords, &up_used[c], nrecv_up[j]++, p, y)) {
            ok = false;
            break;
          }
          acc = R::op(acc, y);
        }
        if (!ok) break;
        if (qu + 1 < nslices) {   // the next reduce slice's own input, read during the waits ahead
          own = load(qu + 1);
          have_own = true;
        }
        if (is_root) {
          store(qu, acc);
          if (has_children && !send_down(acc)) {
            ok = false;
            break;
          }
        } else if (!ll_send(ctl, up_fifo + (size_t)r * kFifoWords, &up_used[r], nup++, p, acc)) {
          ok = false;
          break;
        }
      }
      const int qd = st - dn_lag;
      if (!is_root && qd >= 0 && qd < nslices) {
        u32x4 x;
        if (!ll_recv(ctl, dn_fifo + (size_t)up * kFifoWords, &dn_used[3 * up + my_slot], nrecv_dn++, p, x)) {
          ok = false;
          break;
        }
        store(qd, x);
        if (has_children && !send_down(x)) {
          ok = false;
          break;
        }
      }
    }
    __syncthreads();   // every FIFO item of the task consumed before the restart
  }
}

// ---------------------------------------------------------------------------
// Launch.

template <typename K>
static hipError_t ll_allow_lds(K kernel, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)lds);
}

template <DType T, Op O>
static hipError_t launch_ll_t(bool ring, const StepArgs& a, uint32_t* status, uint32_t spin_limit, int grid,
                              int block, size_t lds, hipStream_t s) {
  if (ring) {
    if (hipError_t e = ll_allow_lds(ll_ring<Red<T, O>, Unit<T>::esz>, lds)) return e;
    hipLaunchKernelGGL((ll_ring<Red<T, O>, Unit<T>::esz>), dim3(grid), dim3(block), lds, s, a,
                       static_cast<const RingTask*>(a.tasks), static_cast<const RingLoopBlock*>(a.table), a.orders,
                       status, spin_limit);
  } else {
    if (hipError_t e = ll_allow_lds(ll_tree<Red<T, O>, Unit<T>::esz>, lds)) return e;
    hipLaunchKernelGGL((ll_tree<Red<T, O>, Unit<T>::esz>), dim3(grid), dim3(block), lds, s, a,
                       static_cast<const TreeTask*>(a.tasks), static_cast<const TreeNode*>(a.table), status,
                       spin_limit);
  }
  return hipGetLastError();
}

hipError_t launch_ll(bool ring, DType t, Op op, const StepArgs& a, uint32_t* status, uint32_t spin_limit, int grid,
                     int block, size_t lds, hipStream_t s) {
  switch (t) {
    case DType::I32: return op == Op::Sum ? launch_ll_t<DType::I32, Op::Sum>(ring, a, status, spin_limit, grid, block, lds, s)
                                          : launch_ll_t<DType::I32, Op::Max>(ring, a, status, spin_limit, grid, block, lds, s);
    case DType::I64: return op == Op::Sum ? launch_ll_t<DType::I64, Op::Sum>(ring, a, status, spin_limit, grid, block, lds, s)
                                          : launch_ll_t<DType::I64, Op::Max>(ring, a, status, spin_limit, grid, block, lds, s);
    case DType::F32: return op == Op::Sum ? launch_ll_t<DType::F32, Op::Sum>(ring, a, status, spin_limit, grid, block, lds, s)
                                          : launch_ll_t<DType::F32, Op::Max>(ring, a, status, spin_limit, grid, block, lds, s);
    case DType::F16: return op == Op::Sum ? launch_ll_t<DType::F16, Op::Sum>(ring, a, status, spin_limit, grid, block, lds, s)
                                          : launch_ll_t<DType::F16, Op::Max>(ring, a, status, spin_limit, grid, block, lds, s);
    case DType::BF16: return op == Op::Sum ? launch_ll_t<DType::BF16, Op::Sum>(ring, a, status, spin_limit, grid, block, lds, s)
                                           : launch_ll_t<DType::BF16, Op::Max>(ring, a, status, spin_limit, grid, block, lds, s);
  }
  return hipErrorInvalidValue;
}

// LDS of the LL kernels for n ranks: FIFOs, consumed counters, abandon flag.
size_t ll_lds(bool ring, int n) {
  const size_t fifo = (size_t)kFifoWords * sizeof(uint64_t);
  return ring ? (size_t)n * fifo + ((size_t)n + 1) * sizeof(uint32_t)
              : 2 * (size_t)n * fifo + (4 * (size_t)n + 1) * sizeof(uint32_t);
}

template <typename K>
static int ll_occupancy_of(K kernel, int block, size_t lds) {
  int blocks = 0;
  if (ll_allow_lds(kernel, lds) != hipSuccess) return 1;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, block, lds);
  return e == hipSuccess && blocks > 0 ? blocks : 1;
}
template <DType T, Op O>
static int ll_occupancy_t(bool ring, int block, size_t lds) {
  return ring ? ll_occupancy_of(ll_ring<Red<T, O>, Unit<T>::esz>, block, lds)
              : ll_occupancy_of(ll_tree<Red<T, O>, Unit<T>::esz>, block, lds);
}
int ll_occupancy(bool ring, DType t, Op op, int block, size_t lds) {
  switch (t) {
    case DType::I32: return op == Op::Sum ? ll_occupancy_t<DType::I32, Op::Sum>(ring, block, lds)
                                          : ll_occupancy_t<DType::I32, Op::Max>(ring, block, lds);
    case DType::I64: return op == Op::Sum ? ll_occupancy_t<DType::I64, Op::Sum>(ring, block, lds)
                                          : ll_occupancy_t<DType::I64, Op::Max>(ring, block, lds);
    case DType::F32: return op == Op::Sum ? ll_occupancy_t<DType::F32, Op::Sum>(ring, block, lds)
                                          : ll_occupancy_t<DType::F32, Op::Max>(ring, block, lds);
    case DType::F16: return op == Op::Sum ? ll_occupancy_t<DType::F16, Op::Sum>(ring, block, lds)
                                          : ll_occupancy_t<DType::F16, Op::Max>(ring, block, lds);
    case DType::BF16: return op == Op::Sum ? ll_occupancy_t<DType::BF16, Op::Sum>(ring, block, lds)
                                           : ll_occupancy_t<DType::BF16, Op::Max>(ring, block, lds);
  }
  return 1;
}

}  // namespace emu
