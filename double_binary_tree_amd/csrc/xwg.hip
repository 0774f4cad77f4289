// Stepwise ring all-reduce across workgroups: every (channel, ring position)
// is a workgroup of its own, as NCCL runs one CTA per channel on every GPU
// (page "NCCL 内部机制：…", sections "Chunk、slice、step 是三个尺度" and
// "Ring：带宽友好…"), and a step's data reaches the next position through a
// FIFO in device memory: the position writes its slice into a slot, the next
// position reads it there.  The workgroups of one call may sit on different
// XCDs, whose L2 caches are not kept coherent with each other, so a hand-off
// needs agent-scope visibility.  Two protocols (page "NCCL 内部机制：…",
// sections "Simple：有效载荷效率与大消息吞吐" and "LL：用更高的元数据比例换
// 低延迟"):
//   SIMPLE  the writer stores the slice, makes its stores visible at agent
//           scope (a release fence: the XCD's L2 writes back), and then bumps
//           the FIFO's tail counter; the reader polls the tail, invalidates
//           its caches (an acquire fence) and reads the slice.
//   LL      every 8-byte word carries 4 data bytes and 4 flag bytes (the
//           item's sequence number) and is written and read with one
//           agent-scope atomic access, so no fence is needed: the reader
//           polls the words until they carry the flag it expects.
// Either way the reader publishes how many items it consumed (head), and a
// writer waits for the slot's previous item to be consumed before reusing
// it (nslots slots per FIFO).
//
// Steps and element order are exactly step_ring's (reduce-scatter: block
// r - s at step s, the own input added to the incoming partial; all-gather:
// finished blocks forwarded).  A step moves its block slice by slice: a
// slice is 256 x V vectors of the global slice-cell grid, and every step of a
// loop moves the same number of slices (the most any block of the loop
// spans; the slices past a shorter block carry nothing), so sender and
// receiver walk the same item sequence.  The counters continue across
// calls (a call starts from the consumed counts its FIFOs hold; at the end
// of every call everything written has been consumed).
//
// Why the FIFO must hold a whole step: step 0 only sends, so every position
// pushes M items (M = slices per step) before it reads any.  Counting items
// sent minus items received at a position, a send happens at a difference
// of at most M - 1 and a receive at a difference of at least 1 (each loop
// sends and receives the same (2N - 2) M items).  If every position waited
// to send, each FIFO would hold nslots unread items, so the differences
// would add up to at least N * nslots > N (M - 1): impossible when
// nslots >= M.  A position waiting to receive item j from a position that
// waits to send would mean that position has written more than j items,
// so item j is there.  Hence no cycle of waits.
//
// Every workgroup of a call must be resident at once (a wait can be for
// any other workgroup), so the call is a cooperative launch, which the
// runtime refuses when the grid does not fit.  Every wait is bounded
// (x.spin_limit polls); on expiry the workgroup sets the abandon word and
// the status word.  Every other wait gives up once it sees the abandon word,
// and a call that starts with it set does nothing: after an abandoned call
// the FIFO counters no longer match, so the host must clear the workspace
// before the transport is used again.
#include "device_ops.h"
#include "xwg.h"

namespace emu {

constexpr int kXThreads = 256;
// 16-byte vectors per thread in one slice (one FIFO item): a larger slice
// spreads the fixed cost of a hand-off over more data.
#ifndef EMU_XWG_VPT_SIMPLE
#define EMU_XWG_VPT_SIMPLE 8
#endif
#ifndef EMU_XWG_VPT_LL
#define EMU_XWG_VPT_LL 2
#endif
constexpr int kXVSimple = EMU_XWG_VPT_SIMPLE, kXVLL = EMU_XWG_VPT_LL;
constexpr uint32_t kXWords = 4;               // LL: 8-byte words per 16-byte vector
// s_waitcnt operand: vector memory count 0, the export and LDS/scalar counts
// left at their maxima (no wait on them)
constexpr int kVmcntZero = 0x0F70;

__device__ __forceinline__ uint32_t xload_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void xstore_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// a is at or past b, counting modulo 2^32
__device__ __forceinline__ bool at_or_past(uint32_t a, uint32_t b) { return (int32_t)(a - b) >= 0; }

template <typename R, int ESZ, bool LL>
__global__ __launch_bounds__(kXThreads) void xring(const StepArgs a, const XArgs x,
                                                    const RingLoopBlock* __restrict__ loops,
                                                    const uint32_t* __restrict__ orders) {
  constexpr int unit = kVecBytes / ESZ;
  constexpr int V = LL ? kXVLL : kXVSimple;
  constexpr uint64_t kSliceElems = (uint64_t)kXThreads * V * unit;
  using Vecs = u32x4[V];
  __shared__ uint32_t wg_bad;      // set (and kept) once a wait of this workgroup gave up
  __shared__ uint32_t wg_seen;     // the counter value thread 0 read last
  __shared__ uint32_t wg_base[2];
  const uint32_t n = a.nranks;
  const uint32_t c = blockIdx.x / n, r = blockIdx.x % n;   // channel, ring position
  const uint32_t t = threadIdx.x;
  const uint32_t prev = (r + n - 1) % n;
  const uint32_t f_out = c * n + r, f_in = c * n + prev;     // FIFO written / read
  const uint32_t me = __builtin_amdgcn_readfirstlane(orders[(size_t)x.chan_ring[c] * kMaxRanks + r]);
  uint32_t* const head_out = x.head + (size_t)f_out * kXCounterStride;
  uint32_t* const head_in = x.head + (size_t)f_in * kXCounterStride;
  uint32_t* const tail_out = x.tail + (size_t)f_out * kXCounterStride;
  uint32_t* const tail_in = x.tail + (size_t)f_in * kXCounterStride;
  const uint32_t nslots = x.nslots;
  // a slot in 16-byte units: a slice of 16-byte vectors, twice that with LL
  // (kXWords 8-byte words a vector, word w of vector j of thread t at
  // (w * V + j) * kXThreads + t)
  const size_t slot_vecs = (size_t)(LL ? kXWords * 8 / kVecBytes : 1) * kXThreads * V;
  u32x4* const fifo = static_cast<u32x4*>(x.fifo);
  u32x4* const slots_out = fifo + (size_t)f_out * nslots * slot_vecs;
  u32x4* const slots_in = fifo + (size_t)f_in * nslots * slot_vecs;

  // Items consumed so far from the FIFO this workgroup writes and from the
  // one it reads: at the start of a call every item written has been
  // consumed, and only the reader moves a head.
  if (t == 0) {
    wg_base[0] = xload_relaxed(head_out);
    wg_base[1] = xload_relaxed(head_in);
    wg_bad = xload_relaxed(x.abandon) != 0;
  }
  __syncthreads();
  if (wg_bad) return;
  const uint32_t base_out = wg_base[0], base_in = wg_base[1];

  auto give_up = [&]() {
    xstore_relaxed(x.abandon, 1u);
    xstore_relaxed(x.status, 1u);
  };
  // Wait until *p reaches `need`; `seen` is the last value read, the same in
  // every thread.  Thread 0 polls; the value (or the failure) reaches every
  // thread through LDS.
  auto wait_counter = [&](const uint32_t* p, uint32_t need, uint32_t& seen) -> bool {
    if (at_or_past(seen, need)) return true;
    if (t == 0) {
      for (uint32_t it = 0;; ++it) {
        const uint32_t v = xload_relaxed(p);
        if (at_or_past(v, need)) {
          wg_seen = v;
          break;
        }
        if (it >= x.spin_limit || ((it & 63) == 63 && xload_relaxed(x.abandon))) {
          give_up();
          wg_bad = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __syncthreads();
    if (wg_bad) return false;
    seen = wg_seen;
    __syncthreads();   // every thread has read wg_seen before thread 0 may write it again
    return true;
  };

  uint32_t nsent = 0, nrecv = 0;
  uint32_t seen_head = base_out, seen_tail = base_in;
  // Send item nsent: wait until the slot's previous item was consumed, write
  // the slice, publish it.
  auto send = [&](const Vecs& v) -> bool {
    const uint32_t k = nsent++;
    if (k >= nslots && !wait_counter(head_out, base_out + k + 1 - nslots, seen_head)) return false;
    u32x4* const slot = slots_out + (size_t)(k % nslots) * slot_vecs;
    if constexpr (LL) {
      uint64_t* const w = reinterpret_cast<uint64_t*>(slot) + t;
      const uint64_t flag = (uint64_t)(base_out + k + 1) << 32;
      constexpr size_t W = (size_t)V * kXThreads;   // words between the 4 words of one vector
#pragma unroll
      for (int j = 0; j < V; ++j) {
        uint64_t* const wj = w + (size_t)j * kXThreads;
        __hip_atomic_store(wj + 0 * W, flag | v[j].x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(wj + 1 * W, flag | v[j].y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(wj + 2 * W, flag | v[j].z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(wj + 3 * W, flag | v[j].w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
#pragma unroll
      for (int j = 0; j < V; ++j) slot[(size_t)j * kXThreads + t] = v[j];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");   // the slice reaches memory the readers see
      __syncthreads();
      if (t == 0) xstore_relaxed(tail_out, base_out + k + 1);
    }
    return true;
  };
  // Receive item nrecv into y (then ack() once y has been used).
  auto recv = [&](Vecs& y) -> bool {
    const uint32_t k = nrecv;
    const u32x4* const slot = slots_in + (size_t)(k % nslots) * slot_vecs;
    if constexpr (LL) {
      const uint64_t* const w = reinterpret_cast<const uint64_t*>(slot) + t;
      const uint32_t flag = base_in + k + 1;
      constexpr size_t W = (size_t)V * kXThreads;
      uint64_t wd[V][kXWords];
      bool good = true;
      for (uint32_t it = 0;; ++it) {
        bool ready = true;
#pragma unroll
        for (int j = 0; j < V; ++j)
#pragma unroll
          for (int q = 0; q < (int)kXWords; ++q) {
            wd[j][q] = __hip_atomic_load(w + (size_t)j * kXThreads + q * W, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
            ready = ready && (uint32_t)(wd[j][q] >> 32) == flag;
          }
        if (ready) break;
        if (it >= x.spin_limit || ((it & 63) == 63 && xload_relaxed(x.abandon))) {
          give_up();
          good = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (!good) wg_bad = 1;
      __syncthreads();
      if (wg_bad) return false;
#pragma unroll
      for (int j = 0; j < V; ++j)
        y[j] = u32x4{(uint32_t)wd[j][0], (uint32_t)wd[j][1], (uint32_t)wd[j][2], (uint32_t)wd[j][3]};
    } else {
      if (!wait_counter(tail_in, base_in + k + 1, seen_tail)) return false;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // no stale cached copy of the slice is read
#pragma unroll
      for (int j = 0; j < V; ++j) y[j] = slot[(size_t)j * kXThreads + t];
    }
    return true;
  };
  // The item received last has been read by every thread: publish it.
  // SIMPLE reads the slot with plain loads, which a workgroup barrier does
  // not wait for, and the value may be used only after the barrier; so
  // every thread first waits for its loads to complete (vmcnt 0), or the
  // writer could refill the slot under a load still in flight.  (LL has
  // compared every word it read already.)
  auto ack = [&]() {
    const uint32_t k = nrecv++;
    if constexpr (!LL) __builtin_amdgcn_s_waitcnt(kVmcntZero);
    __syncthreads();
    if (t == 0) xstore_relaxed(head_in, base_in + k + 1);
  };

  const uint32_t loop_begin = x.chan_loops[2 * c], loop_end = x.chan_loops[2 * c + 1];
  for (uint32_t l = loop_begin; l < loop_end; ++l) {
    const uint32_t m = x.loop_slices[l];
    // block of step s: reduce-scatter (r - s) mod N, all-gather (r + 1 - j)
    // mod N with j = s - N + 1; counted down step by step (the first
    // all-gather step works on block r)
    uint32_t b = r;
    for (uint32_t s = 0; s + 1 < 2 * n; ++s) {
      if (s == n) b = r;
      else if (s > 0) b = b == 0 ? n - 1 : b - 1;
      const RingLoopBlock d = loops[(size_t)l * n + b];
      const uint64_t end = d.offset + d.nelem;
      for (uint32_t q = 0; q < m; ++q) {
        uint64_t pos[V];
        int nb[V];
#pragma unroll
        for (int j = 0; j < V; ++j) {
          pos[j] = ((uint64_t)d.first_cell + q) * kSliceElems + ((uint64_t)j * kXThreads + t) * unit;
          nb[j] = 0;
          if (pos[j] >= d.offset && pos[j] < end)
            nb[j] = end - pos[j] >= (uint64_t)unit ? kVecBytes : (int)((end - pos[j]) * ESZ);
        }
        // The own input: whole vectors are loaded before the item is
        // received (the loads overlap the wait; out-of-range offsets, no
        // branch), a partial vector, only ever at a block's end, once it is
        // in (own_part).  Loading both under conditions before the wait made
        // the merge of the two a register copy that waited for every load.
        const char* const own_cell =
            static_cast<const char*>(a.send[me]) + ((uint64_t)d.first_cell + q) * kSliceElems * ESZ;
        const auto own_rs = buffer_view(own_cell);
        auto lane_off = [&](int j) { return ((uint32_t)j * kXThreads + t) * (uint32_t)kVecBytes; };
        auto own = [&](Vecs& v) {
#pragma unroll
          for (int j = 0; j < V; ++j) v[j] = ld_buf(own_rs, nb[j] == kVecBytes ? lane_off(j) : kNoLoad);
        };
        auto own_part = [&](Vecs& v) {
#pragma unroll
          for (int j = 0; j < V; ++j) {
            if (nb[j] > 0 && nb[j] < kVecBytes) v[j] = ld_part(own_cell, lane_off(j), nb[j]);
            v[j] = R::pre(v[j]);
          }
        };
        auto out = [&](const Vecs& v) {
#pragma unroll
          for (int j = 0; j < V; ++j)
            if (nb[j]) st_any(a.recv[me], pos[j] * ESZ, nb[j], R::post(v[j]));
        };
        Vecs v, y;
        if (s == 0) {
          own(v);
          own_part(v);
          if (n == 1) out(v);   // one rank: its own block is the result
          else if (!send(v)) return;
        } else if (s < n) {
          own(v);
          if (!recv(y)) return;
          own_part(v);
#pragma unroll
          for (int j = 0; j < V; ++j) v[j] = R::op(v[j], y[j]);
          ack();
          if (s == n - 1) out(v);   // the finished block (r + 1) mod N
          if (!send(v)) return;
        } else {
          if (!recv(y)) return;
          out(y);
          ack();
          if (s + 2 < 2 * n && !send(y)) return;
        }
      }
    }
  }
}

template <DType T, Op O>
static const void* xring_fn(bool ll) {
  return ll ? reinterpret_cast<const void*>(xring<Red<T, O>, Unit<T>::esz, true>)
            : reinterpret_cast<const void*>(xring<Red<T, O>, Unit<T>::esz, false>);
}

static const void* xring_kernel(bool ll, DType t, Op op) {
  switch (t) {
#define EMU_XCASE(T) \
  case DType::T:     \
    return op == Op::Sum ? xring_fn<DType::T, Op::Sum>(ll) : xring_fn<DType::T, Op::Max>(ll);
    EMU_XCASE(I32)
    EMU_XCASE(I64)
    EMU_XCASE(F32)
    EMU_XCASE(F16)
    EMU_XCASE(BF16)
#undef EMU_XCASE
  }
  return nullptr;
}

hipError_t launch_xring(bool ll, DType t, Op op, const StepArgs& a, const XArgs& x, const RingLoopBlock* loops,
                        const uint32_t* orders, int grid, hipStream_t s) {
  const void* f = xring_kernel(ll, t, op);
  if (!f) return hipErrorInvalidValue;
  void* args[] = {const_cast<StepArgs*>(&a), const_cast<XArgs*>(&x), &loops, &orders};
  return hipLaunchCooperativeKernel(f, dim3(grid), dim3(kXThreads), args, 0, s);
}

int xring_threads() { return kXThreads; }
// 16-byte vectors in one slice.
int xring_slice_vectors(bool ll) { return kXThreads * (ll ? kXVLL : kXVSimple); }

// Workgroups of the kernel that can be resident at once on the device.
int xring_capacity(bool ll, DType t, Op op, int cus) {
  const void* f = xring_kernel(ll, t, op);
  int per_cu = 0;
  if (!f || hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, kXThreads, 0) != hipSuccess) return 0;
  return per_cu * cus;
}

}  // namespace emu
