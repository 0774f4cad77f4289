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
//   lane group p is ring position p, played by the rank the channel's order
//   puts there.  step 0: position p sends its block p;  steps 1..N-1: it
//   receives block (p-s) mod N, adds its own input, sends it on (the last
//   of these writes the finished block); then N-1 all-gather steps forward
//   finished blocks.
// Tree (page "NCCL 专家课程 13", sections "runTreeSplit 如何流水" and "每种
// rank 的操作"): a rank at depth d reduces slice q at stage q + (H - d)
// (children's partials arrive from the previous stage) and, if not the root,
// broadcasts slice q at stage q + H + d; the root writes the result at its
// reduce stage.  Reduce-up and broadcast-down run concurrently on different
// slices, with separate slot sets, as the split thread groups of the pages do.
#include <algorithm>

#include "device_ops.h"

namespace emu {

// Occupancy targets (waves per SIMD the compiler must leave registers for;
// 0: none), build-time tuning knobs.  A 1024-thread workgroup is 4 waves per
// SIMD, so two resident workgroups need 8.  Measured on MI355X (3
// alternating rounds against the uncapped build): the ring with two or four
// ranks per wave needs 70-91 VGPRs, one workgroup per CU; held to 8 waves
// (64 VGPRs, 24-120 bytes per lane spilled) it ran 13% faster on 4 x 8 ranks
// f16, 7% on 16 ranks bf16, 5% on 4 x 8 ranks i64, and within 0.5% with 8
// ranks and for the standalone reduce-scatter and all-gather.  The tree with
// two ranks per wave ran 1-3% slower held to 8 waves: its pipeline is then
// split into twice as many shorter pieces, each paying its fill and drain.
#ifndef EMU_RING_WAVES_PER_EU
#define EMU_RING_WAVES_PER_EU 8
#endif
#ifndef EMU_TREE_WAVES_PER_EU
#define EMU_TREE_WAVES_PER_EU 0
#endif
#if EMU_RING_WAVES_PER_EU
#define EMU_RING_OCCUPANCY __attribute__((amdgpu_waves_per_eu(EMU_RING_WAVES_PER_EU)))
#else
#define EMU_RING_OCCUPANCY
#endif
#if EMU_TREE_WAVES_PER_EU
#define EMU_TREE_OCCUPANCY __attribute__((amdgpu_waves_per_eu(EMU_TREE_WAVES_PER_EU)))
#else
#define EMU_TREE_OCCUPANCY
#endif

// LDS barrier for step hand-off: LDS writes are complete before the barrier;
// outstanding global loads (prefetches of the next step) stay in flight.
__device__ __forceinline__ void step_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// ---------------------------------------------------------------------------
// Ring.
// Vectors per lane per step and how many steps of a rank's own input are
// loaded ahead.  Larger values keep more bytes in flight per wave but cost
// registers (and so resident workgroups); these are the measured optima for
// each kernel on MI355X.
#ifndef EMU_RING_VPT
#define EMU_RING_VPT 1
#endif
// The ring's own-input queue is one entry deep: it is refilled in place
// once the step has used it, so the load for step s + 1 is issued at the end
// of step s and waited for at the start of step s + 1, its latency under the
// barrier.  Deeper queues are moved on by register copies, which the
// compiler makes wait for every load in flight (measured on MI355X against
// two entries: full-size legs 1-3% faster at 8, 16 and 32 ranks, 16 ranks
// 3-6% faster up to 1 MiB per rank, 32 ranks 9% faster at 8-16 MiB and 5%
// slower at 256 KiB-2 MiB).
#ifndef EMU_RING_PREFETCH
#define EMU_RING_PREFETCH 1
#endif

#ifndef EMU_RING_PREFETCH_WAVE
#define EMU_RING_PREFETCH_WAVE 1
#endif
// All-reduce tasks take slice (q + b * skew) mod (slices of the loop) of
// block b rather than slice q of every block.  Each block still gets every
// slice once and no element's order changes; what changes is which slices
// are in flight together.  Without a skew the workgroups running at once
// read and write the same offsets of N^2 (rank, block) regions that lie
// whole multiples of the chunk apart.  Measured on MI355X with 8 ranks and
// 512 KiB chunks: stepwise ring 226 -> 204 us with a skew of 100-384
// slices; the standalone reduce-scatter / all-gather were slower with it,
// so they keep slice q.
#ifndef EMU_RING_SKEW
#define EMU_RING_SKEW 100
#endif
#ifndef EMU_TREE_VPT
#define EMU_TREE_VPT 1
#endif
#ifndef EMU_TREE_PREFETCH
#define EMU_TREE_PREFETCH 2
#endif
#ifndef EMU_TREE_PREFETCH_WAVE
#define EMU_TREE_PREFETCH_WAVE 3
#endif

// COLL selects the collective: the all-reduce runs both halves; the
// standalone reduce-scatter stops after its N-1 steps and writes the
// finished block (the position's own block) to its rank's output, one
// block lower; the standalone all-gather starts from each position's own
// input (one block lower) and runs only the N-1 forwarding steps.
//
// WAVE: the group is one wave (G = 64), so the position, its rank and every
// block descriptor are wave-uniform; they are moved to scalar registers and
// only the lane's place in the slice stays per lane.
//
// The task and record tables come as their own read-only arguments: uniform
// reads from them then go through the scalar unit, whose counter is separate
// from the vector-memory counter; a vector load there would make the wait
// for it also wait for every store issued before it.
template <bool WAVE>
__device__ __forceinline__ uint32_t wave_u32(uint32_t x) {
  if constexpr (WAVE) return __builtin_amdgcn_readfirstlane(x);
  return x;
}
template <bool WAVE>
__device__ __forceinline__ uint64_t wave_u64(uint64_t x) {
  if constexpr (WAVE)
    return (uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)x) |
           (uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(x >> 32)) << 32;
  return x;
}

template <typename R, int ESZ, int COLL, int RPW>
__global__ __launch_bounds__(1024) EMU_RING_OCCUPANCY void step_ring(const StepArgs a, const RingTask* __restrict__ tasks,
                                                   const RingLoopBlock* __restrict__ loops,
                                                   const uint32_t* __restrict__ orders) {
  constexpr bool WAVE = RPW == 1;
  constexpr uint32_t G = 64u / RPW;
  constexpr int unit = kVecBytes / ESZ;
  constexpr int V = EMU_RING_VPT;
  constexpr int kPrefetch = WAVE ? EMU_RING_PREFETCH_WAVE : EMU_RING_PREFETCH;
  constexpr uint32_t kSkew = COLL == kAllReduce ? EMU_RING_SKEW : 0;
  extern __shared__ u32x4 fifo[];   // slots [2][N][V][G], descriptors [2][N], ring orders [2][kMaxRanks] bytes
  const uint32_t n = a.nranks, g = G;
  // r: ring position (the lane's); the wave holds positions wave*RPW .. wave*RPW + RPW-1
  const uint32_t wave = wave_u32<true>(threadIdx.x / 64u);
  const uint32_t grp = WAVE ? 0u : (threadIdx.x % 64u) / G;
  const uint32_t r = wave * RPW + grp;
  const uint32_t p = threadIdx.x % G;
  const bool active = r < n;
  const uint32_t prev = active ? (r + n - 1) % n : 0;
  auto slot = [&](uint32_t parity, uint32_t rank, int v) -> u32x4& {
    return fifo[((parity * n + rank) * V + v) * g + p];
  };
  // Block descriptors of the current and the next task, staged in LDS (two
  // sets) so that no step waits on a descriptor load: the next task's are
  // copied during the current task's first step.  (Measured on MI355X:
  // staging with per-wave scalar loads, or a queue unrolled to rotate by
  // name as the tree does, were each about 15% slower here.)
  RingLoopBlock* desc = reinterpret_cast<RingLoopBlock*>(fifo + 2 * (size_t)n * V * g);   // [2][N]
  uint8_t* order = reinterpret_cast<uint8_t*>(desc + 2 * n);                                // [2][kMaxRanks]
  // The staged descriptor of block b holds, in place of the block's first
  // cell, the cell this task reads and writes in it (its slice q of the
  // block, skewed per block for the all-reduce), so the steps compute no
  // index modulo the slice count.
  auto stage_desc = [&](uint32_t t, uint32_t set) {
    if (t < a.ntasks && threadIdx.x < n) {
      const RingTask tk = tasks[t];
      RingLoopBlock d = loops[(size_t)tk.loop * n + threadIdx.x];
      d.first_cell += kSkew ? (tk.slice + threadIdx.x * kSkew) % tk.nslices : tk.slice;
      desc[set * n + threadIdx.x] = d;
      order[set * kMaxRanks + threadIdx.x] = (uint8_t)orders[(size_t)tk.ring * kMaxRanks + threadIdx.x];
    }
  };
  stage_desc(blockIdx.x, 0);
  step_barrier();

  uint32_t set = 0;
  for (uint32_t t = blockIdx.x; t < a.ntasks; t += gridDim.x, set ^= 1) {
    const RingLoopBlock* blk = desc + set * n;
    // The rank at the lane's position, and its buffers, looked up once per
    // task: with several ranks per wave the rank differs between lanes, and
    // indexing the argument's pointer table with it is a vector load whose
    // wait (vmcnt 0) would also wait for every prefetch in flight.
    const uint32_t me = active ? wave_u32<WAVE>(order[set * kMaxRanks + r]) : 0;
    const char* const src_me = static_cast<const char*>(a.send[me]);
    char* const dst_me = static_cast<char*>(a.recv[me]);
    // byte distance between a block's place and the rank's own buffer
    const uint64_t my_shift = COLL == kAllReduce ? 0 : (uint64_t)me * a.block * ESZ;
    const uint64_t load_shift = COLL == kAllGather ? my_shift : 0;
    const uint64_t store_shift = COLL == kReduceScatter ? my_shift : 0;
    // The same for every position of the wave, wave-uniform: the loads of
    // position k read with a buffer view of that rank's buffer.
    const char* wsrc[RPW];
    uint64_t wshift[RPW];
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
      const uint32_t rk = wave * RPW + k;
      const uint32_t mk = wave_u32<true>(order[set * kMaxRanks + (rk < n ? rk : 0)]);
      wsrc[k] = static_cast<const char*>(a.send[mk]);
      wshift[k] = COLL == kAllGather ? (uint64_t)mk * a.block * ESZ : 0;
    }
    if (n > 1) stage_desc(t + gridDim.x, set ^ 1);   // visible after this task's barriers
    // Slice q of block b is the q-th slice-size cell of the global element
    // grid that the block overlaps; lane p's vector v sits at a fixed place in
    // the cell (aligned accesses), and is live only inside the block.
    const uint64_t slice_elems = (uint64_t)V * g * unit;
    // Block b as seen by this task: the first element of its slice cell and
    // its [start, end) range.  view_u: for a wave-uniform b, in scalar
    // registers; view_of: for the lane's own block.
    struct View { uint64_t cell, start, end; };
    auto view_u_of = [&](const RingLoopBlock& d) -> View {
      const uint64_t start = wave_u64<true>(d.offset);
      const uint32_t nelem = wave_u32<true>(d.nelem), cell = wave_u32<true>(d.first_cell);
      return {(uint64_t)cell * slice_elems, start, start + nelem};
    };
    auto view_u = [&](uint32_t b) -> View { return view_u_of(blk[b]); };
    auto view_from = [&](const RingLoopBlock& d) -> View {
      if constexpr (WAVE) return view_u_of(d);
      return {(uint64_t)d.first_cell * slice_elems, d.offset, d.offset + d.nelem};
    };
    auto view_of = [&](uint32_t b) -> View { return view_from(blk[b]); };
    // A cell that lies wholly inside its block: every lane holds a whole
    // vector, so no lane needs its bounds checked.
    auto whole = [&](const View& w) { return w.start <= w.cell && w.cell + slice_elems <= w.end; };
    auto nbytes_of = [&](const View& w, uint64_t pos) -> int {
      if (pos < w.start || pos >= w.end) return 0;
      const uint64_t left = w.end - pos;
      return left >= (uint64_t)unit ? kVecBytes : (int)(left * ESZ);
    };
    // Loads block bk[k] of the rank at position k of the wave into x[k], for
    // every k: one buffer view per position based at the block's slice cell
    // (uniform), in which only that position's lanes pass a real offset
    // (whole vectors; other lanes read zeros, the hardware range check).  A
    // partial vector at the message end is read when it is consumed
    // (fix_block).  Issued for the whole wave, outside any per-lane branch,
    // and never into a register that anything but a load writes.
    auto load_blocks = [&](const uint32_t (&bk)[RPW], u32x4 (&x)[RPW][V], bool enable, View* w0 = nullptr) {
#pragma unroll
      for (int k = 0; k < RPW; ++k) {
        const bool en = enable && wave * RPW + k < n;
        const View w = view_u(bk[k]);
        if (k == 0 && w0) *w0 = w;
        const auto rs = buffer_view(wsrc[k] + (w.cell * ESZ - wshift[k]));
        const bool mine = WAVE || grp == (uint32_t)k;
        if (en && whole(w)) {
#pragma unroll
          for (int v = 0; v < V; ++v) x[k][v] = ld_buf(rs, mine ? (uint32_t)((v * g + p) * kVecBytes) : kNoLoad);
        } else {
#pragma unroll
          for (int v = 0; v < V; ++v) {
            const uint32_t lane = (uint32_t)((v * g + p) * unit);
            x[k][v] = ld_buf(rs, en && mine && nbytes_of(w, w.cell + lane) == kVecBytes ? lane * ESZ : kNoLoad);
          }
        }
      }
    };
    auto take = [&](const u32x4 (&x)[RPW][V], u32x4 (&out)[V]) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        out[v] = x[0][v];
#pragma unroll
        for (int k = 1; k < RPW; ++k) out[v] |= x[k][v];
      }
    };
    auto fix_view = [&](const View& w, u32x4 (&x)[V]) {
      if (w.cell + slice_elems <= w.end) return;   // a partial vector can only sit at the block end
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const uint64_t pos = w.cell + (uint32_t)((v * g + p) * unit);
        const int nb = nbytes_of(w, pos);
        if (nb > 0 && nb < kVecBytes) x[v] = ld_part(src_me, pos * ESZ - load_shift, nb);
      }
    };
    auto fix_block = [&](uint32_t b, u32x4 (&x)[V]) { fix_view(view_of(b), x); };
    auto store_view = [&](const View& w, const u32x4 (&x)[V]) {
      if (whole(w)) {
#pragma unroll
        for (int v = 0; v < V; ++v)
          st_vec(dst_me, (w.cell + (uint32_t)((v * g + p) * unit)) * ESZ - store_shift, R::post(x[v]));
        return;
      }
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const uint64_t pos = w.cell + (uint32_t)((v * g + p) * unit);
        const int nb = nbytes_of(w, pos);
        if (nb) st_any(dst_me, pos * ESZ - store_shift, nb, R::post(x[v]));
      }
    };
    auto store_block = [&](uint32_t b, const u32x4 (&x)[V]) { store_view(view_of(b), x); };
    // the positions of the wave, for block indices counted per position
    uint32_t pos_k[RPW];
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
      const uint32_t rk = wave * RPW + k;
      pos_k[k] = rk < n ? rk : 0;
    }

    if (n == 1) {
      u32x4 x[RPW][V], own[V];
      load_blocks(pos_k, x, true);
      if (active) {
        take(x, own);
        fix_block(0, own);
        store_block(0, own);
      }
      // one rank: no steps, so stage the next descriptor here
      step_barrier();
      stage_desc(t + gridDim.x, set ^ 1);
      step_barrier();
      continue;
    }
    if constexpr (COLL == kAllGather) {
      // the position's own input is the finished block (r+1) mod N: write it
      // to its own output and into the slot the forwarding steps read first
      uint32_t bk[RPW];
#pragma unroll
      for (int k = 0; k < RPW; ++k) bk[k] = pos_k[k] + 1 == n ? 0 : pos_k[k] + 1;
      u32x4 x[RPW][V];
      load_blocks(bk, x, true);
      if (active) {
        u32x4 own[V];
        take(x, own);
        fix_block((r + 1) % n, own);
        store_block((r + 1) % n, own);
#pragma unroll
        for (int v = 0; v < V; ++v) slot((n - 1) & 1, r, v) = R::pre(own[v]);
      }
      step_barrier();
    } else {
    // step 0: send own block r; the blocks of steps 1..PF are loaded ahead
    // (queue q[0] is the next step's block).  Block of step s at position
    // k: (k - s) mod N, counted down per position.
    // With one rank per wave the block's view (read from LDS to place its
    // load) rides in the queue beside the data, so the step that consumes
    // the block reads no descriptor again.
    u32x4 own[RPW][V], q[kPrefetch][RPW][V];
    View own_v, qv[kPrefetch];
    uint32_t bpf[RPW];
    load_blocks(pos_k, own, true, &own_v);
#pragma unroll
    for (int k = 0; k < RPW; ++k) bpf[k] = pos_k[k];
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i) {
#pragma unroll
      for (int k = 0; k < RPW; ++k) bpf[k] = bpf[k] == 0 ? n - 1 : bpf[k] - 1;
      load_blocks(bpf, q[i], (uint32_t)i + 1 < n, &qv[i]);
    }
    if (active) {
      u32x4 mine[V];
      take(own, mine);
      if constexpr (WAVE) fix_view(own_v, mine); else fix_block(r, mine);
#pragma unroll
      for (int v = 0; v < V; ++v) slot(0, r, v) = R::pre(mine[v]);
    }
    step_barrier();
    // the lane's block of step s, (r - s) mod N, counted down step by step
    uint32_t b = r;
    for (uint32_t s = 1; s < n; ++s) {
      b = b == 0 ? n - 1 : b - 1;
      u32x4 mine[V];
      take(q[0], mine);   // this step's entry (waits for its loads only)
      const View wb = qv[0];   // the view of block b (one rank per wave)
      if (active) {
        if constexpr (WAVE) fix_view(wb, mine); else fix_block(b, mine);
        u32x4 res[V];
#pragma unroll
        for (int v = 0; v < V; ++v) res[v] = R::op(R::pre(mine[v]), slot((s - 1) & 1, prev, v));
        if (s == n - 1) {
          if constexpr (WAVE) store_view(wb, res); else store_block(b, res);
        }
#pragma unroll
        for (int v = 0; v < V; ++v) slot(s & 1, r, v) = res[v];
      }
      // The queue moves on after this step's entry is consumed, and its last
      // entry is refilled unconditionally (a load of nothing past the last
      // step).  Refilling earlier, or under a condition, leaves the entry's
      // old value live (or two definitions to merge) where the new load
      // lands, and the compiler moves the loaded registers into place with
      // copies that wait for every load in flight before the barrier.
#pragma unroll
      for (int i = 0; i + 1 < kPrefetch; ++i) {
        qv[i] = qv[i + 1];
#pragma unroll
        for (int k = 0; k < RPW; ++k)
#pragma unroll
          for (int v = 0; v < V; ++v) q[i][k][v] = q[i + 1][k][v];
      }
#pragma unroll
      for (int k = 0; k < RPW; ++k) bpf[k] = bpf[k] == 0 ? n - 1 : bpf[k] - 1;
      load_blocks(bpf, q[kPrefetch - 1], s + kPrefetch < n, &qv[kPrefetch - 1]);
      step_barrier();
    }
    }
    if (COLL == kReduceScatter) continue;
    // all-gather steps 1..N-1: block (r + 1 - j) mod N, counted down.  The
    // descriptor of the next step's block is read from LDS one step ahead
    // (the task's descriptor set does not change during the task), so its
    // latency passes under this step's work and barrier.
    uint32_t bg = (r + 1) % n;
    bg = bg == 0 ? n - 1 : bg - 1;   // step 1's block
    RingLoopBlock dn = blk[bg];
    for (uint32_t j = 1; j < n; ++j) {
      const RingLoopBlock d = dn;
      if (j + 1 < n) {
        bg = bg == 0 ? n - 1 : bg - 1;
        dn = blk[bg];
      }
      if (active) {
        u32x4 x[V];
#pragma unroll
        for (int v = 0; v < V; ++v) x[v] = slot((n - 2 + j) & 1, prev, v);
        store_view(view_from(d), x);
        if (j + 1 < n) {
#pragma unroll
          for (int v = 0; v < V; ++v) slot((n - 1 + j) & 1, r, v) = x[v];
        }
      }
      step_barrier();
    }
  }
}

// ---------------------------------------------------------------------------
// Tree.
// RPW: virtual ranks per wave (64 / G).  Every rank of a wave is known to the
// whole wave (ranks wave*RPW .. wave*RPW + RPW-1), so each rank's record,
// stage lag and current slice are wave-uniform, and a rank's own input is
// read with a buffer view based at that slice's cell (scalar registers):
// one load per rank of the wave, in which only that rank's lanes pass a
// real offset and every other lane an out-of-range one (the hardware range
// check returns zeros).  A lane ORs the RPW results of a queue entry when it
// consumes them.  So no queue entry is ever written by anything but a load,
// and the wait for an entry counts only the loads issued after it: zeroing
// an entry in registers for lanes without a slice would make the compiler
// wait for every load in flight, since the entry may still have a load
// outstanding.
template <typename R, int ESZ, int RPW>
__global__ __launch_bounds__(1024) EMU_TREE_OCCUPANCY void step_tree(const StepArgs a, const TreeTask* __restrict__ tasks,
                                                   const TreeNode* __restrict__ nodes) {
  constexpr int unit = kVecBytes / ESZ;
  constexpr int V = EMU_TREE_VPT;
  constexpr uint32_t G = 64u / RPW;
  constexpr int kPrefetch = RPW == 1 ? EMU_TREE_PREFETCH_WAVE : EMU_TREE_PREFETCH;
  extern __shared__ u32x4 fifo[];   // up[2][N][V][G] then down[2][N][V][G]
  const uint32_t n = a.nranks, g = G;
  const uint32_t wave = wave_u32<true>(threadIdx.x / 64u);
  const uint32_t grp = RPW == 1 ? 0u : (threadIdx.x % 64u) / G;   // the lane's rank among the wave's
  const uint32_t r = wave * RPW + grp;
  const uint32_t p = threadIdx.x % G;
  const bool active = r < n;
  const int H = (int)a.height;
  const uint32_t slice_elems = V * g * unit;
  // The buffers: each rank of the wave (uniform) for the loads, the lane's
  // own rank for partial vectors and stores.
  const char* wsrc[RPW];
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const uint32_t rk = wave * RPW + k;
    wsrc[k] = static_cast<const char*>(a.send[rk < n ? rk : 0]);
  }
  const char* const src_r = static_cast<const char*>(a.send[active ? r : 0]);
  char* const dst_r = static_cast<char*>(a.recv[active ? r : 0]);
  auto up_slot = [&](int parity, uint32_t rank, int v) -> u32x4& {
    return fifo[(((uint32_t)parity * n + rank) * V + v) * g + p];
  };
  auto dn_slot = [&](int parity, uint32_t rank, int v) -> u32x4& {
    return fifo[(((2u + (uint32_t)parity) * n + rank) * V + v) * g + p];
  };

  for (uint32_t t = blockIdx.x; t < a.ntasks; t += gridDim.x) {
    const TreeTask task = tasks[t];
    // the records of the wave's ranks (uniform); the lane's own is one of them
    int lag_k[RPW];
    bool live_k[RPW];
    struct { int up, down[3]; } me = {-1, {-1, -1, -1}};
    int depth = 0;
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
      const uint32_t rk = wave * RPW + k;
      const TreeNode rec = nodes[task.channel * n + (rk < n ? rk : 0)];
      lag_k[k] = H - rec.depth;
      live_k[k] = rk < n;
      if (RPW == 1 || grp == (uint32_t)k) {
        me.up = rec.up;
#pragma unroll
        for (int s = 0; s < 3; ++s) me.down[s] = rec.down[s];
        depth = rec.depth;
      }
    }
    const bool is_root = me.up < 0;
    const bool has_children = me.down[0] >= 0;
    // Slices are the slice-size cells of the global element grid that the
    // task overlaps; lanes outside [start, start + nelem) sit out.
    const uint64_t first_cell = task.start / slice_elems;
    const uint64_t end = task.start + task.nelem;
    const int nslices = (int)((end + slice_elems - 1) / slice_elems - first_cell);
    auto pos_of = [&](int q, int v) -> uint64_t {
      return (first_cell + (uint64_t)q) * slice_elems + ((uint64_t)v * g + p) * unit;
    };
    auto nbytes_of = [&](int q, int v) -> int {
      const uint64_t pos = pos_of(q, v);
      if (pos < task.start || pos >= end) return 0;
      const uint64_t left = end - pos;
      return left >= (uint64_t)unit ? kVecBytes : (int)(left * ESZ);
    };
    auto boff_of = [&](int q, int v) -> uint64_t { return pos_of(q, v) * ESZ; };
    // Every slice but the first and the last lies inside the task: each lane
    // holds a whole vector there, so a store needs no per-lane bounds.
    // (Range checks compare as unsigned: one compare for both bounds.)
    auto interior = [&](int q) { return (uint32_t)(q - 1) < (uint32_t)(nslices - 2); };
    // Own input of the wave's ranks for stage st + kPrefetch (rank k reduces
    // slice st - lag_k there): one buffer load per rank, based at its
    // slice's cell (uniform: a running base per rank that moves one slice on
    // at every stage, so that the view sits in scalar registers without a
    // 64-bit product per stage); whole vectors only, a partial vector at the
    // task end is read when it is consumed (fix_slice).  A base outside the
    // buffer is never used: the range check is on the offset, and every lane
    // without a slice passes kNoLoad.  (Offsets for the first and the last
    // slice computed once per task instead of per stage took a fifth off a
    // stage at small sizes too, but with the running base made the 8-rank
    // chain 6-10% slower from 16 MiB per rank up; either change alone did not.)
    const uint64_t slice_bytes = (uint64_t)slice_elems * ESZ;
    uint32_t lane_off[V];
#pragma unroll
    for (int v = 0; v < V; ++v) lane_off[v] = (uint32_t)((v * g + p) * kVecBytes);
    // The view base of rank k's last load: the first call (stage 0, slice
    // -lag_k) moves it one slice on before use.  Wraps as unsigned, like
    // the slice index it follows.
    uint64_t lbase[RPW];
#pragma unroll
    for (int k = 0; k < RPW; ++k)
      lbase[k] = (uint64_t)wsrc[k] + (first_cell - (uint64_t)(int64_t)(lag_k[k] + 1)) * slice_bytes;
    auto load_stage = [&](int st, u32x4 (&x)[RPW][V]) {
#pragma unroll
      for (int k = 0; k < RPW; ++k) {
        const int qk = st - lag_k[k];
        const bool en = live_k[k] && (uint32_t)qk < (uint32_t)nslices;
        lbase[k] += slice_bytes;
        const auto rs = buffer_view(reinterpret_cast<const void*>(lbase[k]));
        const bool mine = RPW == 1 || grp == (uint32_t)k;
#pragma unroll
        for (int v = 0; v < V; ++v) {
          x[k][v] = ld_buf(rs, en && mine && nbytes_of(qk, v) == kVecBytes ? lane_off[v] : kNoLoad);
        }
      }
    };
    auto fix_slice = [&](int q, u32x4 (&x)[V]) {
      if (q + 1 < nslices) return;   // a partial vector can only sit at the task end
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int nb = nbytes_of(q, v);
        if (nb > 0 && nb < kVecBytes) x[v] = ld_part(src_r, boff_of(q, v), nb);
      }
    };
    auto store_slice = [&](int q, const u32x4 (&x)[V]) {
      if (interior(q)) {
#pragma unroll
        for (int v = 0; v < V; ++v) st_vec(dst_r, boff_of(q, v), R::post(x[v]));
        return;
      }
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int nb = nbytes_of(q, v);
        if (nb) st_any(dst_r, boff_of(q, v), nb, R::post(x[v]));
      }
    };
    const int up_lag = H - depth;        // reduce slice q at stage q + up_lag
    const int dn_lag = H + depth;        // broadcast slice q at stage q + dn_lag
    const int nstages = nslices + 2 * H;

    // The own input that a rank reduces at stage st is loaded PF stages
    // earlier into queue entry st mod PF: the stage loop is unrolled by PF,
    // and at unrolled position i every rank loads the slice it will reduce
    // PF stages later into entry i and reduces the one in entry i.  The
    // entry depends on the stage only, not on the rank's lag, so the ranks of
    // one wave share the queue.  Every entry is refilled unconditionally (a
    // load of nothing when there is no slice), so entries rotate by name and
    // are never merged or copied while their loads are in flight.  Stages
    // -PF .. -1 only refill; every wave meets the barriers of stages
    // 0 .. nstages-1 in order.
    u32x4 q[kPrefetch][RPW][V];
    for (int st0 = -kPrefetch; st0 < nstages; st0 += kPrefetch) {
#pragma unroll
      for (int i = 0; i < kPrefetch; ++i) {
        const int st = st0 + i;
        const bool live = (uint32_t)st < (uint32_t)nstages;
        const int cur = st & 1, prv = cur ^ 1;
        const int qu = st - up_lag;
        // (outside stages 0 .. nstages-1 both slice indices are out of range:
        // 0 <= depth <= H)
        if (active && (uint32_t)qu < (uint32_t)nslices) {
          u32x4 acc[V];
#pragma unroll
          for (int v = 0; v < V; ++v) {
            acc[v] = q[i][0][v];
#pragma unroll
            for (int k = 1; k < RPW; ++k) acc[v] |= q[i][k][v];
          }
          fix_slice(qu, acc);
#pragma unroll
          for (int v = 0; v < V; ++v) acc[v] = R::pre(acc[v]);
#pragma unroll
          for (int s = 0; s < 3; ++s) {
            const int c = me.down[s];
            if (c >= 0) {
#pragma unroll
              for (int v = 0; v < V; ++v) acc[v] = R::op(acc[v], up_slot(prv, (uint32_t)c, v));
            }
          }
          if (is_root) {
            store_slice(qu, acc);
            if (has_children) {
#pragma unroll
              for (int v = 0; v < V; ++v) dn_slot(cur, r, v) = acc[v];
            }
          } else {
#pragma unroll
            for (int v = 0; v < V; ++v) up_slot(cur, r, v) = acc[v];
          }
        }
        load_stage(st + kPrefetch, q[i]);
        if (live) {
          const int qd = st - dn_lag;
          if (active && !is_root && (uint32_t)qd < (uint32_t)nslices) {
            u32x4 x[V];
#pragma unroll
            for (int v = 0; v < V; ++v) x[v] = dn_slot(prv, (uint32_t)me.up, v);
            store_slice(qd, x);
            if (has_children) {
#pragma unroll
              for (int v = 0; v < V; ++v) dn_slot(cur, r, v) = x[v];
            }
          }
          step_barrier();
        }
      }
    }
  }
}

// Kernels that use more than 64 KiB of dynamic LDS must say so before launch.
template <typename K>
static hipError_t allow_lds(K kernel, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)lds);
}

template <DType T, Op O, int COLL, int RPW>
static hipError_t launch_ring_w(const StepArgs& a, int grid, int block, size_t lds, hipStream_t s) {
  if (hipError_t e = allow_lds(step_ring<Red<T, O>, Unit<T>::esz, COLL, RPW>, lds)) return e;
  hipLaunchKernelGGL((step_ring<Red<T, O>, Unit<T>::esz, COLL, RPW>), dim3(grid), dim3(block), lds, s, a,
                     static_cast<const RingTask*>(a.tasks), static_cast<const RingLoopBlock*>(a.table), a.orders);
  return hipGetLastError();
}
template <DType T, Op O, int COLL>
static hipError_t launch_ring_t(const StepArgs& a, int grid, int block, size_t lds, hipStream_t s) {
  switch (a.group) {
    case 64: return launch_ring_w<T, O, COLL, 1>(a, grid, block, lds, s);
    case 32: return launch_ring_w<T, O, COLL, 2>(a, grid, block, lds, s);
    case 16: return launch_ring_w<T, O, COLL, 4>(a, grid, block, lds, s);
    default: return hipErrorInvalidValue;   // the planner keeps the group at 16, 32 or 64 lanes
  }
}
template <DType T, Op O, int RPW>
static hipError_t launch_tree_w(const StepArgs& a, int grid, int block, size_t lds, hipStream_t s) {
  if (hipError_t e = allow_lds(step_tree<Red<T, O>, Unit<T>::esz, RPW>, lds)) return e;
  hipLaunchKernelGGL((step_tree<Red<T, O>, Unit<T>::esz, RPW>), dim3(grid), dim3(block), lds, s, a,
                     static_cast<const TreeTask*>(a.tasks), static_cast<const TreeNode*>(a.table));
  return hipGetLastError();
}
template <DType T, Op O>
static hipError_t launch_tree_t(const StepArgs& a, int grid, int block, size_t lds, hipStream_t s) {
  switch (a.group) {
    case 64: return launch_tree_w<T, O, 1>(a, grid, block, lds, s);
    case 32: return launch_tree_w<T, O, 2>(a, grid, block, lds, s);
    case 16: return launch_tree_w<T, O, 4>(a, grid, block, lds, s);
    default: return hipErrorInvalidValue;   // the planner keeps the group at 16, 32 or 64 lanes
  }
}

template <DType T>
static hipError_t launch_step_t(Coll coll, bool ring, Op op, const StepArgs& a, int grid, int block, size_t lds,
                                hipStream_t s) {
  if (coll == kReduceScatter)
    return op == Op::Sum ? launch_ring_t<T, Op::Sum, kReduceScatter>(a, grid, block, lds, s)
                         : launch_ring_t<T, Op::Max, kReduceScatter>(a, grid, block, lds, s);
  if (ring)
    return op == Op::Sum ? launch_ring_t<T, Op::Sum, kAllReduce>(a, grid, block, lds, s)
                         : launch_ring_t<T, Op::Max, kAllReduce>(a, grid, block, lds, s);
  return op == Op::Sum ? launch_tree_t<T, Op::Sum>(a, grid, block, lds, s)
                       : launch_tree_t<T, Op::Max>(a, grid, block, lds, s);
}

hipError_t launch_stepwise(Coll coll, bool ring, DType t, Op op, const StepArgs& a, int grid, int block,
                           size_t lds, hipStream_t s) {
  if (coll == kAllGather) {
    // a copy: only the element size matters
    switch (elem_size(t)) {
      case 2: return launch_ring_t<DType::F16, Op::Sum, kAllGather>(a, grid, block, lds, s);
      case 4: return launch_ring_t<DType::I32, Op::Sum, kAllGather>(a, grid, block, lds, s);
      case 8: return launch_ring_t<DType::I64, Op::Sum, kAllGather>(a, grid, block, lds, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (t) {
    case DType::I32: return launch_step_t<DType::I32>(coll, ring, op, a, grid, block, lds, s);
    case DType::I64: return launch_step_t<DType::I64>(coll, ring, op, a, grid, block, lds, s);
    case DType::F32: return launch_step_t<DType::F32>(coll, ring, op, a, grid, block, lds, s);
    case DType::F16: return launch_step_t<DType::F16>(coll, ring, op, a, grid, block, lds, s);
    case DType::BF16: return launch_step_t<DType::BF16>(coll, ring, op, a, grid, block, lds, s);
  }
  return hipErrorInvalidValue;
}

int stepwise_vectors_per_lane(bool ring) { return ring ? EMU_RING_VPT : EMU_TREE_VPT; }

template <typename K>
static int occupancy_of(K kernel, int block, size_t lds) {
  int blocks = 0;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, block, lds);
  return e == hipSuccess && blocks > 0 ? blocks : 1;
}

template <DType T, Op O>
static int occupancy_t(bool ring, bool wave, int block, size_t lds, int group) {
  if (!ring)
    return group == 64   ? occupancy_of(step_tree<Red<T, O>, Unit<T>::esz, 1>, block, lds)
           : group == 32 ? occupancy_of(step_tree<Red<T, O>, Unit<T>::esz, 2>, block, lds)
                         : occupancy_of(step_tree<Red<T, O>, Unit<T>::esz, 4>, block, lds);
  return group == 64   ? occupancy_of(step_ring<Red<T, O>, Unit<T>::esz, kAllReduce, 1>, block, lds)
         : group == 32 ? occupancy_of(step_ring<Red<T, O>, Unit<T>::esz, kAllReduce, 2>, block, lds)
                       : occupancy_of(step_ring<Red<T, O>, Unit<T>::esz, kAllReduce, 4>, block, lds);
}

// Resident workgroups per CU for the stepwise kernels at this block/LDS size
// and group (64 lanes: the one-wave-per-rank variant).  The ring all-reduce
// kernel stands for its reduce-scatter and all-gather forms.
int stepwise_occupancy(bool ring, DType t, Op op, int block, size_t lds, int group) {
  const bool wave = group == 64;
  switch (t) {
    case DType::I32: return op == Op::Sum ? occupancy_t<DType::I32, Op::Sum>(ring, wave, block, lds, group)
                                          : occupancy_t<DType::I32, Op::Max>(ring, wave, block, lds, group);
    case DType::I64: return op == Op::Sum ? occupancy_t<DType::I64, Op::Sum>(ring, wave, block, lds, group)
                                          : occupancy_t<DType::I64, Op::Max>(ring, wave, block, lds, group);
    case DType::F32: return op == Op::Sum ? occupancy_t<DType::F32, Op::Sum>(ring, wave, block, lds, group)
                                          : occupancy_t<DType::F32, Op::Max>(ring, wave, block, lds, group);
    case DType::F16: return op == Op::Sum ? occupancy_t<DType::F16, Op::Sum>(ring, wave, block, lds, group)
                                          : occupancy_t<DType::F16, Op::Max>(ring, wave, block, lds, group);
    case DType::BF16: return op == Op::Sum ? occupancy_t<DType::BF16, Op::Sum>(ring, wave, block, lds, group)
                                           : occupancy_t<DType::BF16, Op::Max>(ring, wave, block, lds, group);
  }
  return 1;
}

}  // namespace emu
