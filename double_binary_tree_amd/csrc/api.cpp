// C ABI of libemucomm: argument checks, the process-global communicator,
// per-shape plans (device tables), and kernel launches.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <tuple>
#include <vector>

#include "common.h"
#include "plan.h"
#include "topology.h"
#include "xwg.h"

namespace emu {

// Defined in fused.hip / stepwise.hip.
hipError_t launch_fused(Coll coll, DType t, Op op, int mode, const FusedArgs& a, const Tile* tiles,
                        const uint32_t* rows, int grid, hipStream_t stream);
int fused_tile_vectors();
hipError_t launch_stepwise(Coll coll, bool ring, DType t, Op op, const StepArgs& a, int grid, int block,
                           size_t lds, hipStream_t s);
int stepwise_occupancy(bool ring, DType t, Op op, int block, size_t lds, int group);
int stepwise_vectors_per_lane(bool ring);
// Defined in ll.hip.
hipError_t launch_ll(bool ring, DType t, Op op, const StepArgs& a, uint32_t* status, uint32_t spin_limit, int grid,
                     int block, size_t lds, hipStream_t s);
size_t ll_lds(bool ring, int n);
int ll_occupancy(bool ring, DType t, Op op, int block, size_t lds);
constexpr int kLLMaxRanks = 16;   // one wave per rank in one workgroup
// Defined in xwg.hip.
hipError_t launch_xring(bool ll, DType t, Op op, const StepArgs& a, const XArgs& x, const RingLoopBlock* loops,
                        const uint32_t* orders, int grid, hipStream_t s);
int xring_threads();
int xring_slice_vectors(bool ll);
int xring_capacity(bool ll, DType t, Op op, int cus);
constexpr size_t kXMaxWorkspace = (size_t)4 << 30;       // per communicator and device
// Defined in noalloc.hip: the static scratch array of the no-allocation
// entry point, its size, and its address on a device (looked up once per
// device; with create == false only reported if already looked up).
hipError_t scratch_address(int dev, bool create, void** out);
size_t scratch_bytes();
// Defined in stream.hip.
hipError_t launch_stream(int kind, const void* src, void* dst, uint64_t bytes, uint32_t key, int cus,
                         hipStream_t s);

namespace {

// Tuning knobs and test hooks from the environment.  They are read only
// when EMU_DEBUG is set (any value): without it every knob takes its
// built-in value, so a deployment's behaviour never depends on stray
// environment variables.
bool debug_env() {
  const char* v = std::getenv("EMU_DEBUG");
  return v && *v;
}

long env_long(const char* name, long fallback) {
  if (!debug_env()) return fallback;
  const char* v = std::getenv(name);
  if (!v || !*v) return fallback;
  char* end = nullptr;
  const long x = std::strtol(v, &end, 10);
  return (end && *end == '\0' && x > 0) ? x : fallback;
}

// As env_long, but 0 is a valid value.
long env_count(const char* name, long fallback) {
  if (!debug_env()) return fallback;
  const char* v = std::getenv(name);
  if (!v || !*v) return fallback;
  char* end = nullptr;
  const long x = std::strtol(v, &end, 10);
  return (end && *end == '\0' && x >= 0) ? x : fallback;
}

// Smallest k with 2^k >= x (x >= 1).
int ceil_log2(uint64_t x) {
  int k = 0;
  while (((uint64_t)1 << k) < x) ++k;
  return k;
}

// Every device allocation of the library goes through these two, which
// keep the count and size of what is live (emu_device_memory).
size_t g_live_allocs = 0, g_live_bytes = 0;

bool dev_alloc(void** p, size_t bytes) {
  *p = nullptr;
  if (hipMalloc(p, bytes) != hipSuccess) {
    *p = nullptr;
    return false;
  }
  ++g_live_allocs;
  g_live_bytes += bytes;
  return true;
}

void dev_free(void* p, size_t bytes) {
  if (!p) return;
  (void)hipFree(p);
  --g_live_allocs;
  g_live_bytes -= bytes;
}

struct DeviceBuffer {
  void* ptr = nullptr;
  size_t bytes = 0;
  DeviceBuffer() = default;
  DeviceBuffer(const DeviceBuffer&) = delete;
  DeviceBuffer& operator=(const DeviceBuffer&) = delete;
  ~DeviceBuffer() { dev_free(ptr, bytes); }
  int alloc(size_t n) {
    if (!dev_alloc(&ptr, n)) return EMU_ERR_HIP;
    bytes = n;
    return EMU_SUCCESS;
  }
  int upload(const void* src, size_t n) {
    if (n == 0) return EMU_SUCCESS;
    if (int e = alloc(n)) return e;
    if (hipMemcpy(ptr, src, n, hipMemcpyHostToDevice) != hipSuccess) return EMU_ERR_HIP;
    return EMU_SUCCESS;
  }
};

// The tables a launch reads, by role.
enum TableId : int { kTiles = 0, kRows, kTasks, kTable, kOrders, kXChan, kXSlices, kNumTables };

struct Plan {
  uint64_t serial = 0;        // unique per plan in the process
  // Host copy of every table (the no-allocation entry point copies them into
  // its static scratch); device copies are made on first use by the
  // allocating entry points.
  std::vector<unsigned char> host[kNumTables];
  DeviceBuffer dev[kNumTables];
  bool uploaded = false;
  // fused
  uint32_t ntiles = 0;
  int fused_grid = 0;
  // stepwise
  uint32_t ntasks = 0;
  int group = 0, block = 0, grid = 0;
  size_t lds = 0;
  uint32_t height = 0;
  bool dynamic = false;       // tree: short pieces, one workgroup each
  bool ll = false;            // runs the LL-protocol kernels (one workgroup)
  // stepwise ring across workgroups: xchan = [nch][2] loop ranges then [nch]
  // ring rows; xslices = slices per step, per loop
  bool xwg = false;

  template <class T>
  void keep(TableId id, const std::vector<T>& v) {
    const unsigned char* b = reinterpret_cast<const unsigned char*>(v.data());
    host[id].assign(b, b + v.size() * sizeof(T));
  }
  int upload() {
    if (uploaded) return EMU_SUCCESS;
    for (int i = 0; i < kNumTables; ++i)
      if (int e = dev[i].upload(host[i].data(), host[i].size())) return e;
    uploaded = true;
    return EMU_SUCCESS;
  }
};
uint64_t g_plan_serial = 0;

// FIFOs and counters of the cross-workgroup ring, per communicator and
// device: [fifo | tail counters | head counters | abandon word], all zero
// when created.
struct XWorkspace {
  DeviceBuffer mem;
  size_t bytes = 0, fifo_bytes = 0, counter_bytes = 0;
  uint32_t nslots = 0;
};

struct Comm {
  int nranks = 0, nnodes = 0, nchannels = 0;
  Algo algo = Algo::Ring;     // the fixed algorithm, or the ring for reduce-scatter / all-gather
  bool auto_algo = false;     // EMU_ALGO_AUTO: ring or tree per call, by the cost model
  bool fused = false;
  bool ll = false;            // stepwise all-reduce with the LL protocol
  bool xwg = false;           // stepwise ring all-reduce across workgroups (EMU_TRANSPORT_DEVICE)
  size_t chunk_bytes = 0;
  std::map<int, std::unique_ptr<XWorkspace>> xws;   // device -> workspace
  Topology topo;
  FusedOrders ring_orders;   // fused ring all-reduce and reduce-scatter: how each tile names its order
  FusedOrders tree_orders;   // fused tree all-reduce (built when the tree may run)
  // (device, count, dtype, op, collective, algo) -> plan
  std::map<std::tuple<int, uint64_t, int, int, int, int>, std::unique_ptr<Plan>> plans;
};

using CommKey = std::tuple<int, int, int, int, size_t, int, std::vector<int>>;
// The library's state lives on the heap and is never destroyed by the C++
// runtime.  A static destructor would run at process exit, after the HIP
// runtime (and any profiler attached to it) may already be torn down, and
// the hipFree calls of the device tables from there can crash the exiting
// process.  emu_comm_destroy releases everything; whatever is still held when
// the process ends is reclaimed with the process.
std::map<CommKey, std::unique_ptr<Comm>>& g_comms = *new std::map<CommKey, std::unique_ptr<Comm>>();
Comm* g_active = nullptr;
constexpr size_t kMaxCachedComms = 16;

std::map<int, int>& g_cu_count = *new std::map<int, int>();
std::map<int, size_t>& g_lds_limit = *new std::map<int, size_t>();
// Per device: the word an LL kernel sets when it abandons a call.
std::map<int, uint32_t*>& g_ll_status = *new std::map<int, uint32_t*>();

uint32_t* ll_status_word(int dev) {
  auto it = g_ll_status.find(dev);
  if (it != g_ll_status.end()) return it->second;
  void* p = nullptr;
  if (!dev_alloc(&p, sizeof(uint32_t))) return nullptr;
  if (hipMemset(p, 0, sizeof(uint32_t)) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    dev_free(p, sizeof(uint32_t));
    return nullptr;
  }
  g_ll_status[dev] = static_cast<uint32_t*>(p);
  return static_cast<uint32_t*>(p);
}

size_t lds_per_block(int dev) {
  auto it = g_lds_limit.find(dev);
  if (it != g_lds_limit.end()) return it->second;
  int bytes = 0;
  if (hipDeviceGetAttribute(&bytes, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || bytes <= 0)
    bytes = 65536;
  g_lds_limit[dev] = (size_t)bytes;
  return (size_t)bytes;
}

// Slices per ring step that a loop can need: a block holds at most
// chunk_bytes bytes and so spans at most chunk_bytes / slice bytes + 1 cells.
uint64_t xring_slice_bytes(const Comm& c) { return (uint64_t)xring_slice_vectors(c.ll) * kVecBytes; }
uint32_t xring_max_slices(const Comm& c) {
  return (uint32_t)((c.chunk_bytes + xring_slice_bytes(c) - 1) / xring_slice_bytes(c) + 1);
}

// The communicator's workspace on `dev`, created (zeroed) on first use.
// FIFO depth: two steps' worth of slices, so that a loop's first step can
// start while the previous loop drains (tuning override EMU_XWG_SLOTS, at
// least one step's worth).
int xring_workspace(Comm& c, int dev, XWorkspace** out) {
  auto it = c.xws.find(dev);
  if (it != c.xws.end()) {
    *out = it->second.get();
    return EMU_SUCCESS;
  }
  const uint32_t m = xring_max_slices(c);
  const uint64_t nslots = std::max<uint64_t>(m, (uint64_t)env_long("EMU_XWG_SLOTS", 2 * (long)m));
  const uint64_t nfifo = (uint64_t)c.nchannels * c.nranks;
  const uint64_t slot_bytes = (c.ll ? 2 : 1) * xring_slice_bytes(c);
  const uint64_t fifo_bytes = nfifo * nslots * slot_bytes;
  const uint64_t counter_bytes = nfifo * kXCounterStride * sizeof(uint32_t);
  const uint64_t bytes = fifo_bytes + 2 * counter_bytes + 256;
  if (nslots > UINT32_MAX || bytes > kXMaxWorkspace) return EMU_ERR_INVALID_ARGUMENT;
  auto w = std::make_unique<XWorkspace>();
  if (int e = w->mem.alloc(bytes)) return e;
  if (hipMemset(w->mem.ptr, 0, bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) return EMU_ERR_HIP;
  w->bytes = bytes;
  w->fifo_bytes = fifo_bytes;
  w->counter_bytes = counter_bytes;
  w->nslots = (uint32_t)nslots;
  *out = w.get();
  c.xws[dev] = std::move(w);
  return EMU_SUCCESS;
}

int cu_count(int dev) {
  auto it = g_cu_count.find(dev);
  if (it != g_cu_count.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  g_cu_count[dev] = cus;
  return cus;
}

// `count` is the elements per rank of the all-reduce, or the block size of
// the reduce-scatter / all-gather.
int make_plan(Comm& c, Coll coll, Algo algo, int dev, uint64_t count, DType t, Op op, Plan* p) {
  const int esz = elem_size(t);
  const uint64_t unit = kVecBytes / esz;
  const uint64_t chunk_count = c.chunk_bytes / esz;
  const int cus = cu_count(dev);
  if (c.xwg && coll == kAllReduce) {
    // One workgroup per (channel, ring position); all resident at once.
    p->xwg = true;
    const uint64_t slice_elems = (uint64_t)xring_slice_vectors(c.ll) * unit;
    if (count / slice_elems >= ((uint64_t)1 << 32)) return EMU_ERR_INVALID_ARGUMENT;   // cell index is 32-bit
    p->grid = c.nchannels * c.nranks;
    if (xring_capacity(c.ll, t, op, cus) < p->grid) return EMU_ERR_INVALID_ARGUMENT;
    XWorkspace* w = nullptr;
    if (int e = xring_workspace(c, dev, &w)) return e;
    std::vector<RingLoopBlock> loops;
    std::vector<RingTask> tasks;
    std::vector<uint32_t> orders;
    build_ring_tasks(c.topo, count, unit, chunk_count, slice_elems, &loops, &tasks, &orders);
    const size_t nloops = loops.size() / (size_t)c.nranks;
    std::vector<uint32_t> slices(nloops, 0);
    for (const RingTask& k : tasks) slices[k.loop] = k.nslices;
    for (uint32_t m : slices)
      if (m == 0 || m > w->nslots) return EMU_ERR_INTERNAL;
    std::vector<uint32_t> chan = ring_channel_loops(c.topo, count, unit, chunk_count);
    if (chan.size() != 2u * c.nchannels || (c.nchannels && chan.back() != nloops)) return EMU_ERR_INTERNAL;
    for (const ChannelTopology& ch : c.topo.channels) chan.push_back((uint32_t)ch.ring_id);
    p->keep(kTable, loops);
    p->keep(kOrders, orders);
    p->keep(kXChan, chan);
    p->keep(kXSlices, slices);
    p->block = xring_threads();
    return EMU_SUCCESS;
  }
  if (c.fused) {
    std::vector<Tile> tiles;
    const uint64_t tile_elems = (uint64_t)fused_tile_vectors() * unit;
    const FusedOrders& ord = algo == Algo::Ring ? c.ring_orders : c.tree_orders;
    if (coll == kAllReduce)
      build_fused_tiles(c.topo, algo, ord, count, unit, chunk_count, tile_elems, &tiles);
    else
      build_fused_coll_tiles(c.topo, coll, ord, count, unit, tile_elems, &tiles);
    p->ntiles = (uint32_t)tiles.size();
    p->keep(kTiles, tiles);
    p->keep(kRows, ord.rows);
    // One tile per workgroup: the hardware deals the workgroups out in
    // order, so the tiles in flight always form one window that slides over
    // the message.  Capping the grid (each workgroup walking several tiles
    // a grid apart) measured slower from 128 MiB per rank on MI355X (8 ranks
    // f32: 256 MiB 818 -> 763 us, 128 MiB 401 -> 379 us, smaller unchanged).
    // The dispatch holds the grid in work-items as a 32-bit count, so beyond
    // 2^22 tiles (8 GiB per rank) the workgroups walk the rest grid-strided.
    // Debug knob EMU_FUSED_BLOCKS_PER_CU caps the grid at that many per CU.
    constexpr uint64_t kMaxFusedGrid = (uint64_t)1 << 22;
    const long per_cu = env_long("EMU_FUSED_BLOCKS_PER_CU", 0);
    const uint64_t cap = per_cu > 0 ? std::min<uint64_t>(kMaxFusedGrid, (uint64_t)cus * per_cu) : kMaxFusedGrid;
    p->fused_grid = (int)std::max<uint64_t>(1, std::min<uint64_t>(p->ntiles, cap));
    return EMU_SUCCESS;
  }
  const int n = c.nranks;
  const bool ring = algo == Algo::Ring;
  // The LL protocol runs the all-reduce with one wave (64 lanes, one vector
  // each) per rank; reduce-scatter and all-gather keep the slot protocol.
  p->ll = c.ll && !c.xwg && coll == kAllReduce;
  const int vpl = p->ll ? 1 : stepwise_vectors_per_lane(ring);
  // Lanes per virtual rank: the widest group that fits one workgroup
  // (N*G <= 1024 threads) and the device's LDS per workgroup.
  const size_t lds_limit = lds_per_block(dev);
  // Lanes per rank: 64, 32 or 16 (one, two or four ranks per wave; 64 ranks
  // in 1024 threads need 16).  Debug knob EMU_STEP_GROUP.
  p->group = p->ll ? 64 : (int)env_long("EMU_STEP_GROUP", 64);
  if (p->group > 64 || p->group < 16 || (p->group & (p->group - 1))) p->group = 64;
  // LDS: ring 2 parities of slots plus 2 x N staged block descriptors and
  // 2 staged ring orders, tree 2 parities x (up, down) slots.
  auto lds_of = [&](int g) {
    if (p->ll) return ll_lds(ring, n);
    return (ring ? 2u : 4u) * (size_t)n * g * vpl * kVecBytes +
           (ring ? 2u * n * sizeof(RingLoopBlock) + 2u * kMaxRanks : 0u);
  };
  while (!p->ll && p->group > 16 && (n * p->group > 1024 || lds_of(p->group) > lds_limit)) p->group /= 2;
  if (n * p->group > 1024 || lds_of(p->group) > lds_limit) return EMU_ERR_INTERNAL;
  p->block = (n * p->group + 63) / 64 * 64;
  const uint64_t slice_elems = (uint64_t)p->group * vpl * unit;
  p->lds = lds_of(p->group);
  if (ring) {
    std::vector<RingLoopBlock> loops;
    std::vector<RingTask> tasks;
    std::vector<uint32_t> orders;
    // cell index is 32-bit
    const uint64_t span = coll == kAllReduce ? count : count * (uint64_t)n;
    if (span / slice_elems >= ((uint64_t)1 << 32)) return EMU_ERR_INVALID_ARGUMENT;
    if (coll == kAllReduce)
      build_ring_tasks(c.topo, count, unit, chunk_count, slice_elems, &loops, &tasks, &orders);
    else
      build_ring_coll_tasks(c.topo, count, unit, chunk_count, slice_elems, &loops, &tasks, &orders);
    p->ntasks = (uint32_t)tasks.size();
    p->keep(kTasks, tasks);
    p->keep(kTable, loops);
    p->keep(kOrders, orders);
  } else {
    const int occ_t = p->ll ? ll_occupancy(false, t, op, p->block, p->lds)
                            : stepwise_occupancy(false, t, op, p->block, p->lds, p->group);
    uint32_t h = 0;
    for (const auto& ch : c.topo.channels) h = std::max<uint32_t>(h, (uint32_t)ch.height);
    const uint64_t cells = (count + slice_elems - 1) / slice_elems;
    std::vector<TreeTask> tasks;
    std::vector<TreeNode> nodes;
    // One rank per wave, slot protocol, and a message of at least one full
    // round of resident workgroups at that length: short pieces of
    // max(8, 2^ceil(log2 H)) slices, one workgroup each, which the hardware
    // dispatches as slots free up.  Workgroups sharing a CU do not progress
    // evenly (the older ones are served first), so with one long piece per
    // resident workgroup the last quarter of the call ran with a CU's slots
    // emptying one by one (kernel timestamps: same-length pieces ending
    // between 98 and 205 us at 8 ranks x 64 MiB).  Short pieces keep every
    // slot busy to the end; their fill and drain overlap the steady stages
    // of the other workgroups.  Measured on MI355X against one piece per
    // resident workgroup (2 alternating rounds, 8 ranks f32 and 15/16 ranks
    // bf16): pieces of 8 slices 8-12% faster from 64 MiB per rank up at 8
    // ranks, 2% at 32, equal at 16, 6-7% on 15 and 16 ranks x 32 MiB; 4
    // slices 4-10% slower, 16 and 32 slices in between, lengths off a power
    // of two slower still.  The number of pieces is capped (128 per CU), so
    // the task table stays small; beyond that pieces grow, in powers of two.
    const uint64_t short_piece = std::max<uint64_t>(8, (uint64_t)1 << ceil_log2(std::max<uint32_t>(h, 1)));
    const uint64_t resident = (uint64_t)cus * (uint64_t)occ_t;
    p->dynamic = !p->ll && p->group == 64 && env_long("EMU_TREE_LONG_PIECES", 0) == 0 &&
                 cells >= short_piece * resident;
    if (p->dynamic) {
      const uint64_t cap = (uint64_t)cus * 128;
      const uint64_t piece = (uint64_t)1 << ceil_log2(std::max<uint64_t>(short_piece, (cells + cap - 1) / cap));
      build_tree_tasks(c.topo, count, unit, slice_elems, cells, &tasks, &nodes, piece);
    } else {
      // One pipeline per resident workgroup (tasks per CU = occupancy, or
      // the tuning override EMU_TREE_TASKS_PER_CU).
      const long per_cu = env_long("EMU_TREE_TASKS_PER_CU", occ_t);
      // Pieces of at least min_piece * H slices, as long as the message
      // still gives every CU a piece.  A piece pays 2H stages of fill and
      // drain, and one piece per resident workgroup leaves a small message's
      // pieces a slice or two each, so nearly every stage is fill or drain
      // while eight waves per SIMD contend to issue each stage's scalar-heavy
      // control.  Measured on MI355X (slot protocol, one rank per wave; 2
      // alternating rounds): pieces of at least H slices ran 8 ranks x 1 / 2
      // / 4 MiB in 11.6 / 16.3 / 20.9 us instead of 17.7 / 19.8 / 22.0 (16
      // ranks x 1 MiB: 12.3 against 19.0 us) and left 8 MiB and up unchanged;
      // 2H and longer were slower, as was any minimum with two ranks per wave
      // (17-32 ranks) or below one slice per CU.  Debug knob
      // EMU_TREE_PIECE_MIN.
      const long min_piece = env_count("EMU_TREE_PIECE_MIN", !p->ll && p->group == 64 ? 1 : 0);
      const uint64_t min_cells =
          min_piece > 0 ? std::min<uint64_t>((uint64_t)min_piece * std::max<uint32_t>(h, 1), (cells + cus - 1) / cus)
                        : 1;
      build_tree_tasks(c.topo, count, unit, slice_elems, (uint64_t)cus * per_cu, &tasks, &nodes, min_cells);
    }
    p->ntasks = (uint32_t)tasks.size();
    p->height = h;
    p->keep(kTasks, tasks);
    p->keep(kTable, nodes);
  }
  const int occ = p->ll ? ll_occupancy(ring, t, op, p->block, p->lds)
                        : stepwise_occupancy(ring, t, op, p->block, p->lds, p->group);
  // Short tree pieces: one workgroup per piece (the hardware balances the
  // CUs); otherwise at most the resident workgroups, each looping over tasks.
  p->grid = (int)std::max<uint64_t>(1, p->dynamic ? p->ntasks : std::min<uint64_t>(p->ntasks, (uint64_t)cus * occ));
  // Stepwise ring with at least 12 tasks per resident workgroup: one
  // workgroup per task.  Workgroups sharing a CU progress unevenly and a
  // long task list per workgroup lets the gap grow (kernel timestamps, 8
  // ranks x 256 MiB: workgroups of 32 tasks each ending between 680 and
  // 836 us); one task each lets the hardware balance the CUs, at the cost
  // of a workgroup start per task.  Measured on MI355X (2 alternating
  // rounds): 8 ranks x 96 / 128 / 256 MiB 2 / 5 / 6% faster, 16 ranks bf16
  // x 128 MiB 6%, 32 ranks f16 x 64 MiB 3%; at 8 tasks per workgroup
  // (8 ranks x 64 MiB) 1% slower, so shorter lists keep the loop (as do the
  // standalone reduce-scatter and all-gather, not measured so).
  if (ring && coll == kAllReduce && !p->ll && p->ntasks >= 12 * (uint64_t)p->grid && p->ntasks <= 0x7fffffffu)
    p->grid = (int)p->ntasks;
  return EMU_SUCCESS;
}

// Cost model (page "NCCL 专家课程 13", section "理想成本模型"; page "all-reduce
// 每张卡要发多少数据?", section "α–β 模型"): per mode and algorithm, alpha
// (us per dependent stage, the fixed cost of a call folded in) and the
// bandwidth B (bytes/us).  Predicted time of S bytes per rank:
//   ring 2(N-1)*alpha + 2(N-1)/N * S/B,   tree 2*D*alpha + 2*S/B,
// D the deepest channel tree.  The parameters are kept per rank-count
// class, since the emulation's cost per stage and per byte changes with N
// (one, two or four virtual ranks per wave; deeper trees): classes are
// centred on the measured 8, 16 and 32 ranks, with boundaries at their
// geometric midpoints.
constexpr int kCostClasses = 3;
int cost_class(int nranks) { return nranks * nranks <= 128 ? 0 : nranks * nranks <= 512 ? 1 : 2; }
struct Cost { double alpha_us, bw; };
// Defaults: least-squares fits to message-size sweeps measured on MI355X
// (graph-replayed launches, library buffer placement): 8 ranks on one node,
// f32, 12 channels; 16 ranks on 16 nodes, bf16, 8 channels; 4 x 8 ranks,
// f16, 16 channels.  The points are kept in the repository's profiles
// (sweep_points.txt); `costfit profiles/sweep_points.txt --defaults`
// prints this table.
Cost g_cost[kCostClasses][2][2] = {   // [class][stepwise, fused][ring, tree]: {alpha us, bytes/us}
    {{{0.567544, 671660}, {0.449822, 741354}}, {{0.191954, 668336}, {0.165805, 824927}}},   // 8 ranks
    {{{0.583629, 463726}, {0.815003, 407189}}, {{0.122226, 422618}, {0.63201, 462468}}},    // 16 ranks
    {{{0.630384, 233903}, {0.705246, 177256}}, {{0.0688502, 197104}, {0.388422, 218334}}},  // 32 ranks
};

double predict_us(const Comm& c, bool fused, Algo algo, double nbytes) {
  const int n = c.nranks;
  const Cost& k = g_cost[cost_class(n)][fused ? 1 : 0][algo == Algo::Ring ? 0 : 1];
  if (algo == Algo::Ring) return (double)(2 * (n - 1)) * k.alpha_us + 2.0 * (n - 1) / n * nbytes / k.bw;
  int depth = 0;
  for (const auto& ch : c.topo.channels) depth = std::max(depth, ch.height);
  return (double)(2 * depth) * k.alpha_us + 2.0 * nbytes / k.bw;
}

// The smaller predicted time; the ring on an exact tie.
Algo select_algo(const Comm& c, double nbytes) {
  return predict_us(c, c.fused, Algo::Tree, nbytes) < predict_us(c, c.fused, Algo::Ring, nbytes) ? Algo::Tree
                                                                                                  : Algo::Ring;
}

bool valid_dtype(int d) { return d >= EMU_INT32 && d <= EMU_BFLOAT16; }
bool valid_op(int o) { return o == EMU_SUM || o == EMU_MAX; }

}  // namespace
}  // namespace emu

using namespace emu;

extern "C" {

int emu_comm_init_graph(int nranks, int nnodes, int algo, int nchannels, size_t chunk_bytes, int pattern,
                        const int* intra) {
  const int base = algo & 0xFF;
  const int mode = algo & ~0xFF & ~EMU_PROTO_LL & ~EMU_TRANSPORT_DEVICE;
  const bool ll = (algo & EMU_PROTO_LL) != 0;
  const bool xwg = (algo & EMU_TRANSPORT_DEVICE) != 0;
  if (base != EMU_ALGO_RING && base != EMU_ALGO_TREE && base != EMU_ALGO_AUTO) return EMU_ERR_INVALID_ARGUMENT;
  if (mode != EMU_MODE_STEPWISE && mode != EMU_MODE_FUSED) return EMU_ERR_INVALID_ARGUMENT;
  if (xwg && (mode == EMU_MODE_FUSED || base != EMU_ALGO_RING)) return EMU_ERR_INVALID_ARGUMENT;
  if (ll && !xwg && (mode == EMU_MODE_FUSED || nranks > kLLMaxRanks)) return EMU_ERR_INVALID_ARGUMENT;
  if (chunk_bytes == 0 || chunk_bytes % kVecBytes != 0 || chunk_bytes > ((size_t)1 << 30))
    return EMU_ERR_INVALID_ARGUMENT;
  if (nranks < 1 || nranks > kMaxRanks || nnodes < 1 || nranks % nnodes != 0 || nchannels < 1 ||
      nchannels > kMaxChannels)
    return EMU_ERR_INVALID_ARGUMENT;
  // The key holds the orders as given (identity when intra is NULL), so
  // equal graphs share one cached communicator.
  std::vector<int> order((size_t)nchannels * nranks);
  for (size_t i = 0; i < order.size(); ++i) order[i] = intra ? intra[i] : (int)(i % nranks);
  const CommKey key{nranks, nnodes, algo, nchannels, chunk_bytes, pattern, order};
  auto it = g_comms.find(key);
  if (it != g_comms.end()) {
    g_active = it->second.get();
    return EMU_SUCCESS;
  }
  auto c = std::make_unique<Comm>();
  c->nranks = nranks;
  c->nnodes = nnodes;
  c->nchannels = nchannels;
  c->algo = base == EMU_ALGO_TREE ? Algo::Tree : Algo::Ring;
  c->auto_algo = base == EMU_ALGO_AUTO;
  c->fused = mode == EMU_MODE_FUSED;
  c->ll = ll;
  c->xwg = xwg;
  c->chunk_bytes = chunk_bytes;
  if (int e = build_topology(nranks, nnodes, nchannels, pattern, order.data(), &c->topo)) return e;
  if (int e = build_fused_orders(c->topo, Algo::Ring, &c->ring_orders)) return e;
  if (base != EMU_ALGO_RING)
    if (int e = build_fused_orders(c->topo, Algo::Tree, &c->tree_orders)) return e;
  if (g_comms.size() >= kMaxCachedComms) {
    // Drop every cached communicator except the active one.  Their device
    // tables may still be read by enqueued kernels: wait for the device first.
    bool has_plans = false;
    for (const auto& kv : g_comms) has_plans = has_plans || !kv.second->plans.empty();
    if (has_plans) (void)hipDeviceSynchronize();
    for (auto i = g_comms.begin(); i != g_comms.end();) {
      if (i->second.get() == g_active) ++i;
      else i = g_comms.erase(i);
    }
  }
  g_active = c.get();
  g_comms[key] = std::move(c);
  return EMU_SUCCESS;
}

int emu_comm_init(int nranks, int nnodes, int algo, int nchannels, size_t chunk_bytes) {
  return emu_comm_init_graph(nranks, nnodes, algo, nchannels, chunk_bytes, EMU_PATTERN_TREE, nullptr);
}

}  // extern "C"

namespace emu {
namespace {

// The no-allocation entry point keeps its tables in a static device array
// (noalloc.hip), one per device: [status word | tables, each 256-byte
// aligned].  Per device, the serial of the plan whose tables it holds.
constexpr size_t kScratchAlign = 256;
std::map<int, uint64_t>& g_scratch_serial = *new std::map<int, uint64_t>();

// Device addresses of the tables one launch reads.
struct Tables {
  const void* t[kNumTables] = {};
  uint32_t* status = nullptr;   // LL / device-transport abandon word
};

// Points `tb` at the plan's tables in the scratch array of `dev`, copying
// them there (stream-ordered on `s`) unless the array already holds them.
int stage_scratch(const Plan& p, int dev, hipStream_t s, Tables* tb) {
  void* base = nullptr;
  if (scratch_address(dev, true, &base) != hipSuccess || !base) return EMU_ERR_HIP;
  size_t off[kNumTables];
  size_t end = kScratchAlign;   // the status word sits at offset 0
  for (int i = 0; i < kNumTables; ++i) {
    off[i] = end;
    end += (p.host[i].size() + kScratchAlign - 1) / kScratchAlign * kScratchAlign;
  }
  if (end > scratch_bytes()) return EMU_ERR_INVALID_ARGUMENT;
  unsigned char* b = static_cast<unsigned char*>(base);
  auto it = g_scratch_serial.find(dev);
  if (it == g_scratch_serial.end() || it->second != p.serial) {
    g_scratch_serial[dev] = 0;   // no plan until every copy is enqueued
    for (int i = 0; i < kNumTables; ++i) {
      if (p.host[i].empty()) continue;
      if (hipMemcpyAsync(b + off[i], p.host[i].data(), p.host[i].size(), hipMemcpyHostToDevice, s) != hipSuccess)
        return EMU_ERR_HIP;
    }
    g_scratch_serial[dev] = p.serial;
  }
  for (int i = 0; i < kNumTables; ++i) tb->t[i] = p.host[i].empty() ? nullptr : b + off[i];
  tb->status = reinterpret_cast<uint32_t*>(b);
  return EMU_SUCCESS;
}

// Shared by the collectives: argument checks (before anything is enqueued),
// plan lookup, launch.  Rank r's send buffer holds send_elems elements and
// its receive buffer recv_elems; `count` is the all-reduce count or the
// block size.  In place means recvbufs[r] == sendbufs[r] + inplace_off
// elements (0 for the all-reduce, r*count for reduce-scatter); for
// all-gather, sendbufs[r] == recvbufs[r] + r*count.  `noalloc`: the tables
// go to the static scratch array and nothing is allocated on the device.
int run_collective(Coll coll, const void* const sendbufs[], void* const recvbufs[], size_t count, int dtype,
                   int op, void* stream, bool noalloc = false) {
  Comm* c = g_active;
  if (!c) return EMU_ERR_NOT_INITIALIZED;
  if (!valid_dtype(dtype) || !valid_op(op) || !sendbufs || !recvbufs) return EMU_ERR_INVALID_ARGUMENT;
  // the device transport's FIFOs are far larger than the scratch array
  if (noalloc && c->xwg) return EMU_ERR_INVALID_ARGUMENT;
  const DType t = static_cast<DType>(dtype);
  const Op o = static_cast<Op>(op);
  const int n = c->nranks;
  const size_t esz = (size_t)elem_size(t);
  const uint64_t limit = ((uint64_t)1 << 40) / esz;
  if (count > limit || (coll != kAllReduce && count > limit / (uint64_t)n)) return EMU_ERR_INVALID_ARGUMENT;
  // blocks of reduce-scatter / all-gather sit at multiples of count: keep
  // them 16-byte aligned
  if (coll != kAllReduce && (count * esz) % kVecBytes) return EMU_ERR_INVALID_ARGUMENT;
  const uint64_t send_bytes = (coll == kReduceScatter ? (uint64_t)n : 1) * count * esz;
  const uint64_t recv_bytes = (coll == kAllGather ? (uint64_t)n : 1) * count * esz;
  for (int r = 0; r < n; ++r) {
    if (!sendbufs[r] || !recvbufs[r]) return EMU_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)sendbufs[r] | (uintptr_t)recvbufs[r]) % kVecBytes) return EMU_ERR_INVALID_ARGUMENT;
  }
  if (count == 0) return EMU_SUCCESS;
  // No two distinct buffers may overlap, except a rank's in-place pair.
  struct Span { uintptr_t lo, hi; };
  std::vector<Span> spans;
  for (int r = 0; r < n; ++r) {
    const uintptr_t s0 = (uintptr_t)sendbufs[r], r0 = (uintptr_t)recvbufs[r];
    bool inplace = false;
    if (coll == kAllReduce) inplace = s0 == r0;
    else if (coll == kReduceScatter) inplace = r0 == s0 + (uint64_t)r * count * esz;
    else inplace = s0 == r0 + (uint64_t)r * count * esz;
    if (inplace) {
      spans.push_back({std::min(s0, r0), std::max(s0 + send_bytes, r0 + recv_bytes)});
    } else {
      spans.push_back({s0, s0 + send_bytes});
      spans.push_back({r0, r0 + recv_bytes});
    }
  }
  std::sort(spans.begin(), spans.end(), [](const Span& x, const Span& y) { return x.lo < y.lo; });
  for (size_t i = 1; i < spans.size(); ++i)
    if (spans[i].lo < spans[i - 1].hi) return EMU_ERR_INVALID_ARGUMENT;

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return EMU_ERR_HIP;
  const Algo algo = coll != kAllReduce ? Algo::Ring
                    : c->auto_algo      ? select_algo(*c, (double)count * (double)esz)
                                        : c->algo;
  const int op_key = (c->fused && coll == kAllReduce) || coll == kAllGather ? 0 : op;
  const auto key = std::make_tuple(dev, (uint64_t)count, coll == kAllGather ? elem_size(t) : dtype, op_key, (int)coll,
                                   (int)algo);
  auto it = c->plans.find(key);
  if (it == c->plans.end()) {
    auto p = std::make_unique<Plan>();
    p->serial = ++g_plan_serial;
    if (int e = make_plan(*c, coll, algo, dev, count, t, o, p.get())) return e;
    it = c->plans.emplace(key, std::move(p)).first;
  }
  Plan& p = *it->second;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Tables tb;
  if (noalloc) {
    if (int e = stage_scratch(p, dev, s, &tb)) return e;
  } else {
    if (int e = p.upload()) return e;
    for (int i = 0; i < kNumTables; ++i) tb.t[i] = p.dev[i].ptr;
    if (p.ll || p.xwg) {
      tb.status = ll_status_word(dev);
      if (!tb.status) return EMU_ERR_HIP;
    }
  }
  hipError_t err;
  if (c->fused) {
    FusedArgs a{};
    const FusedOrders& ord = algo == Algo::Ring ? c->ring_orders : c->tree_orders;
    for (int r = 0; r < n; ++r) {
      // kRotate folds pointer j as the j-th rank of the shared order
      const bool rotate = ord.mode == kRotate && coll != kAllGather;
      a.send[r] = sendbufs[rotate ? ord.rotate_perm[r] : r];
      a.recv[r] = recvbufs[r];
    }
    a.block_bytes = (uint64_t)count * esz;
    a.ntiles = p.ntiles;
    a.nranks = (uint32_t)n;
    // Each XCD takes a contiguous run of tiles from 12 ranks up.  Measured
    // on MI355X (fused, full-size workloads): 15, 16 and 32 ranks gain up to
    // 20% with buffers where torch places them and stay within 2% with the
    // staggered layout; 8 ranks lose 4-8% either way.  Debug knob
    // EMU_FUSED_XCD_RUNS: 1 off, 2 on.
    a.xcd_runs = env_long("EMU_FUSED_XCD_RUNS", n >= 12 ? 2 : 1) == 2 ? 1 : 0;
    err = launch_fused(coll, t, o, ord.mode, a, static_cast<const Tile*>(tb.t[kTiles]),
                       static_cast<const uint32_t*>(tb.t[kRows]), p.fused_grid, s);
  } else {
    StepArgs a{};
    for (int r = 0; r < n; ++r) { a.send[r] = sendbufs[r]; a.recv[r] = recvbufs[r]; }
    a.tasks = tb.t[kTasks];
    a.table = tb.t[kTable];
    a.orders = static_cast<const uint32_t*>(tb.t[kOrders]);
    a.count = count;
    a.block = count;
    a.ntasks = p.ntasks;
    a.nranks = (uint32_t)n;
    a.group = (uint32_t)p.group;
    a.height = p.height;
    if (p.xwg) {
      const XWorkspace& w = *c->xws.at(dev);
      char* base = static_cast<char*>(w.mem.ptr);
      const uint32_t* chan = static_cast<const uint32_t*>(tb.t[kXChan]);
      XArgs x{};
      x.chan_loops = chan;
      x.chan_ring = chan + 2 * c->nchannels;
      x.loop_slices = static_cast<const uint32_t*>(tb.t[kXSlices]);
      x.fifo = base;
      x.tail = reinterpret_cast<uint32_t*>(base + w.fifo_bytes);
      x.head = reinterpret_cast<uint32_t*>(base + w.fifo_bytes + w.counter_bytes);
      x.abandon = reinterpret_cast<uint32_t*>(base + w.fifo_bytes + 2 * w.counter_bytes);
      x.status = tb.status;
      x.nslots = w.nslots;
      // polls before a wait is abandoned; the debug hook EMU_XWG_SPIN_LIMIT
      // lowers it so that tests can force the abandon path from the host
      x.spin_limit = (uint32_t)env_count("EMU_XWG_SPIN_LIMIT", 1L << 22);
      err = launch_xring(c->ll, t, o, a, x, static_cast<const RingLoopBlock*>(tb.t[kTable]),
                         static_cast<const uint32_t*>(tb.t[kOrders]), p.grid, s);
    } else if (p.ll) {
      // polls before a wait is abandoned; the debug hook EMU_LL_SPIN_LIMIT
      // lowers it so that tests can force the abandon path from the host
      const uint32_t spin = (uint32_t)env_count("EMU_LL_SPIN_LIMIT", 1L << 22);
      err = launch_ll(algo == Algo::Ring, t, o, a, tb.status, spin, p.grid, p.block, p.lds, s);
    } else {
      err = launch_stepwise(coll, algo == Algo::Ring, t, o, a, p.grid, p.block, p.lds, s);
    }
  }
  return err == hipSuccess ? EMU_SUCCESS : EMU_ERR_HIP;
}

}  // namespace
}  // namespace emu

extern "C" {

int emu_allreduce(const void* const sendbufs[], void* const recvbufs[], size_t count, int dtype, int op,
                  void* stream) {
  return run_collective(kAllReduce, sendbufs, recvbufs, count, dtype, op, stream);
}

int emu_allreduce_noalloc(const void* const sendbufs[], void* const recvbufs[], size_t count, int dtype, int op,
                          void* stream) {
  return run_collective(kAllReduce, sendbufs, recvbufs, count, dtype, op, stream, true);
}

int emu_reduce_scatter(const void* const sendbufs[], void* const recvbufs[], size_t recvcount, int dtype, int op,
                       void* stream) {
  return run_collective(kReduceScatter, sendbufs, recvbufs, recvcount, dtype, op, stream);
}

int emu_all_gather(const void* const sendbufs[], void* const recvbufs[], size_t sendcount, int dtype,
                   void* stream) {
  return run_collective(kAllGather, sendbufs, recvbufs, sendcount, dtype, EMU_SUM, stream);
}

int emu_set_cost_model_ranks(int algo, int nranks, double alpha_us, double bw_bytes_per_us) {
  const int base = algo & 0xFF, mode = algo & ~0xFF;
  if ((base != EMU_ALGO_RING && base != EMU_ALGO_TREE) || (mode != EMU_MODE_STEPWISE && mode != EMU_MODE_FUSED))
    return EMU_ERR_INVALID_ARGUMENT;
  if (nranks != 0 && (nranks < 1 || nranks > kMaxRanks)) return EMU_ERR_INVALID_ARGUMENT;
  if (!(alpha_us >= 0.0) || !(bw_bytes_per_us > 0.0) || alpha_us > 1e9 || bw_bytes_per_us > 1e15)
    return EMU_ERR_INVALID_ARGUMENT;
  for (int k = 0; k < kCostClasses; ++k)
    if (nranks == 0 || k == cost_class(nranks))
      g_cost[k][mode == EMU_MODE_FUSED ? 1 : 0][base == EMU_ALGO_RING ? 0 : 1] = {alpha_us, bw_bytes_per_us};
  return EMU_SUCCESS;
}

int emu_set_cost_model(int algo, double alpha_us, double bw_bytes_per_us) {
  return emu_set_cost_model_ranks(algo, 0, alpha_us, bw_bytes_per_us);
}

int emu_get_cost_model(int algo, int nranks, double* alpha_us, double* bw_bytes_per_us) {
  const int base = algo & 0xFF, mode = algo & ~0xFF;
  if ((base != EMU_ALGO_RING && base != EMU_ALGO_TREE) || (mode != EMU_MODE_STEPWISE && mode != EMU_MODE_FUSED))
    return EMU_ERR_INVALID_ARGUMENT;
  if (nranks < 1 || nranks > kMaxRanks || !alpha_us || !bw_bytes_per_us) return EMU_ERR_INVALID_ARGUMENT;
  const Cost& k = g_cost[cost_class(nranks)][mode == EMU_MODE_FUSED ? 1 : 0][base == EMU_ALGO_RING ? 0 : 1];
  *alpha_us = k.alpha_us;
  *bw_bytes_per_us = k.bw;
  return EMU_SUCCESS;
}

int emu_predict_us(int algo, size_t count, int dtype, double* us) {
  const Comm* c = g_active;
  if (!c) return EMU_ERR_NOT_INITIALIZED;
  const int base = algo & 0xFF, mode = algo & ~0xFF;
  if ((base != EMU_ALGO_RING && base != EMU_ALGO_TREE) || (mode != EMU_MODE_STEPWISE && mode != EMU_MODE_FUSED) ||
      !valid_dtype(dtype) || !us)
    return EMU_ERR_INVALID_ARGUMENT;
  *us = predict_us(*c, mode == EMU_MODE_FUSED, base == EMU_ALGO_RING ? Algo::Ring : Algo::Tree,
                   (double)count * (double)elem_size(static_cast<DType>(dtype)));
  return EMU_SUCCESS;
}

int emu_select_algo(size_t count, int dtype, int* algo) {
  const Comm* c = g_active;
  if (!c) return EMU_ERR_NOT_INITIALIZED;
  if (!valid_dtype(dtype) || !algo) return EMU_ERR_INVALID_ARGUMENT;
  const Algo a = c->auto_algo ? select_algo(*c, (double)count * (double)elem_size(static_cast<DType>(dtype))) : c->algo;
  *algo = a == Algo::Ring ? EMU_ALGO_RING : EMU_ALGO_TREE;
  return EMU_SUCCESS;
}

int emu_tree_topology(int channel, int rank, int* up, int down[3]) {
  const Comm* c = g_active;
  if (!c) return EMU_ERR_NOT_INITIALIZED;
  if (!up || !down || channel < 0 || channel >= c->nchannels || rank < 0 || rank >= c->nranks)
    return EMU_ERR_INVALID_ARGUMENT;
  const RankRecord& rec = c->topo.channels[channel].ranks[rank];
  *up = rec.up;
  for (int s = 0; s < 3; ++s) down[s] = rec.down[s];
  return EMU_SUCCESS;
}

int emu_tree_depth(int* depth) {
  const Comm* c = g_active;
  if (!c) return EMU_ERR_NOT_INITIALIZED;
  if (!depth) return EMU_ERR_INVALID_ARGUMENT;
  *depth = c->topo.depth_approx;
  return EMU_SUCCESS;
}

int emu_comm_destroy(void) {
  bool has_plans = !g_ll_status.empty();
  for (const auto& kv : g_comms) has_plans = has_plans || !kv.second->plans.empty();
  if (has_plans) (void)hipDeviceSynchronize();
  g_active = nullptr;
  g_comms.clear();
  for (auto& kv : g_ll_status) dev_free(kv.second, sizeof(uint32_t));
  g_ll_status.clear();
  return EMU_SUCCESS;
}

int emu_device_memory(size_t* allocations, size_t* bytes) {
  if (!allocations || !bytes) return EMU_ERR_INVALID_ARGUMENT;
  *allocations = g_live_allocs;
  *bytes = g_live_bytes;
  return EMU_SUCCESS;
}

int emu_buffer_layout(size_t nbufs, size_t bytes, size_t offsets[], size_t* pool_bytes) {
  constexpr size_t kSlotAlign = (size_t)64 << 10, kStagger = (size_t)6 << 10;
  if (nbufs == 0 || !offsets || !pool_bytes) return EMU_ERR_INVALID_ARGUMENT;
  if (bytes > SIZE_MAX - 2 * kSlotAlign) return EMU_ERR_INVALID_ARGUMENT;
  const size_t slot = (bytes + kSlotAlign - 1) / kSlotAlign * kSlotAlign + kStagger;
  if (nbufs > SIZE_MAX / slot) return EMU_ERR_INVALID_ARGUMENT;
  for (size_t i = 0; i < nbufs; ++i) offsets[i] = i * slot;
  *pool_bytes = nbufs * slot;
  return EMU_SUCCESS;
}

int emu_protocol_status(int* abandoned) {
  if (!abandoned) return EMU_ERR_INVALID_ARGUMENT;
  *abandoned = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return EMU_ERR_HIP;
  auto it = g_ll_status.find(dev);
  void* scratch = nullptr;
  (void)scratch_address(dev, false, &scratch);
  if (it == g_ll_status.end() && !scratch) return EMU_SUCCESS;
  if (hipDeviceSynchronize() != hipSuccess) return EMU_ERR_HIP;
  uint32_t v = 0;
  if (scratch) {
    // the no-allocation entry point's LL calls report in the scratch array
    if (hipMemcpy(&v, scratch, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return EMU_ERR_HIP;
    if (v && hipMemset(scratch, 0, sizeof(uint32_t)) != hipSuccess) return EMU_ERR_HIP;
  }
  if (it != g_ll_status.end()) {
    uint32_t w = 0;
    if (hipMemcpy(&w, it->second, sizeof(w), hipMemcpyDeviceToHost) != hipSuccess) return EMU_ERR_HIP;
    if (w && hipMemset(it->second, 0, sizeof(uint32_t)) != hipSuccess) return EMU_ERR_HIP;
    v |= w;
  }
  if (v) {
    // An abandoned cross-workgroup call leaves its FIFO counters mismatched:
    // clear every such workspace on the device with the status word.
    for (const auto& kv : g_comms) {
      auto w = kv.second->xws.find(dev);
      if (w != kv.second->xws.end() && hipMemset(w->second->mem.ptr, 0, w->second->bytes) != hipSuccess)
        return EMU_ERR_HIP;
    }
    if (hipDeviceSynchronize() != hipSuccess) return EMU_ERR_HIP;
  }
  *abandoned = v ? 1 : 0;
  return EMU_SUCCESS;
}

int emu_stream_probe(int kind, const void* src, void* dst, size_t bytes, void* stream) {
  if (kind != EMU_STREAM_READ && kind != EMU_STREAM_WRITE && kind != EMU_STREAM_COPY) return EMU_ERR_INVALID_ARGUMENT;
  if (bytes % kVecBytes) return EMU_ERR_INVALID_ARGUMENT;
  const bool reads = kind != EMU_STREAM_WRITE;
  if (!dst || (uintptr_t)dst % kVecBytes) return EMU_ERR_INVALID_ARGUMENT;
  if (reads && (!src || (uintptr_t)src % kVecBytes)) return EMU_ERR_INVALID_ARGUMENT;
  if (kind == EMU_STREAM_COPY) {
    const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
    if (a < b + bytes && b < a + bytes) return EMU_ERR_INVALID_ARGUMENT;
  }
  if (bytes == 0) return EMU_SUCCESS;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return EMU_ERR_HIP;
  const uint32_t key = 0x9E3779B9u ^ (uint32_t)(bytes >> 4);
  return launch_stream(kind, src, dst, bytes, key, cu_count(dev), static_cast<hipStream_t>(stream)) == hipSuccess
             ? EMU_SUCCESS
             : EMU_ERR_HIP;
}

const char* emu_strerror(int code) {
  switch (code) {
    case EMU_SUCCESS: return "success";
    case EMU_ERR_INVALID_ARGUMENT: return "invalid argument";
    case EMU_ERR_NOT_INITIALIZED: return "communicator not initialized";
    case EMU_ERR_INTERNAL: return "internal error (topology or program check failed)";
    case EMU_ERR_HIP: return "HIP runtime error (allocation, copy or launch)";
    default: return "unknown error code";
  }
}

}  // extern "C"
