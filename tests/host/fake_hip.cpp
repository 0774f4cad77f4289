// A host-only stand-in for the parts of the HIP runtime and of the kernel
// launchers that the library's host code (api.cpp) calls, so that its
// resource handling can be checked on a machine without a GPU.
//
// "Device" allocations are host memory, tracked one by one: a free of an
// unknown pointer, a copy or fill that leaves a live allocation (or the
// static scratch array), or a table pointer handed to a launcher outside
// live memory aborts with a message.  Launchers copy the tables they
// receive, so that a driver can compare what two entry points pass.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "common.h"
#include "fake_hip.h"
#include "xwg.h"

namespace {

std::map<const unsigned char*, size_t>& live() {
  static auto* m = new std::map<const unsigned char*, size_t>();
  return *m;
}

alignas(256) unsigned char g_scratch[EMU_NOALLOC_SCRATCH_BYTES];
bool g_scratch_seen = false;
size_t g_mallocs = 0;

[[noreturn]] void fail(const std::string& what) {
  std::fprintf(stderr, "fake HIP runtime: %s\n", what.c_str());
  std::abort();
}

// True if [p, p + n) lies inside one live allocation or the scratch array.
bool in_device_memory(const void* p, size_t n) {
  const unsigned char* q = static_cast<const unsigned char*>(p);
  if (q >= g_scratch && q + n <= g_scratch + sizeof(g_scratch)) return g_scratch_seen;
  auto it = live().upper_bound(q);
  if (it == live().begin()) return false;
  --it;
  return q >= it->first && q + n <= it->first + it->second;
}

void require(const void* p, size_t n, const char* what) {
  if (n == 0) return;
  if (!p || !in_device_memory(p, n)) fail(std::string("table outside device memory: ") + what);
}

std::vector<unsigned char> grab(const void* p, size_t n) {
  const unsigned char* q = static_cast<const unsigned char*>(p);
  return n ? std::vector<unsigned char>(q, q + n) : std::vector<unsigned char>();
}

}  // namespace

namespace fake {

std::vector<Launch> launches;

size_t live_allocations() { return live().size(); }
size_t live_bytes() {
  size_t b = 0;
  for (const auto& kv : live()) b += kv.second;
  return b;
}
size_t malloc_calls() { return g_mallocs; }

}  // namespace fake

extern "C" {

hipError_t hipMalloc(void** ptr, size_t size) {
  ++g_mallocs;
  const size_t n = (size + 255) / 256 * 256;
  void* p = std::aligned_alloc(256, n ? n : 256);
  if (!p) return hipErrorOutOfMemory;
  live()[static_cast<unsigned char*>(p)] = size;
  *ptr = p;
  return hipSuccess;
}

hipError_t hipFree(void* ptr) {
  if (!ptr) return hipSuccess;
  auto it = live().find(static_cast<unsigned char*>(ptr));
  if (it == live().end()) fail("hipFree of a pointer that is not a live allocation");
  live().erase(it);
  std::free(ptr);
  return hipSuccess;
}

hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind kind) {
  if (kind == hipMemcpyHostToDevice && !in_device_memory(dst, n)) fail("copy to the device outside device memory");
  if (kind == hipMemcpyDeviceToHost && !in_device_memory(src, n)) fail("copy from the device outside device memory");
  std::memcpy(dst, src, n);
  return hipSuccess;
}

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind kind, hipStream_t) {
  return hipMemcpy(dst, src, n, kind);
}

hipError_t hipMemset(void* dst, int value, size_t n) {
  if (!in_device_memory(dst, n)) fail("fill outside device memory");
  std::memset(dst, value, n);
  return hipSuccess;
}

hipError_t hipDeviceSynchronize(void) { return hipSuccess; }

hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int) {
  *v = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 160 * 1024;
  return hipSuccess;
}

}  // extern "C"

namespace emu {

hipError_t launch_fused(Coll coll, DType, Op, int mode, const FusedArgs& a, const Tile* tiles, const uint32_t* rows,
                        int grid, hipStream_t) {
  require(tiles, (size_t)a.ntiles * sizeof(Tile), "fused tiles");
  if (mode != kRotate) require(rows, sizeof(uint32_t), "fused order rows");
  if (grid < 1) fail("fused grid < 1");
  fake::launches.push_back({"fused", (int)coll, grab(tiles, (size_t)a.ntiles * sizeof(Tile))});
  return hipSuccess;
}
int fused_tile_vectors() { return 256; }

hipError_t launch_stepwise(Coll coll, bool ring, DType, Op, const StepArgs& a, int grid, int block, size_t,
                           hipStream_t) {
  const size_t task = ring ? sizeof(RingTask) : sizeof(TreeTask);
  require(a.tasks, a.ntasks * task, "stepwise tasks");
  require(a.table, ring ? sizeof(RingLoopBlock) : sizeof(TreeNode), "stepwise table");
  if (ring) require(a.orders, sizeof(uint32_t), "ring orders");
  if (grid < 1 || block < 64) fail("stepwise launch shape");
  fake::launches.push_back({ring ? "step_ring" : "step_tree", (int)coll, grab(a.tasks, a.ntasks * task)});
  return hipSuccess;
}
int stepwise_occupancy(bool, DType, Op, int, size_t, int) { return 2; }
int stepwise_vectors_per_lane(bool) { return 1; }

hipError_t launch_ll(bool ring, DType, Op, const StepArgs& a, uint32_t* status, uint32_t, int, int, size_t,
                     hipStream_t) {
  const size_t task = ring ? sizeof(RingTask) : sizeof(TreeTask);
  require(a.tasks, a.ntasks * task, "LL tasks");
  require(status, sizeof(uint32_t), "LL status word");
  fake::launches.push_back({ring ? "ll_ring" : "ll_tree", (int)kAllReduce, grab(a.tasks, a.ntasks * task)});
  return hipSuccess;
}
size_t ll_lds(bool ring, int n) { return (size_t)n * (ring ? 4096 : 8192); }
int ll_occupancy(bool, DType, Op, int, size_t) { return 2; }

hipError_t launch_xring(bool, DType, Op, const StepArgs&, const XArgs& x, const RingLoopBlock* loops,
                        const uint32_t* orders, int, hipStream_t) {
  require(loops, sizeof(RingLoopBlock), "xring loops");
  require(orders, sizeof(uint32_t), "xring orders");
  require(x.fifo, 16, "xring FIFOs");
  require(x.status, sizeof(uint32_t), "xring status word");
  fake::launches.push_back({"xring", (int)kAllReduce, {}});
  return hipSuccess;
}
int xring_threads() { return 256; }
int xring_slice_vectors(bool ll) { return 256 * (ll ? 2 : 8); }
int xring_capacity(bool, DType, Op, int cus) { return 2 * cus; }

hipError_t scratch_address(int, bool create, void** out) {
  *out = nullptr;
  if (!g_scratch_seen && !create) return hipSuccess;
  g_scratch_seen = true;
  *out = g_scratch;
  return hipSuccess;
}
size_t scratch_bytes() { return sizeof(g_scratch); }

hipError_t launch_stream(int kind, const void* src, void* dst, uint64_t bytes, uint32_t, int, hipStream_t) {
  if (kind != EMU_STREAM_WRITE) require(src, bytes, "stream source");
  require(dst, kind == EMU_STREAM_READ ? 16 : bytes, "stream destination");
  fake::launches.push_back({"stream", kind, {}});
  return hipSuccess;
}

}  // namespace emu
