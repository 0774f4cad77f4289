// Resource handling of the library's host code, linked against the host-only
// HIP stand-in (fake_hip.cpp): what emu_comm_destroy frees, and what
// dropping cached communicators frees.  Prints "ok" and
// exits 0, or names the first failed check and exits 1.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "emu_comm.h"
#include "fake_hip.h"

namespace {

int g_failed = 0;

#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      g_failed = 1;                                                        \
    }                                                                      \
  } while (0)

// Per-rank buffers: 16-byte aligned host memory standing in for the
// caller's device buffers (the library never dereferences them on the host).
struct Buffers {
  std::vector<void*> send, recv;
  Buffers(int n, size_t bytes) {
    for (int r = 0; r < n; ++r) {
      send.push_back(std::aligned_alloc(64, (bytes + 63) / 64 * 64 + 64));
      recv.push_back(std::aligned_alloc(64, (bytes + 63) / 64 * 64 + 64));
    }
  }
  ~Buffers() {
    for (void* p : send) std::free(p);
    for (void* p : recv) std::free(p);
  }
};

size_t lib_allocs() {
  size_t n = 0, b = 0;
  CHECK(emu_device_memory(&n, &b) == EMU_SUCCESS);
  CHECK(n == fake::live_allocations());
  CHECK(b == fake::live_bytes());
  return n;
}

// Every kind of call the library has, on one communicator each; returns
// with the library still holding their device memory.
void exercise_all_modes() {
  const int n = 8;
  const size_t count = (1 << 20) + 5;
  Buffers b(n, count * 4);
  Buffers rs(n, (size_t)n * 4096 * 4);
  struct Case { int algo; int expect_launch_kind; };
  const int algos[] = {EMU_ALGO_RING, EMU_ALGO_TREE, EMU_ALGO_RING | EMU_MODE_FUSED, EMU_ALGO_TREE | EMU_MODE_FUSED,
                       EMU_ALGO_RING | EMU_PROTO_LL, EMU_ALGO_TREE | EMU_PROTO_LL, EMU_ALGO_AUTO,
                       EMU_ALGO_RING | EMU_TRANSPORT_DEVICE, EMU_ALGO_RING | EMU_TRANSPORT_DEVICE | EMU_PROTO_LL};
  for (int algo : algos) {
    CHECK(emu_comm_init(n, 1, algo, 4, 64 << 10) == EMU_SUCCESS);
    const size_t before = fake::launches.size();
    CHECK(emu_allreduce(b.send.data(), b.recv.data(), count, EMU_FLOAT32, EMU_SUM, nullptr) == EMU_SUCCESS);
    CHECK(emu_allreduce(b.send.data(), b.send.data(), count, EMU_FLOAT32, EMU_SUM, nullptr) == EMU_SUCCESS);
    CHECK(emu_reduce_scatter(rs.send.data(), rs.recv.data(), 4096, EMU_FLOAT32, EMU_SUM, nullptr) == EMU_SUCCESS);
    CHECK(emu_all_gather(rs.recv.data(), rs.send.data(), 4096, EMU_FLOAT32, nullptr) == EMU_SUCCESS);
    CHECK(fake::launches.size() == before + 4);
  }
  int abandoned = -1;
  CHECK(emu_protocol_status(&abandoned) == EMU_SUCCESS && abandoned == 0);
}

void destroy_frees_everything() {
  exercise_all_modes();
  CHECK(lib_allocs() > 0);
  CHECK(emu_comm_destroy() == EMU_SUCCESS);
  CHECK(fake::live_allocations() == 0);
  CHECK(lib_allocs() == 0);
  // destroying twice, and using the library again afterwards
  CHECK(emu_comm_destroy() == EMU_SUCCESS);
  exercise_all_modes();
  CHECK(emu_comm_destroy() == EMU_SUCCESS);
  CHECK(fake::live_allocations() == 0);
}

void eviction_frees_dropped_communicators() {
  // more configurations than the cache keeps: the dropped ones are freed
  const size_t count = 4096;
  Buffers b(4, count * 4);
  for (int nch = 1; nch <= 40; ++nch) {
    CHECK(emu_comm_init(4, 1, EMU_ALGO_TREE | EMU_MODE_FUSED, nch, 4096) == EMU_SUCCESS);
    CHECK(emu_allreduce(b.send.data(), b.recv.data(), count, EMU_INT32, EMU_SUM, nullptr) == EMU_SUCCESS);
    CHECK(lib_allocs() <= 2 * 17);   // tiles and order rows of at most 17 communicators
  }
  CHECK(emu_comm_destroy() == EMU_SUCCESS);
  CHECK(fake::live_allocations() == 0);
}

}  // namespace

int main() {
  destroy_frees_everything();
  eviction_frees_dropped_communicators();
  if (g_failed) return 1;
  std::printf("ok\n");
  return 0;
}
