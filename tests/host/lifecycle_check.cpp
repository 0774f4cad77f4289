// Resource handling of the library's host code, linked against the host-only
// HIP stand-in (fake_hip.cpp): what emu_comm_destroy frees, what the
// no-allocation all-reduce allocates (nothing) and passes to its kernels
// (the same tables as emu_allreduce), and what it refuses.  Prints "ok" and
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

// The tables the last launch received.
std::vector<unsigned char> last_tables() { return fake::launches.back().tasks; }

void noalloc_allocates_nothing_and_passes_the_same_tables() {
  const int n = 8;
  const int algos[] = {EMU_ALGO_RING | EMU_MODE_FUSED, EMU_ALGO_TREE | EMU_MODE_FUSED, EMU_ALGO_RING,
                       EMU_ALGO_TREE, EMU_ALGO_RING | EMU_PROTO_LL, EMU_ALGO_TREE | EMU_PROTO_LL};
  const size_t counts[] = {(1 << 20) + 5, 4099, 77777};
  Buffers b(n, counts[0] * 8);
  for (int algo : algos) {
    // reference tables from the allocating entry point, per shape
    std::vector<std::vector<unsigned char>> ref;
    CHECK(emu_comm_destroy() == EMU_SUCCESS);
    CHECK(emu_comm_init(n, 2, algo, 5, 32 << 10) == EMU_SUCCESS);
    for (size_t c : counts) {
      CHECK(emu_allreduce(b.send.data(), b.recv.data(), c, EMU_FLOAT16, EMU_SUM, nullptr) == EMU_SUCCESS);
      ref.push_back(last_tables());
    }
    CHECK(emu_comm_destroy() == EMU_SUCCESS);
    CHECK(fake::live_allocations() == 0);
    const size_t mallocs = fake::malloc_calls();
    CHECK(emu_comm_init(n, 2, algo, 5, 32 << 10) == EMU_SUCCESS);
    // shapes in turn and back again: each call stages what it needs
    const int order[] = {0, 1, 0, 2, 2, 1, 0};
    for (int i : order) {
      CHECK(emu_allreduce_noalloc(b.send.data(), b.recv.data(), counts[i], EMU_FLOAT16, EMU_SUM, nullptr) ==
            EMU_SUCCESS);
      CHECK(last_tables() == ref[i]);
      CHECK(emu_allreduce_noalloc(b.send.data(), b.send.data(), counts[i], EMU_FLOAT16, EMU_SUM, nullptr) ==
            EMU_SUCCESS);
      CHECK(last_tables() == ref[i]);
    }
    int abandoned = -1;
    CHECK(emu_protocol_status(&abandoned) == EMU_SUCCESS && abandoned == 0);
    CHECK(fake::malloc_calls() == mallocs);
    CHECK(lib_allocs() == 0);
  }
  CHECK(emu_comm_destroy() == EMU_SUCCESS);
}

void noalloc_refusals() {
  const int n = 4;
  Buffers b(n, 64);
  const size_t mallocs = fake::malloc_calls();
  const size_t launches = fake::launches.size();
  // the device transport's FIFOs do not fit the scratch array
  CHECK(emu_comm_init(n, 1, EMU_ALGO_RING | EMU_TRANSPORT_DEVICE, 2, 4096) == EMU_SUCCESS);
  CHECK(emu_allreduce_noalloc(b.send.data(), b.recv.data(), 16, EMU_FLOAT32, EMU_SUM, nullptr) ==
        EMU_ERR_INVALID_ARGUMENT);
  // fused tiles of 1 GiB per rank exceed it (the buffers are never touched:
  // the call is refused before anything is enqueued)
  std::vector<const void*> send;
  std::vector<void*> recv;
  const size_t big = (size_t)1 << 30;
  for (int r = 0; r < n; ++r) {
    send.push_back(reinterpret_cast<const void*>((uintptr_t)(2 * r + 1) * (big << 1)));
    recv.push_back(reinterpret_cast<void*>((uintptr_t)(2 * r + 2) * (big << 1)));
  }
  CHECK(emu_comm_init(n, 1, EMU_ALGO_RING | EMU_MODE_FUSED, 2, 4096) == EMU_SUCCESS);
  CHECK(emu_allreduce_noalloc(send.data(), recv.data(), big / 4, EMU_FLOAT32, EMU_SUM, nullptr) ==
        EMU_ERR_INVALID_ARGUMENT);
  // argument errors as emu_allreduce's
  CHECK(emu_allreduce_noalloc(b.send.data(), b.recv.data(), 16, 9, EMU_SUM, nullptr) == EMU_ERR_INVALID_ARGUMENT);
  CHECK(emu_allreduce_noalloc(b.send.data(), b.send.data() + 0, 0, EMU_FLOAT32, EMU_SUM, nullptr) == EMU_SUCCESS);
  CHECK(fake::launches.size() == launches);
  CHECK(fake::malloc_calls() == mallocs);
  CHECK(emu_comm_destroy() == EMU_SUCCESS);
  CHECK(emu_allreduce_noalloc(b.send.data(), b.recv.data(), 16, EMU_FLOAT32, EMU_SUM, nullptr) ==
        EMU_ERR_NOT_INITIALIZED);
  CHECK(fake::live_allocations() == 0);
}

}  // namespace

int main() {
  destroy_frees_everything();
  eviction_frees_dropped_communicators();
  noalloc_allocates_nothing_and_passes_the_same_tables();
  noalloc_refusals();
  if (g_failed) return 1;
  std::printf("ok\n");
  return 0;
}
