// Streaming kernels over plain device buffers: read-only, write-only and
// copy, with the access style of the collectives (whole 16-byte vectors per
// lane, non-temporal, 4 KiB tiles of 256 lanes).  They measure, in the same
// run, the HBM rates an all-reduce is compared with: its bytes are half
// reads and half writes, so its practical ceiling lies between the
// read-only and the write-only rate, and the copy rate moves the same mix.
#include "device_ops.h"

namespace emu {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;   // tiles whose accesses a lane issues back to back

// A read that nobody consumes would be removed by the compiler, so every
// lane folds what it reads and stores the fold only if it equals `key`,
// which the host draws so that this practically never happens; `sink` is
// 16 bytes.
template <int KIND>
__global__ __launch_bounds__(kStreamThreads) void stream_kernel(const void* __restrict__ src, void* __restrict__ dst,
                                                              uint64_t nvec, uint32_t key, void* __restrict__ sink) {
  const uint64_t ntiles = (nvec + kStreamThreads - 1) / kStreamThreads;
  const uint64_t step = (uint64_t)gridDim.x * kStreamUnroll;
  u32x4 acc = {0, 0, 0, 0};
  const u32x4 pattern = {key, ~key, key ^ 0x5A5A5A5Au, key + 1u};
  for (uint64_t t0 = (uint64_t)blockIdx.x * kStreamUnroll; t0 < ntiles; t0 += step) {
    uint64_t off[kStreamUnroll];
    bool ok[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const uint64_t v = (t0 + u) * kStreamThreads + threadIdx.x;
      ok[u] = v < nvec;
      off[u] = v * kVecBytes;
    }
    if constexpr (KIND == EMU_STREAM_WRITE) {
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u)
        if (ok[u]) st_vec(dst, off[u], pattern);
    } else {
      u32x4 x[kStreamUnroll];
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) x[u] = ok[u] ? ld_vec(src, off[u]) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) {
        if constexpr (KIND == EMU_STREAM_COPY) {
          if (ok[u]) st_vec(dst, off[u], x[u]);
        } else {
          acc ^= x[u];
        }
      }
    }
  }
  if constexpr (KIND == EMU_STREAM_READ) {
    if (acc.x == key && acc.y == ~key && acc.z == key && acc.w == ~key) *static_cast<u32x4*>(sink) = acc;
  }
}

hipError_t launch_stream(int kind, const void* src, void* dst, uint64_t bytes, uint32_t key, int cus,
                         hipStream_t s) {
  const uint64_t nvec = bytes / kVecBytes;
  const uint64_t groups = (nvec + (uint64_t)kStreamThreads * kStreamUnroll - 1) / ((uint64_t)kStreamThreads * kStreamUnroll);
  // a few waves of resident workgroups, each walking the tiles grid-strided
  const int grid = (int)std::max<uint64_t>(1, std::min<uint64_t>(groups, (uint64_t)cus * 32));
  switch (kind) {
    case EMU_STREAM_READ:
      hipLaunchKernelGGL(stream_kernel<EMU_STREAM_READ>, dim3(grid), dim3(kStreamThreads), 0, s, src, nullptr, nvec,
                         key, dst);
      break;
    case EMU_STREAM_WRITE:
      hipLaunchKernelGGL(stream_kernel<EMU_STREAM_WRITE>, dim3(grid), dim3(kStreamThreads), 0, s, nullptr, dst, nvec,
                         key, nullptr);
      break;
    default:
      hipLaunchKernelGGL(stream_kernel<EMU_STREAM_COPY>, dim3(grid), dim3(kStreamThreads), 0, s, src, dst, nvec, key,
                         nullptr);
      break;
  }
  return hipGetLastError();
}

}  // namespace emu
