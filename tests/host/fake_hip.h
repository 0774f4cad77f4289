// What the host-only HIP stand-in (fake_hip.cpp) records, for the drivers
// that link it.
#pragma once

#include <cstddef>
#include <string>
#include <vector>

namespace fake {

struct Launch {
  std::string kernel;                 // "fused", "step_ring", "step_tree", "ll_ring", "ll_tree", "xring"
  int coll;                           // all-reduce, reduce-scatter or all-gather
  std::vector<unsigned char> tasks;   // the tile or task table the launch received
};

extern std::vector<Launch> launches;

size_t live_allocations();   // "device" allocations not yet freed
size_t live_bytes();
size_t malloc_calls();       // hipMalloc calls so far

}  // namespace fake
