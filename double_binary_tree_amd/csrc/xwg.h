// Stepwise ring all-reduce across workgroups (one workgroup per channel and
// ring position, FIFOs in device memory between them): the arguments that
// the host passes beside StepArgs.
#pragma once

#include <cstdint>

#include "common.h"

namespace emu {

// Counters are uint32, each in a line of its own (kXCounterStride words
// apart).
constexpr uint32_t kXCounterStride = 32;
struct XArgs {
  const uint32_t* chan_loops;   // [nch][2]: first loop, end loop of the channel in the loop table
  const uint32_t* chan_ring;    // [nch]: the channel's row of the ring order table
  const uint32_t* loop_slices;  // [loops]: slices per step of the loop (the most any of its blocks spans)
  void* fifo;                   // SIMPLE: [nch*N][slots][lanes] 16-byte vectors; LL: [nch*N][slots][4][lanes] words
  uint32_t* tail;               // SIMPLE: items written into FIFO f, at f * kXCounterStride
  uint32_t* head;               // items consumed from FIFO f, at f * kXCounterStride
  uint32_t* abandon;            // nonzero once a call was abandoned (sticky until the host resets it)
  uint32_t* status;             // set when a call is abandoned
  uint32_t nslots;              // FIFO depth in slices, at least every loop's loop_slices
  uint32_t spin_limit;          // polls before a wait is abandoned
};

}  // namespace emu
