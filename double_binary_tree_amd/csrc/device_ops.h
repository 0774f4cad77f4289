// Device-side element operators on one 128-bit vector per lane.
//
// Every operator works lane-wise on a 16-byte vector (4 x i32/f32, 2 x i64,
// 8 x f16/bf16) and gives the bits of the rounded binary reduction:
//   i32/i64 sum : two's-complement wrap
//   f32 sum     : one IEEE add, round to nearest even, subnormals kept
//   f16 sum     : the correctly rounded f16 add (native packed f16 add)
//   bf16 sum    : f32 add, then round to nearest even into bf16 (the
//                 hardware conversion); equal to the correctly rounded bf16
//                 add, since f32 carries more than 2p+2 significand bits
//   max         : integers plain; floats in "key" space, where the bit
//                 pattern is mapped to a signed integer that orders -0
//                 below +0 and otherwise follows the float order, so the
//                 max is commutative and associative.
// pre() maps a loaded vector into the operator's working space, post()
// maps back before storing (identity except for float max).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"

namespace emu {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef long long i64x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

template <typename T, typename U>
__device__ __forceinline__ T bits(U v) {
  return __builtin_bit_cast(T, v);
}

template <DType T, Op O>
struct Red;

template <>
struct Red<DType::I32, Op::Sum> {
  static __device__ __forceinline__ u32x4 pre(u32x4 x) { return x; }
  static __device__ __forceinline__ u32x4 post(u32x4 x) { return x; }
  static __device__ __forceinline__ u32x4 op(u32x4 a, u32x4 b) { return a + b; }
};
template <>
struct Red<DType::I32, Op::Max> {
  static __device__ __forceinline__ u32x4 pre(u32x4 x) { return x; }
  static __device__ __forceinline__ u32x4 post(u32x4 x) { return x; }
  static __device__ __forceinline__ u32x4 op(u32x4 a, u32x4 b) {
    return bits<u32x4>(__builtin_elementwise_max(bits<i32x4>(a), bits<i32x4>(b)));
  }
};
template <>
struct Red<DType::I64, Op::Sum> {
  static __device__ __forceinline__ u32x4 pre(u32x4 x) { return x; }
  static __device__ __forceinline__ u32x4 post(u32x4 x) { return x; }
  static __device__ __forceinline__ u32x4 op(u32x4 a, u32x4 b) {
    return bits<u32x4>(bits<i64x2>(a) + bits<i64x2>(b));
  }
};
template <>
struct Red<DType::I64, Op::Max> {
  static __device__ __forceinline__ u32x4 pre(u32x4 x) { return x; }
  static __device__ __forceinline__ u32x4 post(u32x4 x) { return x; }
  static __device__ __forceinline__ u32x4 op(u32x4 a, u32x4 b) {
    return bits<u32x4>(__builtin_elementwise_max(bits<i64x2>(a), bits<i64x2>(b)));
  }
};
template <>
struct Red<DType::F32, Op::Sum> {
  static __device__ __forceinline__ u32x4 pre(u32x4 x) { return x; }
  static __device__ __forceinline__ u32x4 post(u32x4 x) { return x; }
  static __device__ __forceinline__ u32x4 op(u32x4 a, u32x4 b) {
    return bits<u32x4>(bits<f32x4>(a) + bits<f32x4>(b));
  }
};
// f32 key: negative patterns get their magnitude bits flipped, so signed
// integer order equals float order with -0 < +0.  The map is its own inverse.
template <>
struct Red<DType::F32, Op::Max> {
  static __device__ __forceinline__ u32x4 key(u32x4 x) {
    const i32x4 s = bits<i32x4>(x);
    return bits<u32x4>(s ^ ((s >> 31) & 0x7FFFFFFF));
  }
  static __device__ __forceinline__ u32x4 pre(u32x4 x) { return key(x); }
  static __device__ __forceinline__ u32x4 post(u32x4 x) { return key(x); }
  static __device__ __forceinline__ u32x4 op(u32x4 a, u32x4 b) {
    return bits<u32x4>(__builtin_elementwise_max(bits<i32x4>(a), bits<i32x4>(b)));
  }
};
template <>
struct Red<DType::F16, Op::Sum> {
  static __device__ __forceinline__ u32x4 pre(u32x4 x) { return x; }
  static __device__ __forceinline__ u32x4 post(u32x4 x) { return x; }
  static __device__ __forceinline__ u32x4 op(u32x4 a, u32x4 b) {
    return bits<u32x4>(bits<f16x8>(a) + bits<f16x8>(b));
  }
};
template <>
struct Red<DType::BF16, Op::Sum> {
  static __device__ __forceinline__ u32x4 pre(u32x4 x) { return x; }
  static __device__ __forceinline__ u32x4 post(u32x4 x) { return x; }
  // Widen both operands to f32 (exact), add, and round the sums to bf16
  // with the hardware's round-to-nearest-even conversion (subnormals kept
  // under the kernel's float mode; overflow gives infinity).
  static __device__ __forceinline__ u32x4 op(u32x4 a, u32x4 b) {
    const f32x8 s = __builtin_convertvector(bits<bf16x8>(a), f32x8) + __builtin_convertvector(bits<bf16x8>(b), f32x8);
    return bits<u32x4>(__builtin_convertvector(s, bf16x8));
  }
};
// 16-bit float key, same idea as the f32 key, on each half.
struct Key16 {
  static __device__ __forceinline__ u32x4 key(u32x4 x) {
    const i16x8 s = bits<i16x8>(x);
    return bits<u32x4>(s ^ ((s >> 15) & (short)0x7FFF));
  }
  static __device__ __forceinline__ u32x4 pre(u32x4 x) { return key(x); }
  static __device__ __forceinline__ u32x4 post(u32x4 x) { return key(x); }
  static __device__ __forceinline__ u32x4 op(u32x4 a, u32x4 b) {
    return bits<u32x4>(__builtin_elementwise_max(bits<i16x8>(a), bits<i16x8>(b)));
  }
};
template <>
struct Red<DType::F16, Op::Max> : Key16 {};
template <>
struct Red<DType::BF16, Op::Max> : Key16 {};

template <DType T>
struct Unit {
  static constexpr int elems = kVecBytes / (T == DType::I64 ? 8 : (T == DType::F16 || T == DType::BF16) ? 2 : 4);
  static constexpr int esz = kVecBytes / elems;
};

// Whole-vector global accesses.  Every byte is read once and written once,
// so by default both carry the non-temporal (streaming) hint.
#ifndef EMU_LOAD_NT
#define EMU_LOAD_NT 1
#endif
#ifndef EMU_STORE_NT
#define EMU_STORE_NT 1
#endif
// Raw buffer view starting at `base` (wave-uniform).  The hardware returns
// zeros for any offset at or past its range, so a lane that must not read
// passes kNoLoad instead of branching around the load.
constexpr uint32_t kBufRange = 0x7FFFFFF0u;
constexpr uint32_t kNoLoad = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)kBufRange,
                                           0x00020000 /* 32-bit data format */);
}
__device__ __forceinline__ u32x4 ld_buf(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)byte_off, 0,
                                                                         EMU_LOAD_NT ? 2 /* nt */ : 0));
}

__device__ __forceinline__ u32x4 ld_vec(const void* base, uint64_t byte_off) {
  const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const char*>(base) + byte_off);
#if EMU_LOAD_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}
__device__ __forceinline__ void st_vec(void* base, uint64_t byte_off, u32x4 v) {
  u32x4* p = reinterpret_cast<u32x4*>(static_cast<char*>(base) + byte_off);
#if EMU_STORE_NT
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

// Partial vector at the very end of a buffer: `nbytes` (< 16, a multiple of
// 2) valid bytes, never accessed past nbytes; the rest reads as zero.
__device__ __forceinline__ u32x4 ld_part(const void* base, uint64_t byte_off, int nbytes) {
  // Seven half-word loads at most, each from an address inside the nbytes
  // (half-word k < nbytes / 2, else half-word 0): none conditional, so all
  // are issued back to back and combined by selects once they arrive, in
  // one memory round trip.  (Loads under conditions leave values to merge,
  // and the merge copies wait for the loads one by one.)
  const uint16_t* h = reinterpret_cast<const uint16_t*>(static_cast<const char*>(base) + byte_off);
  const int nh = nbytes / 2;
  uint32_t x[7];
#pragma unroll
  for (int k = 0; k < 7; ++k) x[k] = h[k < nh ? k : 0];
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = 2 * i < nh ? x[2 * i] : 0u;
    const uint32_t hi = 2 * i + 1 < nh ? x[2 * i + 1] : 0u;
    w[i] = lo | hi << 16;
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}
__device__ __forceinline__ void st_part(void* base, uint64_t byte_off, int nbytes, u32x4 v) {
  char* c = static_cast<char*>(base) + byte_off;
  uint32_t* d = reinterpret_cast<uint32_t*>(c);
  uint16_t* h = reinterpret_cast<uint16_t*>(c);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (4 * i + 4 <= nbytes) d[i] = w[i];
    else if (4 * i + 2 <= nbytes) h[2 * i] = (uint16_t)w[i];
  }
}

// One vector of `nbytes` (0 to 16; 0 reads as zeros) at `base` + `lane_off`,
// `base` wave-uniform and `lane_off` below kBufRange.  The whole-vector load
// is issued unconditionally through a raw buffer view (kNoLoad where the
// vector is not whole) and only a partial vector takes a branch, which keeps
// the whole-vector value out of any merge: a merge with a value loaded under
// a condition becomes a register copy that waits for the load, so the caller
// could no longer overlap the load with what follows it.
__device__ __forceinline__ u32x4 ld_lane(const void* base, uint32_t lane_off, int nbytes) {
  u32x4 x = ld_buf(buffer_view(base), nbytes == kVecBytes ? lane_off : kNoLoad);
  if (nbytes > 0 && nbytes < kVecBytes) x = ld_part(base, lane_off, nbytes);
  return x;
}

// Store `nbytes` of one vector (16 = whole vector).
__device__ __forceinline__ void st_any(void* base, uint64_t byte_off, int nbytes, u32x4 v) {
  if (nbytes == kVecBytes) st_vec(base, byte_off, v);
  else st_part(base, byte_off, nbytes, v);
}

}  // namespace emu
