// Device-side helpers for the gfx950 kernels: vector types, 16-byte memory
// moves, bf16 packing, MFMA wrappers and wave reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvpaged_internal.h"

namespace kvp {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Streaming load: data read once, marked non-temporal.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) {
  return __builtin_bit_cast(u32x4, v);
}

// bf16 <-> fp32. bf16 -> fp32 is exact (the bf16 bits are the high half).
__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __builtin_bit_cast(float, w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}
// Round-to-nearest-even fp32 -> bf16 of two values, packed (lo, hi): one
// v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Select the low (or high) 16-bit halves of two dwords into one dword:
// result = (a.half, b.half).
__device__ __forceinline__ uint32_t pick_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pick_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// LDS transpose read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane j receives element (j & 3) of the 8-byte chunks addressed by lanes
// (j >> 2) + 4k, k = 0..3. With lane s pointing at row r0 + (s >> 2),
// column c0 + 4 (s & 3) of a row-major 16-bit matrix, lane j receives rows
// r0..r0+3 of column c0 + j.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
__device__ __forceinline__ u32x2 lds_read_tr16(const void* lds_addr) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(lds_addr));
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ float to_f32<bf16>(bf16 v) {
  return static_cast<float>(v);
}
template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float v) {
  return static_cast<bf16>(v);
}

// Workgroup order for the 8 XCDs of MI355X: consecutive workgroup ids are
// dispatched round-robin over the XCDs, and each XCD has its own L2. This
// maps dispatch id `id` (of n) to a logical index such that XCD x runs the
// contiguous logical range x*n/8 .. (x+1)*n/8 - 1 in order, so workgroups
// that are neighbours in logical order (and read the same K/V) share an L2.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_order(int id, int n) {
  const int per = n / kXcds, rem = n % kXcds;
  const int x = id % kXcds, slot = id / kXcds;
  const int base = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  return base + slot;
}

}  // namespace kvp

#define KVP_LAUNCH_CHECK(what)                                              \
  do {                                                                      \
    hipError_t e_ = hipGetLastError();                                      \
    if (e_ != hipSuccess)                                                   \
      return kvp_fail(KV_EHIP, "%s: launch failed: %s", what,               \
                      hipGetErrorString(e_));                               \
  } while (0)
