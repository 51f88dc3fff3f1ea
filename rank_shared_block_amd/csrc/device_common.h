// Device helpers shared by the kernels: bf16 bit conversions, 16-byte loads,
// MFMA operand types and the XCD-aware workgroup remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even fp32 -> bf16 bits (finite values round correctly; NaN stays NaN).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// Streaming (read-once) 16-byte load: non-temporal hint keeps it from displacing
// the reused operands (x, Vt) in L2.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Buffer resource over [base, base + bytes): a raw buffer load whose offset lies
// outside that range returns zeros without touching memory.  This gives
// branch-free predicated loads (rows past N, K past the end of a range, tokens
// past M) so that every load of a step can be in flight at once.  `bytes` must be
// below 2^31 so that kOOB is always out of range.  0x00020000 is the gfx9-family
// descriptor word for raw 32-bit-format access.
constexpr int kOOB = (int)0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ bf16x8 bload16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

// Workgroup ids are handed to the 8 XCDs round-robin (id % 8).  Remap so that
// each XCD works on a contiguous range of logical tiles: tiles that share
// operands then share one L2.  Returns -1 for the padding ids of the last round.
__device__ __forceinline__ int xcd_contiguous_tile(int bid, int ntiles) {
  const int per_xcd = (ntiles + 7) >> 3;
  const int t = (bid & 7) * per_xcd + (bid >> 3);
  return t < ntiles ? t : -1;
}

}  // namespace aq
