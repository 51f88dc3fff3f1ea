// The block-16 FP4 encoder shared by the pack kernels and the fused
// materialise-and-pack kernel ("Internals and extension", section
// "Nvfp4Spec"; the recipe is stated at the top of fp4_pack.hip).
#pragma once

#include <math.h>

#include "device_common.h"

namespace aq {

// E4M3FN bits of a finite q >= 0: round to nearest even, saturate at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_rne_sat(double q) {
  if (!(q > 0.0)) return 0u;
  if (q >= 448.0) return 0x7Eu;
  int e;
  (void)frexp(q, &e);                           // q in [2^(e-1), 2^e)
  const int qexp = e - 4 > -9 ? e - 4 : -9;     // 3 fraction bits; subnormal step 2^-9
  const double n = rint(ldexp(q, -qexp));       // ties to even
  const int ni = (int)n;
  uint32_t bits = qexp == -9 ? (uint32_t)ni : (uint32_t)(((e + 6) << 3) + ni - 8);
  return bits > 0x7Eu ? 0x7Eu : bits;
}

__device__ __forceinline__ double e4m3_value(uint32_t b) {
  return b < 8 ? ldexp((double)b, -9) : ldexp((double)(8 + (b & 7)), (int)(b >> 3) - 10);
}

// One 16-value block (its bf16 bits in q[0..7], element 2i in the low half of
// q[i]) with global scale g: the E4M3 scale byte and the 16 codes.
__device__ __forceinline__ void pack_block16(const uint32_t q[8], float g, uint32_t &lo, uint32_t &hi,
                                             uint32_t &sf) {
  uint32_t amag = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    amag = max(amag, q[i] & 0x7FFFu);
    amag = max(amag, (q[i] >> 16) & 0x7FFFu);
  }
  const double ab = (double)bf2f((uint16_t)amag);
  sf = e4m3_rne_sat(ab / (6.0 * (double)g));
  const float D = (float)((double)g * e4m3_value(sf));
  lo = 0;
  hi = 0;
  if (D >= 0x1p-90f) {
    // Code = number of E2M1 midpoints m_i D below |w| (ties to the even code:
    // strictly above m_0, m_2, m_4, m_6; at or above m_1, m_3, m_5), found by a
    // three-step binary search over the monotone midpoints, in fp32: with
    // p = RN(m_i D) and its exact residual e = m_i D - p (an fma; no underflow
    // for D >= 2^-90), a float x is >= m_i D iff x >= p (e <= 0) or x >= the
    // next float above p (e > 0), and > m_i D iff x >= p (e < 0) or x >= the
    // next float above p (e >= 0).  So every test is one exact fp32 x >= T_i.
    float T[7];
    const float mid[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
#pragma unroll
    for (int i = 0; i < 7; ++i) {
      const float pr = mid[i] * D, e = __builtin_fmaf(mid[i], D, -pr);
      const bool up = (i & 1) ? e > 0.f : e >= 0.f;
      T[i] = up ? __uint_as_float(__float_as_uint(pr) + 1u) : pr;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t bits = (q[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
      const float x = __uint_as_float((bits & 0x7FFFu) << 16);
      const bool b4 = x >= T[3];
      const bool b2 = x >= (b4 ? T[5] : T[1]);
      const float tl = b4 ? (b2 ? T[6] : T[4]) : (b2 ? T[2] : T[0]);
      uint32_t c = (b4 ? 4u : 0u) + (b2 ? 2u : 0u) + (x >= tl ? 1u : 0u);
      if (c != 0 && (bits & 0x8000u)) c |= 8u;
      if (i < 8)
        lo |= c << (4 * i);
      else
        hi |= c << (4 * (i - 8));
    }
  } else if (D > 0.f) {
    // Tiny D: the same search on thresholds exact in fp64.
    const double d = (double)D;
    const double t0 = 0.25 * d, t1 = 0.75 * d, t2 = 1.25 * d, t3 = 1.75 * d, t4 = 2.5 * d,
                 t5 = 3.5 * d, t6 = 5.0 * d;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t bits = (q[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
      const double x = (double)bf2f((uint16_t)(bits & 0x7FFFu));
      const bool b4 = x >= t3;
      const bool b2 = x >= (b4 ? t5 : t1);
      const double tl = b4 ? (b2 ? t6 : t4) : (b2 ? t2 : t0);
      uint32_t c = (b4 ? 4u : 0u) + (b2 ? 2u : 0u) + (x > tl ? 1u : 0u);
      if (c != 0 && (bits & 0x8000u)) c |= 8u;
      if (i < 8)
        lo |= c << (4 * i);
      else
        hi |= c << (4 * (i - 8));
    }
  }
}

// The global scale of a weight from its largest magnitude (bf16 bits):
// RN_f32(A / 2688), 1 where A == 0.
__device__ __forceinline__ float fp4_global_scale(unsigned amax_bits) {
  const float A = bf2f((uint16_t)amax_bits);
  return A == 0.f ? 1.0f : (float)((double)A / 2688.0);
}

}  // namespace aq
