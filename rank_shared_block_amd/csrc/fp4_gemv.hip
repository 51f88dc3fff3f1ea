// FP4 decode GEMV: y = bf16(x Wq^T) for up to 16 tokens, where Wq is a weight
// packed by the block-16 FP4 pack (two E2M1 codes per byte, [N, K/2]; one
// FP8-E4M3 scale per 16 K-values, [N, K/16]; one fp32 global scale g).
//
// What it computes ("Execution paths", section "Precompute-outside": each W_eff
// is quantised to 4 bits at load and used in place of the dense weight;
// container from "Internals and extension", section "Nvfp4Spec"): weight (n, k)
// is E2M1(code) * D, with the block step D = RN_f32(g * E4M3(scale)) of its
// 16-value block; y[m, n] = sum_k x[m, k] * weight(n, k).
//
// Design (MI355X / gfx950): at decode the kernel streams 0.5625 bytes per weight
// (3.56x fewer than bf16), so it is bound by HBM and by the dequantisation on
// the VALU, not by the MFMAs.
// * One 16-byte load per lane brings 32 consecutive codes of one weight row
//   (four lanes: 128 K-values of the row), plus the row's two block-scale bytes
//   for them; the tokens' 64 matching bytes of x come in four 16-byte loads.
// * The codes are dequantised in registers: the E2M1 values' fp32 bits come
//   from byte-permute table lookups (four codes per v_perm_b32), are multiplied
//   by the block step (computed exactly as the pack defines it) and rounded once
//   to bf16, about five VALU operations per weight; the dot products run on
//   v_mfma_f32_16x16x32_bf16 with the weights as 16-row groups and the tokens as
//   the other operand (rows of x beyond M are zero registers, not loads).  A
//   lane's eight codes of one k-step are K positions 32 q + 8 s .. + 7 of its
//   128 (q = lane / 16, s = the k-step); x is loaded with the same permutation,
//   so the contraction is unchanged.  Each weight is rounded to bf16 once, a
//   relative error of at most 2^-8 per weight, inside the bf16 tolerance.
//   Up to four tokens (K % 64 == 0) take k_fp4_gemv_m4 instead, which needs no
//   per-weight rounding (below); one token on a large weight takes
//   k_fp4_gemv_dot, which converts the codes with gfx950's FP4 -> bf16
//   instruction and multiplies on the VALU's packed bf16 dot products (below).
// * Eight waves per workgroup (two per SIMD), so that one wave's dequantisation
//   overlaps another's loads.  Buffer resources make rows past N, K past the
//   range and tokens past M read as zero: the loop is branch-free with two
//   steps in flight per wave.
// * Few rows (long K) split K over S workgroups; fp32 partials are added in
//   split order by a small fold kernel.  Deterministic.

#include <limits.h>
#include <stdlib.h>

#include "aq_internal.h"
#include "device_common.h"

namespace aq {

struct F4Args {
  const uint8_t *packed, *scales;
  const float *g;
  const uint16_t *x;
  uint16_t *y;
  float *part;            // S > 1: [S][M][N] fp32 partials
  int M, N, K, ldx, ldy, rows, ntiles, S, kchunk;
};


// E4M3FN byte (sign clear) as fp32: 1 + m/8 times 2^(e - 7), or m/8 * 2^-6.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
}

// Eight codes (one 32-bit word, code i in bits 4 i .. 4 i + 3) times the block
// step D, rounded to bf16: one MFMA operand, element i = code i.
// The E2M1 magnitudes (0, .5, 1, 1.5, 2, 3, 4, 6) are exact in the upper half of
// an fp32; their two bytes come from byte-permute table lookups (v_perm_b32: a
// selector byte 0..7 picks a byte of the 8-byte table {s1, s0}), four codes per
// lookup: bf16 high bytes 00 3F 3F 3F 40 40 40 40, low bytes 00 00 80 C0 00 40
// 80 C0.  Each value is assembled as fp32 bits, multiplied by D (fp32) and the
// pair rounded to bf16 at once; the code's sign bit is then moved onto the
// bf16 sign (a code of -0 gives -0).
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float D) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const uint32_t mE = w & 0x07070707u, mO = (w >> 4) & 0x07070707u;    // byte j: code 2j, 2j + 1
  const uint32_t hE = __builtin_amdgcn_perm(0x40404040u, 0x3F3F3F00u, mE);
  const uint32_t lE = __builtin_amdgcn_perm(0xC0804000u, 0xC0800000u, mE);
  const uint32_t hO = __builtin_amdgcn_perm(0x40404040u, 0x3F3F3F00u, mO);
  const uint32_t lO = __builtin_amdgcn_perm(0xC0804000u, 0xC0800000u, mO);
  const uint32_t sE = (w << 4) & 0x80808080u, sO = w & 0x80808080u;       // sign at bit 7 of byte j
  uint32_t out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // fp32 bits: byte 3 = high byte, byte 2 = low byte (selector 0x0C = zero)
    const uint32_t sel = 0x0C0Cu | ((uint32_t)j << 16) | ((uint32_t)(4 + j) << 24);
    const float v0 = __uint_as_float(__builtin_amdgcn_perm(hE, lE, sel)) * D;
    const float v1 = __uint_as_float(__builtin_amdgcn_perm(hO, lO, sel)) * D;
    const bf16x2 h = {(__bf16)v0, (__bf16)v1};
    // signs of codes 2j (to bit 15) and 2j + 1 (to bit 31)
    const uint32_t sg = __builtin_amdgcn_perm(sO, sE, 0x000C000Cu | ((uint32_t)j << 8) | ((uint32_t)(4 + j) << 24));
    out[j] = __builtin_bit_cast(uint32_t, h) ^ sg;
  }
  return as_bf16x8(make_uint4(out[0], out[1], out[2], out[3]));
}

__device__ __forceinline__ uint32_t bload_u16(__amdgpu_buffer_rsrc_t r, int off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint4 bload_u128(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Eight codes (one word: code 2j in the low nibble of byte j, code 2j + 1 in
// the high one) as four exact bf16 pairs, element 2j in the low half of pair
// j: gfx950's FP4 -> bf16 conversion with a unit scale, one instruction per
// byte (exact E2M1 values, low nibble into the low half: checked for all 256
// bytes in each byte position).
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t w, int j) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  switch (j) {                     // the byte select is an immediate
    case 0: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0); break;
    case 1: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1); break;
    case 2: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2); break;
    default: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3); break;
  }
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ void e2m1_pairs(uint32_t w, uint32_t (&pr)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) pr[j] = e2m1_pair(w, j);
}

// NG: 16-row groups per workgroup; PART: fp32 partials of a K split.
template <int NG, bool PART>
__global__ __launch_bounds__(512) void k_fp4_gemv(const F4Args a) {
  constexpr int WAVES = 8, KS = 4, KSTEP = 128, NT = 64 * WAVES;
  constexpr int SLOT = NG * 256;
  __shared__ float red[WAVES * SLOT];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j16 = lane & 15, q = lane >> 4;

  const int unit = xcd_contiguous_tile(blockIdx.x, a.ntiles * a.S);
  if (unit < 0) return;
  const int tile = unit / a.S, p = unit - tile * a.S;
  const int K = a.K, row0 = tile * a.rows;
  const int Rv = min(a.rows, a.N - row0);
  const int kbeg = p * a.kchunk, kend = min(K, kbeg + a.kchunk);
  const int nsteps = (kend - kbeg + KSTEP - 1) / KSTEP;
  const float g = *a.g;

  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.packed + (size_t)row0 * (K / 2), (uint32_t)Rv * (K / 2));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales + (size_t)row0 * (K / 16), (uint32_t)Rv * (K / 16));
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)((a.M - 1) * a.ldx + K) * 2);
  const int xoff = j16 < a.M ? j16 * a.ldx * 2 : kOOB;

  f32x4 acc[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) acc[gi] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One step: 128 K-values; this lane's 32 of them start at k = k0 + 32 q.
  auto fetch = [&](int st, uint4 (&cd)[NG], uint32_t (&sc)[NG], uint4 (&xd)[KS]) {
    const int k = kbeg + st * KSTEP + 32 * q;
    const bool in = st < nsteps && k < kend;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int r = gi * 16 + j16;
      cd[gi] = bload_u128(rc, in ? r * (K / 2) + k / 2 : kOOB);
      sc[gi] = bload_u16(rs, in ? r * (K / 16) + k / 16 : kOOB);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) xd[s] = bload_u128(rx, in && xoff != kOOB ? xoff + (k + 8 * s) * 2 : kOOB);
  };
  auto compute = [&](const uint4 (&cd)[NG], const uint32_t (&sc)[NG], const uint4 (&xd)[KS]) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const float D0 = g * e4m3_value(sc[gi] & 0xFFu), D1 = g * e4m3_value(sc[gi] >> 8);
      const uint32_t w[4] = {cd[gi].x, cd[gi].y, cd[gi].z, cd[gi].w};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        acc[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xd[s]), dequant8(w[s], s < 2 ? D0 : D1), acc[gi],
                                                          0, 0, 0);
    }
  };

  // Two register sets in turn; a wave fetches exactly its own steps.
  const int nmine = wave < nsteps ? (nsteps - 1 - wave) / WAVES + 1 : 0;
  uint4 ca[NG], cb[NG], xa[KS], xb[KS];
  uint32_t sa[NG], sb[NG];
  if (nmine > 0) fetch(wave, ca, sa, xa);
  int i = 0;
  for (; i + 2 < nmine; i += 2) {
    fetch(wave + (i + 1) * WAVES, cb, sb, xb);
    __builtin_amdgcn_sched_barrier(0);
    compute(ca, sa, xa);
    __builtin_amdgcn_sched_barrier(0);
    fetch(wave + (i + 2) * WAVES, ca, sa, xa);
    __builtin_amdgcn_sched_barrier(0);
    compute(cb, sb, xb);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (i + 1 < nmine) {
    fetch(wave + (i + 1) * WAVES, cb, sb, xb);
    __builtin_amdgcn_sched_barrier(0);
    compute(ca, sa, xa);
    __builtin_amdgcn_sched_barrier(0);
    compute(cb, sb, xb);
  } else if (i < nmine) {
    compute(ca, sa, xa);
  }

  // Partial sums of the waves added in wave order.  Element v of lane l is
  // token 4 (l / 16) + v, row l % 16 of its group.
  {
    float *slot = red + wave * SLOT;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int v = 0; v < 4; ++v) slot[(gi * 4 + v) * 64 + lane] = acc[gi][v];
  }
  __syncthreads();
  for (int e = tid; e < a.M * Rv; e += NT) {
    const int m = e / Rv, nl = e - m * Rv;
    const int idx = ((nl >> 4) * 4 + (m & 3)) * 64 + ((m >> 2) << 4) + (nl & 15);
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += red[w * SLOT + idx];
    if constexpr (PART)
      a.part[((size_t)p * a.M + m) * a.N + row0 + nl] = v;
    else
      a.y[(size_t)m * a.ldy + row0 + nl] = f2bf(v);
  }
}

// Up to four tokens: exact per-block scaling.  The x operand is spread over
// the MFMA's 16 rows so that row 4 t + q holds token t's values only on the K
// positions of lane group q (zeros elsewhere; the zeros are out-of-range buffer
// loads).  Each output row of a 16x16x32 MFMA is then the partial sum of one
// token over one lane group's eight codes -- eight codes of ONE 16-value block
// -- so the weights enter as their exact E2M1 values (bf16) and the block step
// D is applied once per block and token by an fp32 FMA: no per-weight
// multiply or rounding.  Lane (t, n) receives token t's four partials of row n
// (blocks 2 q + s / 2 of the step, q = 0..3) and adds D[n, block] times each to
// its one accumulator.  Codes become bf16 pairs by gfx950's FP4 -> bf16
// conversion (one byte, two codes, per instruction); E4M3 scale bytes through
// a 256-entry LDS table.
template <int NG, bool PART>
__global__ __launch_bounds__(512) void k_fp4_gemv_m4(const F4Args a) {
  constexpr int WAVES = 8, KS = 4, KSTEP = 128, NT = 64 * WAVES;
  constexpr int SLOT = NG * 64;
  __shared__ float red[WAVES * SLOT];
  __shared__ float scale_lut[256];       // E4M3 byte -> g * value (RN_f32)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j16 = lane & 15, q = lane >> 4;

  const int unit = xcd_contiguous_tile(blockIdx.x, a.ntiles * a.S);
  if (unit < 0) return;
  const int tile = unit / a.S, p = unit - tile * a.S;
  const int K = a.K, row0 = tile * a.rows;
  const int Rv = min(a.rows, a.N - row0);
  const int kbeg = p * a.kchunk, kend = min(K, kbeg + a.kchunk);
  const int nsteps = (kend - kbeg + KSTEP - 1) / KSTEP;

  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.packed + (size_t)row0 * (K / 2), (uint32_t)Rv * (K / 2));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales + (size_t)row0 * (K / 16), (uint32_t)Rv * (K / 16));
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)((a.M - 1) * a.ldx + K) * 2);
  // x operand row j16 = 4 t + q' carries token t only in lane group q' == q.
  const int tx = j16 >> 2;
  const int xoff = ((j16 & 3) == q && tx < a.M) ? tx * a.ldx * 2 : kOOB;

  float acc[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) acc[gi] = 0.f;

  auto fetch = [&](int st, uint4 (&cd)[NG], uint2 (&sc)[NG], uint4 (&xd)[KS]) {
    const int k0 = kbeg + st * KSTEP, k = k0 + 32 * q;
    const bool in = st < nsteps && k < kend, in0 = st < nsteps;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int r = gi * 16 + j16;
      cd[gi] = bload_u128(rc, in ? r * (K / 2) + k / 2 : kOOB);
      // the step's eight scale bytes of row r (blocks past K read as zero)
      const __amdgpu_buffer_rsrc_t rr = rs;
      const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b32(rr, in0 && k0 < kend ? r * (K / 16) + k0 / 16 : kOOB, 0, 0);
      const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b32(rr, in0 && k0 + 64 < kend ? r * (K / 16) + k0 / 16 + 4 : kOOB, 0, 0);
      sc[gi] = make_uint2(lo, hi);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) xd[s] = bload_u128(rx, in && xoff != kOOB ? xoff + (k + 8 * s) * 2 : kOOB);
  };
  auto compute = [&](const uint4 (&cd)[NG], const uint2 (&sc)[NG], const uint4 (&xd)[KS]) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const uint32_t w[4] = {cd[gi].x, cd[gi].y, cd[gi].z, cd[gi].w};
      float D[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) D[b] = scale_lut[((b < 4 ? sc[gi].x : sc[gi].y) >> (8 * (b & 3))) & 0xFFu];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const uint32_t ws = w[s];
        const uint4 wb = make_uint4(e2m1_pair(ws, 0), e2m1_pair(ws, 1), e2m1_pair(ws, 2), e2m1_pair(ws, 3));
        const f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xd[s]), as_bf16x8(wb),
                                                                f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[gi] = fmaf(D[2 * v + (s >> 1)], c[v], acc[gi]);
      }
    }
  };

  const int nmine = wave < nsteps ? (nsteps - 1 - wave) / WAVES + 1 : 0;
  uint4 ca[NG], cb[NG], xa[KS], xb[KS];
  uint2 sa[NG], sb[NG];
  if (nmine > 0) fetch(wave, ca, sa, xa);
  // The step-scale table is built while the first step's loads are in
  // flight (the global scale is a scalar load; the barrier waits for the
  // table's LDS writes only).
  {
    const float g = *a.g;
    if (tid < 256) scale_lut[tid] = g * e4m3_value(tid & 0x7Fu);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  int i = 0;
  for (; i + 2 < nmine; i += 2) {
    fetch(wave + (i + 1) * WAVES, cb, sb, xb);
    __builtin_amdgcn_sched_barrier(0);
    compute(ca, sa, xa);
    __builtin_amdgcn_sched_barrier(0);
    fetch(wave + (i + 2) * WAVES, ca, sa, xa);
    __builtin_amdgcn_sched_barrier(0);
    compute(cb, sb, xb);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (i + 1 < nmine) {
    fetch(wave + (i + 1) * WAVES, cb, sb, xb);
    __builtin_amdgcn_sched_barrier(0);
    compute(ca, sa, xa);
    __builtin_amdgcn_sched_barrier(0);
    compute(cb, sb, xb);
  } else if (i < nmine) {
    compute(ca, sa, xa);
  }

  // Lane (t, n) holds token t, row n of each group; waves added in order.
  {
    float *slot = red + wave * SLOT;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) slot[gi * 64 + lane] = acc[gi];
  }
  __syncthreads();
  for (int e = tid; e < a.M * Rv; e += NT) {
    const int m = e / Rv, nl = e - m * Rv;
    const int idx = (nl >> 4) * 64 + m * 16 + (nl & 15);
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += red[w * SLOT + idx];
    if constexpr (PART)
      a.part[((size_t)p * a.M + m) * a.N + row0 + nl] = v;
    else
      a.y[(size_t)m * a.ldy + row0 + nl] = f2bf(v);
  }
}

// y = bf16(sum of the S partials, in split order).
// Up to MT tokens (M <= 4), packed dot products instead of MFMAs: a wave takes
// NG groups of four rows; lane (row in group, chunk c) holds 32 codes of its row
// per step (a step covers 512 K-values of four rows), converts them into exact
// bf16 pairs (one instruction per byte), and multiplies them with the tokens' x pairs
// (staged once per workgroup in LDS, read by the four row lanes of a chunk
// together) by v_dot2c_f32_bf16 into one fp32 sum per 16-value block; the
// block step D = RN_f32(g E4M3(scale)) then scales that sum into the row's
// accumulator by one FMA.  Products are exact; only the sums and the output
// are rounded.  The 16 chunk lanes of a row add their sums with a butterfly.
constexpr int kFp4DotXCap = 8192;              // K-values of x per workgroup (LDS)
template <int MT, int NG, bool PART>
__global__ __launch_bounds__(256) void k_fp4_gemv_dot(const F4Args a) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // [MT][kchunk] (launch-time size)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, rsub = lane >> 4;
  const int unit = xcd_contiguous_tile(blockIdx.x, a.ntiles * a.S);
  if (unit < 0) return;
  const int tile = unit / a.S, p = unit - tile * a.S;
  const int K = a.K, row0 = tile * a.rows;
  const int Rv = min(a.rows, a.N - row0);
  const int kbeg = p * a.kchunk, kend = min(K, kbeg + a.kchunk), kn = kend - kbeg;
  const float g = *a.g;

  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.packed + (size_t)row0 * (K / 2), (uint32_t)Rv * (K / 2));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales + (size_t)row0 * (K / 16), (uint32_t)Rv * (K / 16));
  float acc[NG][MT];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[gi][m] = 0.f;

  auto fetch = [&](int k0, uint4 (&cd)[NG], uint32_t (&sc)[NG]) {
    const int k = k0 + 32 * c;
    const bool in = k < kend;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int r = (wave * NG + gi) * 4 + rsub;
      cd[gi] = bload_u128(rc, in ? r * (K / 2) + k / 2 : kOOB);
      sc[gi] = bload_u16(rs, in ? r * (K / 16) + k / 16 : kOOB);
    }
  };
  auto compute = [&](int k0, const uint4 (&cd)[NG], const uint32_t (&sc)[NG]) {
    const int kl = k0 + 32 * c - kbeg;          // this lane's 32 K-values in the LDS copy of x
    if (kl >= kn) return;
    uint32_t xp[MT][16];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 q = *reinterpret_cast<const uint4 *>(&xs[m * a.kchunk + kl + 8 * v]);
        xp[m][4 * v] = q.x;
        xp[m][4 * v + 1] = q.y;
        xp[m][4 * v + 2] = q.z;
        xp[m][4 * v + 3] = q.w;
      }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const uint32_t w[4] = {cd[gi].x, cd[gi].y, cd[gi].z, cd[gi].w};
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const float D = g * e4m3_value((sc[gi] >> (8 * b)) & 0x7Fu);
        uint32_t pr[8];
        e2m1_pairs(w[2 * b], *reinterpret_cast<uint32_t(*)[4]>(&pr[0]));
        e2m1_pairs(w[2 * b + 1], *reinterpret_cast<uint32_t(*)[4]>(&pr[4]));
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float ps = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pr[j]),
                                                 __builtin_bit_cast(bf16x2, xp[m][8 * b + j]), ps, false);
          acc[gi][m] = fmaf(D, ps, acc[gi][m]);
        }
      }
    }
  };

  // two steps in flight: the next step's codes load while this one is computed
  constexpr int KSTEP = 512;
  uint4 ca[NG], cb[NG];
  uint32_t sa[NG], sb[NG];
  int k0 = kbeg;
  fetch(k0, ca, sa);
  // x[m][kbeg, kend) into LDS (zeros for tokens past M), 16 bytes per thread,
  // while the first step's codes are in flight
  for (int i = tid; i < MT * (kn / 8); i += 256) {
    const int m = i / (kn / 8), k8 = (i - m * (kn / 8)) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (m < a.M) v = ld16(a.x + (size_t)m * a.ldx + kbeg + k8);
    *reinterpret_cast<uint4 *>(&xs[m * a.kchunk + k8]) = v;
  }
  __syncthreads();
  for (; k0 + KSTEP < kend; k0 += 2 * KSTEP) {
    fetch(k0 + KSTEP, cb, sb);
    compute(k0, ca, sa);
    if (k0 + 2 * KSTEP < kend) fetch(k0 + 2 * KSTEP, ca, sa);
    compute(k0 + KSTEP, cb, sb);
  }
  if (k0 < kend) compute(k0, ca, sa);

  // the row's 16 chunk lanes add their sums (butterfly within 16 lanes)
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int r = (wave * NG + gi) * 4 + rsub;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = acc[gi][m];
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o, 16);
      if (c == 0 && m < a.M && r < Rv) {
        if constexpr (PART)
          a.part[((size_t)p * a.M + m) * a.N + row0 + r] = v;
        else
          a.y[(size_t)m * a.ldy + row0 + r] = f2bf(v);
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_fp4_fold(const float *part, int S, int M, int N, uint16_t *y, int ldy) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)M * N) return;
  const int m = (int)(i / N), n = (int)(i - (long)m * N);
  float s = 0.f;
  for (int p = 0; p < S; ++p) s += part[((size_t)p * M + m) * N + n];
  y[(size_t)m * ldy + n] = f2bf(s);
}

// The kernel for M <= 4: 1 the exact per-block MFMA kernel, 2 the packed-dot
// kernel, 0 the per-weight rounding kernel (plan override).  One token on a
// weight of 2^24 codes or more takes the packed-dot kernel (large-decoder
// shapes at M = 1: stacked gate/up 30.1 us against 45.7, down 20.0 against
// 31.8, o 7.1 against 10.5); smaller weights and more tokens the MFMA kernel
// (the Gemma-3-1B shapes within 0.1-0.5 us of each other; at M = 4 the
// packed-dot kernel's per-token dot products cost more).
static int small_m_kernel(int64_t M, int64_t N, int64_t K) {
  const int dflt = (M == 1 && N * K >= (int64_t(1) << 24)) ? 2 : 1;
  const int k = debug_knob(AQ_DBG_FP4_M4, dflt);
  return k >= 0 && k <= 2 ? k : dflt;
}

void plan_fp4_linear(int64_t M, int64_t N, int64_t K, Fp4LinPlan *pl) {
  // Measured on the Gemma-3-1B decode shapes (graph replays over 26 layers):
  // two workgroups per CU of 32 rows where the rows allow (stacked gate/up
  // 13824 x 1152: 6.0 us against 7.5 with one of 64 rows), else 16-row
  // tiles; K is split only where it is long (down, K = 6912: three ranges,
  // 6.7 us against 7.6 unsplit) -- for K <= 2048 the fold launch costs more than
  // the split saves (QKV 3.4 us unsplit against 5.3, o 3.0 against 4.8).
  int NG = 1;
  for (int ng = 4; ng >= 1; --ng)
    if ((N + 16 * ng - 1) / (16 * ng) >= 400) { NG = ng; break; }
  const int ngo = debug_knob(AQ_DBG_FP4_NG, 0);   // plan overrides (tests): row groups, K splits
  if (ngo >= 1 && ngo <= 4) NG = ngo;
  const int tiles = (int)((N + 16 * NG - 1) / (16 * NG));
  int S = 1;
  if (K > 2048 && tiles < 200) {
    S = kNumCU / tiles;
    const int smax = (int)(K / 1024);
    S = S < smax ? S : smax;
    S = S < 16 ? S : 16;
    S = S > 1 ? S : 1;
  }
  // Very long rows are split into ranges of at most 8192 K-values whatever the
  // row count (the large decoder's down, 5376 x 21504: 31.9 us in three ranges
  // against 41.3 unsplit; K = 4096 and 5376 measured no better split).
  if (K >= 16384) {
    const int sl = (int)((K + 8191) / 8192);
    S = S > sl ? S : sl;
  }
  const int so = debug_knob(AQ_DBG_FP4_S, 0);
  if (so >= 1) S = so;
  if (M <= 4 && small_m_kernel(M, N, K) == 2) {   // x of a K range must fit the LDS copy
    const int sx = (int)((K + kFp4DotXCap - 1) / kFp4DotXCap);
    S = S > sx ? S : sx;
  }
  int kchunk = (int)((K + S - 1) / S);
  kchunk = (kchunk + 127) / 128 * 128;
  S = (int)((K + kchunk - 1) / kchunk);
  pl->NG = NG;
  pl->rows = 16 * NG;
  pl->ntiles = tiles;
  pl->S = S;
  pl->kchunk = kchunk;
  pl->ws_bytes = S > 1 ? kWsReserved + (size_t)S * M * N * 4 : 0;
}

template <int MT, bool PART>
static bool launch_dot(const F4Args &a, int NG, int grid, hipStream_t st) {
  const size_t lds = (size_t)MT * a.kchunk * 2;   // <= 64 KiB: kchunk <= kFp4DotXCap
  switch (NG) {
    case 1: hipLaunchKernelGGL((k_fp4_gemv_dot<MT, 1, PART>), dim3(grid), dim3(256), lds, st, a); return true;
    case 2: hipLaunchKernelGGL((k_fp4_gemv_dot<MT, 2, PART>), dim3(grid), dim3(256), lds, st, a); return true;
    case 3: hipLaunchKernelGGL((k_fp4_gemv_dot<MT, 3, PART>), dim3(grid), dim3(256), lds, st, a); return true;
    case 4: hipLaunchKernelGGL((k_fp4_gemv_dot<MT, 4, PART>), dim3(grid), dim3(256), lds, st, a); return true;
  }
  return false;
}

template <bool PART>
static bool launch_ng(const F4Args &a, int NG, int grid, hipStream_t st) {
  const int smk = small_m_kernel(a.M, a.N, a.K);
  if (a.M <= 4 && smk == 2 && a.kchunk <= kFp4DotXCap) {
    if (a.M == 1) return launch_dot<1, PART>(a, NG, grid, st);
    if (a.M == 2) return launch_dot<2, PART>(a, NG, grid, st);
    return launch_dot<4, PART>(a, NG, grid, st);
  }
  if (a.M <= 4 && a.K % 64 == 0 && smk >= 1) {   // K % 64: the 4-byte scale loads stay aligned
    switch (NG) {
      case 1: hipLaunchKernelGGL((k_fp4_gemv_m4<1, PART>), dim3(grid), dim3(512), 0, st, a); return true;
      case 2: hipLaunchKernelGGL((k_fp4_gemv_m4<2, PART>), dim3(grid), dim3(512), 0, st, a); return true;
      case 3: hipLaunchKernelGGL((k_fp4_gemv_m4<3, PART>), dim3(grid), dim3(512), 0, st, a); return true;
      case 4: hipLaunchKernelGGL((k_fp4_gemv_m4<4, PART>), dim3(grid), dim3(512), 0, st, a); return true;
    }
    return false;
  }
  switch (NG) {
    case 1: hipLaunchKernelGGL((k_fp4_gemv<1, PART>), dim3(grid), dim3(512), 0, st, a); return true;
    case 2: hipLaunchKernelGGL((k_fp4_gemv<2, PART>), dim3(grid), dim3(512), 0, st, a); return true;
    case 3: hipLaunchKernelGGL((k_fp4_gemv<3, PART>), dim3(grid), dim3(512), 0, st, a); return true;
    case 4: hipLaunchKernelGGL((k_fp4_gemv<4, PART>), dim3(grid), dim3(512), 0, st, a); return true;
  }
  return false;
}

hipError_t launch_fp4_linear(int64_t M, int64_t N, int64_t K, const void *x, int64_t ldx, const uint8_t *packed,
                             const uint8_t *scales, const float *gscale, void *y, int64_t ldy,
                             const Fp4LinPlan &pl, void *ws, hipStream_t st) {
  F4Args a = {};
  a.packed = packed;
  a.scales = scales;
  a.g = gscale;
  a.x = (const uint16_t *)x;
  a.y = (uint16_t *)y;
  a.part = pl.S > 1 ? (float *)((char *)ws + kWsReserved) : nullptr;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.ldx = (int)ldx;
  a.ldy = (int)ldy;
  a.rows = pl.rows;
  a.ntiles = pl.ntiles;
  a.S = pl.S;
  a.kchunk = pl.kchunk;
  const int units = pl.ntiles * pl.S;
  const int grid = 8 * ((units + 7) / 8);
  const bool ok = pl.S > 1 ? launch_ng<true>(a, pl.NG, grid, st) : launch_ng<false>(a, pl.NG, grid, st);
  if (!ok) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.S == 1) return e;
  const long n = (long)M * N;
  hipLaunchKernelGGL(k_fp4_fold, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (const float *)a.part, pl.S,
                     (int)M, (int)N, (uint16_t *)y, (int)ldy);
  return hipGetLastError();
}

}  // namespace aq
