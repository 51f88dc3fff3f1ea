// Effective-weight materialisation: W_eff = diag(s) W0 + U Vt, fp32 accumulation,
// one rounding to the storage dtype.  "Execution paths", section
// "Precompute-outside" (rebuilt once at load); "How attnquant works", section
// "The reconstruction identity".
//
// bf16 kernel (gfx950):
// * Streaming W0 in and W_eff out is the bound (2 + 2 bytes per element); the
//   rank-r product costs 2 r flop per element, which at r = 64 would exceed the
//   fp32 VALU roofline, so it runs on v_mfma_f32_32x32x16_bf16 with U as the A
//   operand (row n, 8 contiguous rank values per lane) and Vt as the B operand.
// * A wave owns a strip of 32 * SETS columns.  MFMA column c of "set" e stands for
//   actual column c0 + SETS * c + e, so after SETS MFMAs a lane holds SETS
//   consecutive columns of each of its 16 rows and reads W0 / writes W_eff with
//   SETS * 2-byte accesses instead of 2-byte ones.  The Vt operand of the strip
//   (strided in K) is gathered once into registers and reused for every row
//   block the wave visits.
// * diag(s) W0 is added in fp32 with one fused multiply-add per element; with
//   r = 0 (or U = Vt = 0) the accumulator is +0 and the result is one rounding of
//   the exact product s * w, i.e. bit-exact.
//
// fp32 kernel: one thread per element, rank loop in fp32 FMAs, then one fused
// multiply-add with s * w.

#include "aq_internal.h"
#include "device_common.h"

namespace aq {

struct MatArgs {
  const void *W0, *s, *U, *Vt;
  void *out;
  int N, K, r, ldw, rows_per_wg, ufast;
};

template <int SETS, int JC>
__global__ __launch_bounds__(256) void k_materialize_bf16(const MatArgs a) {
  const uint16_t *W0 = (const uint16_t *)a.W0, *S = (const uint16_t *)a.s;
  const uint16_t *U = (const uint16_t *)a.U, *Vt = (const uint16_t *)a.Vt;
  uint16_t *out = (uint16_t *)a.out;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, hi = lane >> 5;
  const int K = a.K, r = a.r, N = a.N;
  const int c0 = (blockIdx.x * 4 + wave) * (32 * SETS);
  if (c0 >= K) return;                     // no barriers below: a wave may leave alone
  const int kl = c0 + SETS * c32;          // this lane's SETS consecutive columns
  const bool colok = kl < K;               // K % SETS == 0, so all SETS or none

  bf16x8 bv[SETS][JC];
#pragma unroll
  for (int e = 0; e < SETS; ++e)
#pragma unroll
    for (int jc = 0; jc < JC; ++jc) {
      uint16_t v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = jc * 16 + 8 * hi + q;
        v[q] = (j < r && colok) ? Vt[(size_t)j * K + kl + e] : (uint16_t)0;
      }
      uint4 u;
      u.x = v[0] | ((uint32_t)v[1] << 16);
      u.y = v[2] | ((uint32_t)v[3] << 16);
      u.z = v[4] | ((uint32_t)v[5] << 16);
      u.w = v[6] | ((uint32_t)v[7] << 16);
      bv[e][jc] = as_bf16x8(u);
    }

  for (int nb = blockIdx.y * a.rows_per_wg; nb < N; nb += gridDim.y * a.rows_per_wg) {
  const int ne = min(N, nb + a.rows_per_wg);
  for (int n0 = nb; n0 < ne; n0 += 32) {
    f32x16 acc[SETS];
#pragma unroll
    for (int e = 0; e < SETS; ++e)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[e][v] = 0.f;
    const int na = n0 + c32;               // row of this lane's A operand
#pragma unroll
    for (int jc = 0; jc < JC; ++jc) {
      if (jc * 16 >= r) break;
      const int j = jc * 16 + 8 * hi;
      bf16x8 au;
      if (na >= N || j >= r) {
        au = zero_bf16x8();
      } else if (a.ufast) {
        au = as_bf16x8(ld16(U + (size_t)na * r + j));
      } else {
        uint16_t v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = (j + q < r) ? U[(size_t)na * r + j + q] : (uint16_t)0;
        uint4 u;
        u.x = v[0] | ((uint32_t)v[1] << 16);
        u.y = v[2] | ((uint32_t)v[3] << 16);
        u.z = v[4] | ((uint32_t)v[5] << 16);
        u.w = v[6] | ((uint32_t)v[7] << 16);
        au = as_bf16x8(u);
      }
#pragma unroll
      for (int e = 0; e < SETS; ++e)
        acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(au, bv[e][jc], acc[e], 0, 0, 0);
    }
    if (!colok) continue;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int n = n0 + 8 * (v >> 2) + 4 * hi + (v & 3);
      if (n >= ne) continue;
      const float sn = bf2f(S[n]);
      const uint16_t *wr = W0 + (size_t)n * K + kl;
      uint16_t *orow = out + (size_t)n * a.ldw + kl;
      if constexpr (SETS == 4) {
        const uint2 w = *reinterpret_cast<const uint2 *>(wr);
        uint2 o;
        o.x = f2bf(fmaf(sn, bf2f((uint16_t)w.x), acc[0][v])) |
              ((uint32_t)f2bf(fmaf(sn, bf2f((uint16_t)(w.x >> 16)), acc[1][v])) << 16);
        o.y = f2bf(fmaf(sn, bf2f((uint16_t)w.y), acc[2][v])) |
              ((uint32_t)f2bf(fmaf(sn, bf2f((uint16_t)(w.y >> 16)), acc[3][v])) << 16);
        *reinterpret_cast<uint2 *>(orow) = o;
      } else {
#pragma unroll
        for (int e = 0; e < SETS; ++e) orow[e] = f2bf(fmaf(sn, bf2f(wr[e]), acc[e][v]));
      }
    }
  }
  }
}

// Ranks above 16 * JC_MAX: same arithmetic, Vt operand gathered per row block.
__global__ __launch_bounds__(256) void k_materialize_bf16_highrank(const MatArgs a) {
  const uint16_t *W0 = (const uint16_t *)a.W0, *S = (const uint16_t *)a.s;
  const uint16_t *U = (const uint16_t *)a.U, *Vt = (const uint16_t *)a.Vt;
  uint16_t *out = (uint16_t *)a.out;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, hi = lane >> 5;
  const int K = a.K, r = a.r, N = a.N;
  const int c0 = (blockIdx.x * 4 + wave) * 32;
  if (c0 >= K) return;
  const int k = c0 + c32;
  const bool colok = k < K;
  for (int nb = blockIdx.y * a.rows_per_wg; nb < N; nb += gridDim.y * a.rows_per_wg) {
  const int ne = min(N, nb + a.rows_per_wg);
  for (int n0 = nb; n0 < ne; n0 += 32) {
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    const int na = n0 + c32;
    for (int jc = 0; jc * 16 < r; ++jc) {
      uint16_t va[8], vb[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = jc * 16 + 8 * hi + q;
        va[q] = (na < N && j < r) ? U[(size_t)na * r + j] : (uint16_t)0;
        vb[q] = (colok && j < r) ? Vt[(size_t)j * K + k] : (uint16_t)0;
      }
      uint4 ua, ub;
      ua.x = va[0] | ((uint32_t)va[1] << 16); ua.y = va[2] | ((uint32_t)va[3] << 16);
      ua.z = va[4] | ((uint32_t)va[5] << 16); ua.w = va[6] | ((uint32_t)va[7] << 16);
      ub.x = vb[0] | ((uint32_t)vb[1] << 16); ub.y = vb[2] | ((uint32_t)vb[3] << 16);
      ub.z = vb[4] | ((uint32_t)vb[5] << 16); ub.w = vb[6] | ((uint32_t)vb[7] << 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ua), as_bf16x8(ub), acc, 0, 0, 0);
    }
    if (!colok) continue;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int n = n0 + 8 * (v >> 2) + 4 * hi + (v & 3);
      if (n >= ne) continue;
      out[(size_t)n * a.ldw + k] = f2bf(fmaf(bf2f(S[n]), bf2f(W0[(size_t)n * K + k]), acc[v]));
    }
  }
  }
}

__global__ __launch_bounds__(256) void k_materialize_f32(const MatArgs a) {
  const float *W0 = (const float *)a.W0, *S = (const float *)a.s;
  const float *U = (const float *)a.U, *Vt = (const float *)a.Vt;
  float *out = (float *)a.out;
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= a.K) return;
  for (int n = blockIdx.y; n < a.N; n += gridDim.y) {
    float acc = 0.f;
    for (int j = 0; j < a.r; ++j) acc = fmaf(U[(size_t)n * a.r + j], Vt[(size_t)j * a.K + k], acc);
    out[(size_t)n * a.ldw + k] = fmaf(S[n], W0[(size_t)n * a.K + k], acc);
  }
}

hipError_t launch_materialize(aq_dtype dt, int64_t K, const Proj &p, void *w, int64_t ldw,
                              hipStream_t st) {
  MatArgs a = {};
  a.W0 = p.W0;
  a.s = p.s;
  a.U = p.U;
  a.Vt = p.Vt;
  a.out = w;
  a.N = (int)p.N;
  a.K = (int)K;
  a.r = (int)p.r;
  a.ldw = (int)ldw;
  a.ufast = (p.r % 8 == 0) && (((uintptr_t)p.U & 15) == 0);
  if (dt == AQ_F32) {
    dim3 grid((unsigned)((K + 255) / 256), (unsigned)(p.N < 65535 ? p.N : 65535));
    hipLaunchKernelGGL(k_materialize_f32, grid, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  // Row blocks per workgroup: enough workgroups to cover 256 CUs a few times over.
  constexpr int SETS = 4;
  const int colblocks_lo = (int)((K + 4 * 32 * SETS - 1) / (4 * 32 * SETS));
  int rows = 256;
  while (rows > 32 && (long)colblocks_lo * ((p.N + rows - 1) / rows) < 4 * kNumCU) rows /= 2;
  a.rows_per_wg = rows;
  const long nrb = (p.N + rows - 1) / rows;
  const unsigned gy = (unsigned)(nrb < 65535 ? nrb : 65535);
  if (p.r <= 64) {
    dim3 grid((unsigned)colblocks_lo, gy);
    if (p.r <= 16)
      hipLaunchKernelGGL((k_materialize_bf16<SETS, 1>), grid, dim3(256), 0, st, a);
    else if (p.r <= 32)
      hipLaunchKernelGGL((k_materialize_bf16<SETS, 2>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((k_materialize_bf16<SETS, 4>), grid, dim3(256), 0, st, a);
  } else {
    dim3 grid((unsigned)((K + 127) / 128), gy);
    hipLaunchKernelGGL(k_materialize_bf16_highrank, grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace aq
