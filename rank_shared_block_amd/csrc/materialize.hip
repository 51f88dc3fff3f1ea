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
// * A workgroup owns a block of 512 columns (a wave 32 * SETS of them, SETS = 4)
//   and a range of rows.  MFMA column c of "set" e stands for actual column
//   c0 + SETS * c + e, so after SETS MFMAs a lane holds SETS consecutive columns
//   of each of its 16 rows and reads W0 / writes W_eff with 8-byte accesses.
//   The Vt block (K-contiguous, but needed rank-contiguous as an MFMA operand)
//   is staged once in LDS transposed, read back as one 16-byte fragment per
//   rank chunk and reused for every row of the range.  The first row block's W0,
//   s and U are requested before the staging so that the two round trips
//   overlap.
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
__global__ __launch_bounds__(256, 2) void k_materialize_bf16(const MatArgs a) {
  constexpr int CW = 32 * SETS;             // columns per wave
  constexpr int CB = 4 * CW;                // columns per workgroup
  constexpr int RP = 16 * JC + 8;           // LDS row (one column of Vt), padded
  // Vt[:, c0 : c0 + CB] stored transposed: vts[c][j], so that the 8 ranks of one
  // MFMA operand are one 16-byte LDS read.
  __shared__ __attribute__((aligned(16))) uint16_t vts[CB * RP];
  const uint16_t *W0 = (const uint16_t *)a.W0, *S = (const uint16_t *)a.s;
  const uint16_t *U = (const uint16_t *)a.U, *Vt = (const uint16_t *)a.Vt;
  uint16_t *out = (uint16_t *)a.out;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, hi = lane >> 5;
  const int K = a.K, r = a.r, N = a.N;
  const int cb0 = blockIdx.x * CB;
  const int c0 = cb0 + wave * CW;
  const int kl = c0 + SETS * c32;            // this lane's SETS consecutive columns
  const bool colok = kl < K;                 // K % SETS == 0, so all SETS or none
  const int kloc = wave * CW + SETS * c32;   // ... their position in the LDS tile

  // Operands of one 32-row block: W0 and s of this lane's 16 output rows, U of
  // its A-operand row.  The first block's are requested before the Vt staging
  // so that the two memory round trips overlap.
  uint2 w[16];
  float sv[16];
  bf16x8 au[JC];
  auto fetch_rows = [&](int n0, int ne) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int n = n0 + 8 * (v >> 2) + 4 * hi + (v & 3);
      const bool ok = colok && n < ne;
      w[v] = ok ? *reinterpret_cast<const uint2 *>(W0 + (size_t)n * K + kl) : make_uint2(0, 0);
      sv[v] = ok ? bf2f(S[n]) : 0.f;
    }
    const int na = n0 + c32;
#pragma unroll
    for (int jc = 0; jc < JC; ++jc) {
      const int j = jc * 16 + 8 * hi;
      if (na >= N || j >= r) {
        au[jc] = zero_bf16x8();
      } else if (a.ufast) {
        au[jc] = as_bf16x8(ld16(U + (size_t)na * r + j));
      } else {
        uint16_t v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = (j + q < r) ? U[(size_t)na * r + j + q] : (uint16_t)0;
        uint4 u;
        u.x = v[0] | ((uint32_t)v[1] << 16);
        u.y = v[2] | ((uint32_t)v[3] << 16);
        u.z = v[4] | ((uint32_t)v[5] << 16);
        u.w = v[6] | ((uint32_t)v[7] << 16);
        au[jc] = as_bf16x8(u);
      }
    }
  };
  const int nb0 = blockIdx.y * a.rows_per_wg;
  if (nb0 < N) fetch_rows(nb0, min(N, nb0 + a.rows_per_wg));

  // Stage Vt transposed (zeros past r or K).  Consecutive threads take
  // consecutive ranks of one 8-column chunk, so their 2-byte LDS writes fall in
  // consecutive banks.
  for (int i = tid; i < 16 * JC * (CB / 8); i += 256) {
    const int j = i % (16 * JC), c = (i / (16 * JC)) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j < r && cb0 + c < K) v = ld16(Vt + (size_t)j * K + cb0 + c);
    const uint32_t q4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) vts[(c + q) * RP + j] = (uint16_t)(q4[q >> 1] >> ((q & 1) * 16));
  }
  __syncthreads();

  // B operands (Vt): set e, rank chunk jc -> ranks jc*16 + 8*hi .. +7 of column kl + e.
  bf16x8 bv[SETS][JC];
#pragma unroll
  for (int e = 0; e < SETS; ++e)
#pragma unroll
    for (int jc = 0; jc < JC; ++jc)
      bv[e][jc] = as_bf16x8(*reinterpret_cast<const uint4 *>(&vts[(kloc + e) * RP + jc * 16 + 8 * hi]));

  // Every lane stays active through the MFMAs (they read all 64 lanes'
  // operands); lanes past K only skip their loads and stores of W0 / W_eff.
  for (int nb = nb0; nb < N; nb += gridDim.y * a.rows_per_wg) {
    const int ne = min(N, nb + a.rows_per_wg);
    for (int n0 = nb; n0 < ne; n0 += 32) {
      if (n0 != nb0) fetch_rows(n0, ne);
      f32x16 acc[SETS];
#pragma unroll
      for (int e = 0; e < SETS; ++e)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[e][v] = 0.f;
#pragma unroll
      for (int jc = 0; jc < JC; ++jc) {
        if (jc * 16 >= r) break;
#pragma unroll
        for (int e = 0; e < SETS; ++e)
          acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(au[jc], bv[e][jc], acc[e], 0, 0, 0);
      }
      if (!colok) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int n = n0 + 8 * (v >> 2) + 4 * hi + (v & 3);
        if (n >= ne) continue;
        uint2 o;
        o.x = f2bf(fmaf(sv[v], bf2f((uint16_t)w[v].x), acc[0][v])) |
              ((uint32_t)f2bf(fmaf(sv[v], bf2f((uint16_t)(w[v].x >> 16)), acc[1][v])) << 16);
        o.y = f2bf(fmaf(sv[v], bf2f((uint16_t)w[v].y), acc[2][v])) |
              ((uint32_t)f2bf(fmaf(sv[v], bf2f((uint16_t)(w[v].y >> 16)), acc[3][v])) << 16);
        *reinterpret_cast<uint2 *>(out + (size_t)n * a.ldw + kl) = o;
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
  // Column blocks of 512 (4 waves x 128); row blocks sized so that the grid has
  // about two workgroups per CU, each amortising its staged Vt tile over as many
  // rows as possible.
  constexpr int SETS = 4;
  const int colblocks = (int)((K + 4 * 32 * SETS - 1) / (4 * 32 * SETS));
  long rows = (p.N * colblocks + 2 * kNumCU - 1) / (2 * kNumCU);
  rows = (rows + 31) / 32 * 32;
  if (rows < 32) rows = 32;
  a.rows_per_wg = (int)rows;
  const long nrb = (p.N + rows - 1) / rows;
  const unsigned gy = (unsigned)(nrb < 65535 ? nrb : 65535);
  if (p.r <= 64) {
    dim3 grid((unsigned)colblocks, gy);
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
