// Tiled MFMA reconstruction for large batches (prefill), bf16 in, fp32
// accumulation, bf16 out.
//
// What it computes ("How attnquant works", section "The reconstruction identity";
// "Execution paths", section "The GEMM formulation"):
//     t          = x Vt_b^T                        (rank-r down-projection)
//     y[:, col_b + n] = s_b[n] * (x W0_b^T)[:, n] + (t U_b^T)[:, n]
// The pages run this as stock GEMMs: one over [W0^T, V] and one up-projection
// (block-diagonal for Q/K/V and gate/up), then an elementwise combine.  Here:
// * pass 1 (same kernel, plain store): t = x [Vt_q; Vt_k; ...]^T for all blocks
//   of the dispatch, one bf16 [M, sum r] buffer in the caller's workspace;
// * pass 2: the W0 down-contraction on v_mfma_f32_32x32x16_bf16 with 128x128
//   output tiles staged through LDS in 64-deep K slices, then an in-register
//   epilogue: acc *= s[n], acc += t U^T as r/16 further MFMA k-steps (t is the A
//   operand, U the B operand, both read straight from L2), and one rounding to
//   bf16.  t is an MFMA operand and is therefore held in bf16; everything else is
//   fp32 until the final store.
// * Output tiles of all blocks of a fused dispatch form one grid; each tile
//   belongs to exactly one block, so U is applied block-diagonally.  Tiles are
//   ordered m-fastest within a block and handed to XCDs in contiguous ranges, so
//   that the workgroups of one XCD share the W0 rows of a column tile in L2.

#include "aq_internal.h"
#include "device_common.h"

namespace aq {

namespace {
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDSS = BK + 8;    // padded row stride (elements): conflict-free 16-byte reads
}  // namespace

struct PfBlk {
  const uint16_t *W, *s, *U;
  int N;       // valid rows of W (output columns computed)
  int Nst;     // output columns stored (>= N: padding columns are stored as 0)
  int r, col, tcol, ntn, tile0, ufast;
};

struct PfArgs {
  const uint16_t *x;
  uint16_t *y;
  const uint16_t *t;
  int ldx, ldy, ldt, M, K, nblk, ntm, ntiles, epi;
  PfBlk b[kMaxBlocks];
};

__device__ __forceinline__ bf16x8 load_u8(const PfBlk &B, int n, int j) {
  // U[n, j .. j+7], zero beyond r
  if (B.ufast) {
    return j < B.r ? as_bf16x8(ld16(B.U + (size_t)n * B.r + j)) : zero_bf16x8();
  }
  uint16_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (j + e < B.r) ? B.U[(size_t)n * B.r + j + e] : (uint16_t)0;
  uint4 u;
  u.x = v[0] | ((uint32_t)v[1] << 16);
  u.y = v[2] | ((uint32_t)v[3] << 16);
  u.z = v[4] | ((uint32_t)v[5] << 16);
  u.w = v[6] | ((uint32_t)v[7] << 16);
  return as_bf16x8(u);
}

__global__ __launch_bounds__(256, 2) void k_prefill_bf16(const PfArgs a) {
  __shared__ uint16_t As[BM * LDSS];
  __shared__ uint16_t Bs[BN * LDSS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = xcd_contiguous_tile(blockIdx.x, a.ntiles);
  if (tile < 0) return;
  int bi = 0;
  if (a.nblk > 1 && tile >= a.b[1].tile0) bi = 1;
  if (a.nblk > 2 && tile >= a.b[2].tile0) bi = 2;
  const PfBlk B = bi == 0 ? a.b[0] : (bi == 1 ? a.b[1] : a.b[2]);

  const int tin = tile - B.tile0;
  const int tn = tin / a.ntm, tm = tin - tn * a.ntm;
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = a.M, K = a.K;

  // Global -> register loader: thread owns rows lrow + 32 i, 16-byte chunk lch.
  const int lrow = tid >> 3, lch = (tid & 7) * 8;
  uint4 ra[4], rb[4];
  auto gload = [&](int k0) {
    const int gk = k0 + lch;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = lrow + 32 * i;
      const int gm = m0 + row, gn = n0 + row;
      ra[i] = (gm < M && gk < K) ? ld16(a.x + (size_t)gm * a.ldx + gk) : make_uint4(0, 0, 0, 0);
      rb[i] = (gn < B.N && gk < K) ? ld16(B.W + (size_t)gn * K + gk) : make_uint4(0, 0, 0, 0);
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lhi = lane >> 5;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = (K + BK - 1) / BK;
  gload(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = lrow + 32 * i;
      *reinterpret_cast<uint4 *>(&As[row * LDSS + lch]) = ra[i];
      *reinterpret_cast<uint4 *>(&Bs[row * LDSS + lch]) = rb[i];
    }
    __syncthreads();
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + l32;
        af[i] = as_bf16x8(*reinterpret_cast<const uint4 *>(&As[row * LDSS + kk + 8 * lhi]));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wn * 64 + j * 32 + l32;
        bfr[j] = as_bf16x8(*reinterpret_cast<const uint4 *>(&Bs[row * LDSS + kk + 8 * lhi]));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  if (a.epi) {
    // acc *= s[n]; acc += t U^T over the block's rank.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + l32;
      const float sv = n < B.N ? bf2f(B.s[n]) : 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[i][j] *= sv;
    }
    for (int jc = 0; jc < B.r; jc += 16) {
      const int jj = jc + 8 * lhi;
      bf16x8 ta[2], ub[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = m0 + wm * 64 + i * 32 + l32;
        ta[i] = m < M ? as_bf16x8(ld16(a.t + (size_t)m * a.ldt + B.tcol + jj)) : zero_bf16x8();
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 64 + j * 32 + l32;
        ub[j] = n < B.N ? load_u8(B, n, jj) : zero_bf16x8();
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[i], ub[j], acc[i][j], 0, 0, 0);
    }
  }

  // Store.  MFMA 32x32 output layout: lane holds column (lane % 32) and rows
  // 8 (v / 4) + 4 (lane / 32) + (v % 4), v = 0..15.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + l32;
      if (n >= B.Nst) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * lhi + (v & 3);
        if (m < M) a.y[(size_t)m * a.ldy + B.col + n] = f2bf(acc[i][j][v]);
      }
    }
}

// ---------------------------------------------------------------- host side

void plan_prefill(const Recon &rq, PrefillPlan *pl) {
  int c = 0;
  for (int b = 0; b < rq.nblk; ++b) {
    pl->tcol[b] = c;
    c += (int)((rq.blk[b].r + 15) / 16 * 16);
  }
  pl->ldt = c;
  pl->ws_bytes = c > 0 ? kWsReserved + (size_t)rq.M * c * 2 : 0;
}

static hipError_t run(PfArgs &a, hipStream_t st) {
  int t0 = 0;
  for (int b = 0; b < a.nblk; ++b) {
    a.b[b].tile0 = t0;
    a.b[b].ntn = (a.b[b].Nst + BN - 1) / BN;
    t0 += a.b[b].ntn * a.ntm;
  }
  a.ntiles = t0;
  if (t0 == 0) return hipSuccess;
  const int grid = 8 * ((t0 + 7) / 8);
  hipLaunchKernelGGL(k_prefill_bf16, dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_prefill(const Recon &rq, const PrefillPlan &pl, void *ws, hipStream_t st) {
  uint16_t *tbuf = pl.ldt > 0 ? (uint16_t *)((char *)ws + kWsReserved) : nullptr;
  PfArgs a = {};
  a.x = (const uint16_t *)rq.x;
  a.ldx = (int)rq.ldx;
  a.M = (int)rq.M;
  a.K = (int)rq.K;
  a.nblk = rq.nblk;
  a.ntm = (a.M + BM - 1) / BM;

  // pass 1: t = x Vt^T for every block with r > 0 (columns padded to 16 with zeros)
  if (pl.ldt > 0) {
    PfArgs t = a;
    t.y = tbuf;
    t.ldy = pl.ldt;
    t.epi = 0;
    t.nblk = 0;
    for (int b = 0; b < rq.nblk; ++b) {
      if (rq.blk[b].r == 0) continue;
      PfBlk &d = t.b[t.nblk++];
      d = PfBlk{};
      d.W = (const uint16_t *)rq.blk[b].Vt;
      d.N = (int)rq.blk[b].r;
      d.Nst = (int)((rq.blk[b].r + 15) / 16 * 16);
      d.col = pl.tcol[b];
    }
    hipError_t e = run(t, st);
    if (e != hipSuccess) return e;
  }

  // pass 2: y = s * (x W0^T) + t U^T
  a.y = (uint16_t *)rq.y;
  a.ldy = (int)rq.ldy;
  a.t = tbuf;
  a.ldt = pl.ldt;
  a.epi = 1;
  for (int b = 0; b < rq.nblk; ++b) {
    const Proj &P = rq.blk[b];
    PfBlk &d = a.b[b];
    d.W = (const uint16_t *)P.W0;
    d.s = (const uint16_t *)P.s;
    d.U = (const uint16_t *)P.U;
    d.N = (int)P.N;
    d.Nst = (int)P.N;
    d.r = (int)P.r;
    d.col = (int)P.col;
    d.tcol = pl.tcol[b];
    d.ufast = (P.r % 8 == 0) && (((uintptr_t)P.U & 15) == 0);
  }
  return run(a, st);
}

}  // namespace aq
