// Per-element reconstruction for small batches (M <= 16 tokens), bf16 in, fp32
// accumulation, bf16 out: every weight is rebuilt inside the kernel and the
// [out_dim, in_dim] matrix is never materialised ("Execution paths", section
// "The custom op": the generated_linear semantics, one dispatch per projection
// or per fused Q/K/V and gate/up group).
//
// What it computes, for every block b of the dispatch:
//     W_eff[n, k] = bf16( s[n] * W0[n, k] + sum_j U[n, j] Vt[j, k] )
//     y[m, col_b + n] = bf16( sum_k x[m, k] * W_eff[n, k] )
// i.e. the weight the precompute path would store, rebuilt on the fly, then
// contracted with x.  Unlike the factored form there is no t = x Vt^T shared
// between workgroups: each tile rebuilds its own rows from U (its rows) and Vt
// (all of it, read from L2 by every tile).
//
// Design (gfx950):
// * A workgroup of four waves owns up to 16 x NG rows of one block over the
//   whole K or, for long K and few rows, over one of S K ranges (fp32 partials,
//   then a small kernel adds them in range order); its waves take 32-wide K
//   steps in turn.  Per step and 16-row group, the
//   rank-r product is formed on MFMA: v_mfma_f32_16x16x32_bf16 with Vt as the A
//   operand (rows = K positions) and U as the B operand (columns = weight
//   rows), twice (two 16-wide halves of the step), RC = ceil(r / 32) rank chunks
//   each.  The A rows are ordered so that a lane's two 4-value results are the
//   8 consecutive K positions it also loads of W0 (one 16-byte load) -- which
//   is exactly the B-operand layout of the contraction with x that follows.
// * The rebuilt values s W0 + U Vt are rounded once to bf16 and fed as the B
//   operand of one more v_mfma_f32_16x16x32_bf16 against 16 tokens of x (tokens
//   past M are zero).  So the x contraction and the rank-r product both run on
//   the matrix cores; the VALU does one FMA and one conversion per weight.
// * U (the tile's rows, ranks of one chunk per lane) is loaded once per tile.
//   Vt arrives per step as its rows (16 bytes per lane, coalesced) and is
//   transposed through a per-wave LDS buffer, so that a lane reads the 8 ranks
//   of one K position with one 16-byte LDS read.  Every tile reads all of Vt
//   over its K range (from L2): r K values per tile against R K of W0, which is
//   what the rebuild costs over the factored form, where t = x Vt^T is formed
//   once.
// * Loads go through buffer resources (rows past N, K past the end, tokens past
//   M, ranks past r read as zero); two register sets alternate so that one
//   step's loads are in flight while the other is computed.  Waves add their
//   partial sums in LDS in wave order: deterministic.

#include "aq_internal.h"
#include "device_common.h"

namespace aq {

struct alignas(16) RbBlk {
  const uint16_t *W0, *s, *U, *Vt;
  int N, r, col, tile0, ufast, pad[3];
};

struct RbArgs {
  const uint16_t *x;
  uint16_t *y;
  float *part;             // S > 1: [S][M][Ntot] fp32 partials
  int M, K, ldx, ldy, nblk, rows, ntiles, S, kchunk, Ntot;
  RbBlk b[kMaxBlocks];
};

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

template <int NG, int RC>
__global__ __launch_bounds__(256, 2) void k_rebuild_bf16(const RbArgs a) {
  constexpr int WAVES = 4, NT = 64 * WAVES;
  constexpr int RCV = RC > 0 ? RC : 1;
  constexpr int RP = 32 * RCV + 8;                // LDS row pitch (bf16) of the transposed Vt step
  constexpr int VL = 2 * RC;                      // 16-byte Vt loads per lane and step
  __shared__ float red[WAVES * NG * 256];
  __shared__ __attribute__((aligned(16))) uint16_t vts[WAVES][32 * RP];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j16 = lane & 15, g = lane >> 4;

  const int unit = xcd_contiguous_tile(blockIdx.x, a.ntiles * a.S);
  if (unit < 0) return;
  const int tile = unit / a.S, p = unit - tile * a.S;
  int bi = 0;
  if (a.nblk > 1 && tile >= a.b[1].tile0) bi = 1;
  if (a.nblk > 2 && tile >= a.b[2].tile0) bi = 2;
  const RbBlk B = bi == 0 ? a.b[0] : (bi == 1 ? a.b[1] : a.b[2]);
  const int K = a.K, M = a.M;
  const int row0 = (tile - B.tile0) * a.rows;
  const int Rv = min(a.rows, B.N - row0);
  const int kbeg = p * a.kchunk, kend = min(K, kbeg + a.kchunk);
  const int nsteps = (kend - kbeg + 31) / 32;

  const __amdgpu_buffer_rsrc_t rw = make_rsrc(B.W0 + (size_t)row0 * K, (uint32_t)Rv * K * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(B.Vt, RC > 0 && B.r > 0 ? (uint32_t)B.r * K * 2 : 0u);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)((M - 1) * a.ldx + K) * 2);

  // This lane's rows: row0 + 16 gi + j16 (its W0 fragments, s and U);
  // its token for the x fragment: j16.
  float sg[NG];
  bf16x8 uf[NG][RCV];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int nl = gi * 16 + j16;
    const int n = row0 + (nl < Rv ? nl : 0);
    sg[gi] = nl < Rv ? bf2f(B.s[n]) : 0.f;
#pragma unroll
    for (int c = 0; c < RCV; ++c) {
      const int j0 = 32 * c + 8 * g;
      if (RC == 0 || nl >= Rv || j0 >= B.r) {
        uf[gi][c] = zero_bf16x8();
      } else if (B.ufast) {
        uf[gi][c] = as_bf16x8(ld16(B.U + (size_t)n * B.r + j0));
      } else {
        u16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = j0 + e < B.r ? B.U[(size_t)n * B.r + j0 + e] : (uint16_t)0;
        uf[gi][c] = __builtin_bit_cast(bf16x8, v);
      }
    }
  }
  const int xoff = j16 < M ? j16 * a.ldx * 2 : kOOB;
  // Vt rows loaded by this lane per step: 16 q + lane / 4, K positions
  // 8 (lane % 4) .. + 7 of the step.
  const int vrow = lane >> 2, vkc = (lane & 3) * 8;

  f32x4 acc[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) acc[gi] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto fetch = [&](int st, bf16x8 &xf, bf16x8 (&wf)[NG], bf16x8 (&vf)[VL > 0 ? VL : 1]) {
    const int k0 = kbeg + st * 32;
    const int kl = k0 + 8 * g;
    const int koff = st < nsteps && kl < kend ? kl * 2 : kOOB;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) wf[gi] = bload16(rw, koff == kOOB ? kOOB : (gi * 16 + j16) * K * 2 + koff);
    xf = bload16(rx, koff == kOOB || xoff == kOOB ? kOOB : xoff + koff);
#pragma unroll
    for (int q = 0; q < VL; ++q) {
      const int j = 16 * q + vrow, kv = k0 + vkc;
      vf[q] = bload16(rv, st < nsteps && kv < kend && j < B.r ? (j * K + kv) * 2 : kOOB);
    }
  };
  auto compute = [&](const bf16x8 &xf, const bf16x8 (&wf)[NG], const bf16x8 (&vf)[VL > 0 ? VL : 1]) {
    bf16x8 av[2][RCV];
    if constexpr (RC > 0) {
      // Vt of this step transposed into the wave's LDS buffer: [K position][rank].
      uint16_t *vt = vts[wave];
#pragma unroll
      for (int q = 0; q < VL; ++q) {
        const u16x8 v = __builtin_bit_cast(u16x8, vf[q]);
#pragma unroll
        for (int e = 0; e < 8; ++e) vt[(vkc + e) * RP + 16 * q + vrow] = v[e];
      }
      // A operand rows: K positions 8 (i / 4) + i % 4 (first half) and + 4
      // (second half) for row i = lane % 16; ranks 32 c + 8 (lane / 16) ...
      const int kp = 8 * (j16 >> 2) + (j16 & 3);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < RC; ++c)
          av[h][c] = as_bf16x8(*reinterpret_cast<const uint4 *>(vt + (kp + 4 * h) * RP + 32 * c + 8 * g));
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      f32x4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (RC > 0) {
#pragma unroll
        for (int c = 0; c < RC; ++c) {
          d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[0][c], uf[gi][c], d0, 0, 0, 0);
          d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[1][c], uf[gi][c], d1, 0, 0, 0);
        }
      }
      // rebuilt weights of row 16 gi + j16 at K positions 8 (lane / 16) + 0..7
      const u16x8 w0 = __builtin_bit_cast(u16x8, wf[gi]);
      const float d[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
      bf16x8 wb;
#pragma unroll
      for (int e = 0; e < 8; ++e) wb[e] = (__bf16)__builtin_fmaf(sg[gi], bf2f(w0[e]), d[e]);
      acc[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf, wb, acc[gi], 0, 0, 0);
    }
  };

  // Two register sets in turn (as the streaming decode kernel); a wave fetches
  // exactly its own steps.
  const int nmine = wave < nsteps ? (nsteps - 1 - wave) / WAVES + 1 : 0;
  bf16x8 xa, xb, wa[NG], wb_[NG], va[VL > 0 ? VL : 1], vb[VL > 0 ? VL : 1];
  if (nmine > 0) fetch(wave, xa, wa, va);
  int i = 0;
  for (; i + 2 < nmine; i += 2) {
    fetch(wave + (i + 1) * WAVES, xb, wb_, vb);
    __builtin_amdgcn_sched_barrier(0);
    compute(xa, wa, va);
    __builtin_amdgcn_sched_barrier(0);
    fetch(wave + (i + 2) * WAVES, xa, wa, va);
    __builtin_amdgcn_sched_barrier(0);
    compute(xb, wb_, vb);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (i + 1 < nmine) {
    fetch(wave + (i + 1) * WAVES, xb, wb_, vb);
    __builtin_amdgcn_sched_barrier(0);
    compute(xa, wa, va);
    __builtin_amdgcn_sched_barrier(0);
    compute(xb, wb_, vb);
  } else if (i < nmine) {
    compute(xa, wa, va);
  }

  // Partial sums per wave into LDS, added in wave order.  MFMA output layout:
  // lane holds row (output column) 16 gi + lane % 16, tokens 4 (lane / 16) + v.
  {
    float *slot = red + wave * NG * 256;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int v = 0; v < 4; ++v) slot[(gi * 4 + v) * 64 + lane] = acc[gi][v];
  }
  __syncthreads();
  for (int e = tid; e < M * Rv; e += NT) {
    const int m = e / Rv, nl = e - m * Rv;
    const int gi = nl >> 4, idx = (gi * 4 + (m & 3)) * 64 + ((m >> 2) << 4) + (nl & 15);
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += red[w * NG * 256 + idx];
    if (a.S > 1)
      a.part[((size_t)p * M + m) * a.Ntot + B.col + row0 + nl] = v;
    else
      a.y[(size_t)m * a.ldy + B.col + row0 + nl] = f2bf(v);
  }
}

// y = bf16(sum of the S partials, in range order).
__global__ __launch_bounds__(256) void k_rebuild_fold(const float *part, int S, int M, int N, uint16_t *y, int ldy) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)M * N) return;
  const int m = (int)(i / N), n = (int)(i - (long)m * N);
  float v[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) v[q] = q < S ? part[((size_t)q * M + m) * N + n] : 0.f;
  float sum = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q)
    if (q < S) sum += v[q];
  y[(size_t)m * ldy + n] = f2bf(sum);
}

// ---------------------------------------------------------------- host side

void plan_rebuild(const Recon &rq, RebuildPlan *pl) {
  int rmax = 0;
  for (int b = 0; b < rq.nblk; ++b) rmax = rq.blk[b].r > rmax ? (int)rq.blk[b].r : rmax;
  pl->RC = (rmax + 31) / 32;
  // Rows per tile: any count up to 64 (rows past it lie outside the W0
  // resource), the fewest whole rounds of tiles over the 256 CUs, then the
  // most rows: 2 x 6912 rows become 256 tiles of 54, 1536 rows 256 of 6,
  // 2 x 21504 rows 768 of 56.
  // Cost model as the streaming decode kernel's (fixed ~0.8 us per work unit,
  // ~21.5 GB/s per CU when all stream), with every tile also reading its K
  // range of Vt (r rows, from L2, counted at 0.7 of a W0 row) and, with K
  // split over S ranges, the fold launch (~3.7 us).
  auto tiles_of = [&](int R) {
    long t = 0;
    for (int b = 0; b < rq.nblk; ++b) t += (rq.blk[b].N + R - 1) / R;
    return t;
  };
  const double rv = 0.7 * 32.0 * pl->RC;
  int R = 64, S = 1;
  double best = 1e30;
  const int smax = rq.K / 1024 > 1 ? (rq.K / 1024 < 16 ? (int)(rq.K / 1024) : 16) : 1;
  for (int c = 4; c <= 64; ++c) {
    const long t = tiles_of(c);
    for (int sc = 1; sc <= smax; ++sc) {
      const int kc = (int)(((rq.K + sc - 1) / sc + 31) / 32 * 32);
      if ((rq.K + kc - 1) / kc != sc) continue;
      const double cost = (double)((t * sc + kNumCU - 1) / kNumCU) * (0.8 + (c + rv) * kc * 2.0 / 21500.0) +
                          (sc > 1 ? 3.7 : 0.0);
      if (cost <= best) { best = cost; R = c; S = sc; }
    }
  }
  const int ng_o = debug_knob(AQ_DBG_REBUILD_NG, 0);
  if (ng_o >= 1 && ng_o <= 4) R = 16 * ng_o;
  const int r_o = debug_knob(AQ_DBG_REBUILD_ROWS, 0);
  if (r_o >= 1 && r_o <= 64) R = r_o;
  const int s_o = debug_knob(AQ_DBG_REBUILD_S, 0);
  if (s_o >= 1 && s_o <= 16) S = s_o;
  int kchunk = (int)(((rq.K + S - 1) / S + 31) / 32 * 32);
  S = (int)((rq.K + kchunk - 1) / kchunk);
  pl->S = S;
  pl->kchunk = kchunk;
  pl->ws_bytes = S > 1 ? kWsReserved + (size_t)S * rq.M * rq.Ntot * 4 : 0;
  pl->rows = R;
  pl->NG = (R + 15) / 16;
  int t0 = 0;
  for (int b = 0; b < rq.nblk; ++b) {
    pl->tile0[b] = t0;
    t0 += (int)((rq.blk[b].N + R - 1) / R);
  }
  pl->ntiles = t0;
}

template <int NG>
static bool launch_rc(const RbArgs &a, int RC, int grid, hipStream_t st) {
  switch (RC) {
    case 0: hipLaunchKernelGGL((k_rebuild_bf16<NG, 0>), dim3(grid), dim3(256), 0, st, a); return true;
    case 1: hipLaunchKernelGGL((k_rebuild_bf16<NG, 1>), dim3(grid), dim3(256), 0, st, a); return true;
    case 2: hipLaunchKernelGGL((k_rebuild_bf16<NG, 2>), dim3(grid), dim3(256), 0, st, a); return true;
  }
  return false;
}

hipError_t launch_rebuild(const Recon &rq, const RebuildPlan &pl, void *ws, hipStream_t st) {
  RbArgs a = {};
  a.S = pl.S;
  a.kchunk = pl.kchunk;
  a.Ntot = (int)rq.Ntot;
  a.part = pl.S > 1 ? (float *)((char *)ws + kWsReserved) : nullptr;
  a.x = (const uint16_t *)rq.x;
  a.y = (uint16_t *)rq.y;
  a.M = (int)rq.M;
  a.K = (int)rq.K;
  a.ldx = (int)rq.ldx;
  a.ldy = (int)rq.ldy;
  a.nblk = rq.nblk;
  a.rows = pl.rows;
  a.ntiles = pl.ntiles;
  for (int b = 0; b < rq.nblk; ++b) {
    const Proj &P = rq.blk[b];
    RbBlk &d = a.b[b];
    d.W0 = (const uint16_t *)P.W0;
    d.s = (const uint16_t *)P.s;
    d.U = (const uint16_t *)P.U;
    d.Vt = (const uint16_t *)P.Vt;
    d.N = (int)P.N;
    d.r = (int)P.r;
    d.col = (int)P.col;
    d.tile0 = pl.tile0[b];
    d.ufast = (P.r % 8 == 0) && (((uintptr_t)P.U & 15) == 0);
  }
  const int grid = 8 * ((pl.ntiles * pl.S + 7) / 8);
  bool ok = false;
  switch (pl.NG) {
    case 1: ok = launch_rc<1>(a, pl.RC, grid, st); break;
    case 2: ok = launch_rc<2>(a, pl.RC, grid, st); break;
    case 3: ok = launch_rc<3>(a, pl.RC, grid, st); break;
    case 4: ok = launch_rc<4>(a, pl.RC, grid, st); break;
  }
  if (!ok) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.S == 1) return e;
  const long n = (long)rq.M * rq.Ntot;
  // the partials hold all blocks' columns contiguously: fold them into y
  hipLaunchKernelGGL(k_rebuild_fold, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (const float *)a.part,
                     pl.S, (int)rq.M, (int)rq.Ntot, a.y, (int)rq.ldy);
  return hipGetLastError();
}

}  // namespace aq
