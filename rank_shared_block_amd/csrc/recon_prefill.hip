// Tiled MFMA reconstruction for large batches (prefill), bf16 in, fp32
// accumulation, bf16 out.
//
// What it computes ("How attnquant works", section "The reconstruction identity";
// "Execution paths", section "The GEMM formulation"):
//     t                 = x Vt_b^T                       (rank-r down-projection)
//     y[:, col_b + n]   = s_b[n] * (x W0_b^T)[:, n] + (t U_b^T)[:, n]
// The pages run this as stock GEMMs (one over [W0^T, V], one block-diagonal
// up-projection) plus an elementwise combine.  Here:
// * pass 1: t = x [Vt_q; Vt_k; ...]^T for every block of the dispatch with the
//   same GEMM kernel, into a bf16 [M, sum r] buffer of the caller's workspace.
//   The contraction is long and the output narrow, so it is split along K into
//   fp32 partials over enough workgroups to cover the CUs, and a small kernel
//   folds them (in split order) into t;
// * pass 2: the W0 contraction on v_mfma_f32_32x32x16_bf16 and an in-register
//   epilogue: acc *= s[n], then acc += t U^T as r/16 further MFMA k-steps (t is
//   the A operand, U the B operand, both read from L2), then one rounding to
//   bf16.  t is an MFMA operand and therefore held in bf16; everything else is
//   fp32 until the final store.
//
// GEMM design (gfx950):
// * BM x BN output tile per workgroup of 4 waves (2 x 2), each wave a
//   (BM/2) x (BN/2) block of 32x32 MFMA tiles; K in slices of 64.
// * Operands go global -> LDS directly (buffer_load ... lds, 16 bytes per lane):
//   no staging registers, and rows or K past the end fall outside the buffer
//   resource and land in LDS as zeros.  Two LDS stages: the loads of slice s+1
//   are in flight while slice s is multiplied.
// * LDS rows are 128 bytes (64 bf16); the 16-byte chunk c of row r is stored at
//   chunk position c ^ (r mod 8), so the 32 rows read by one MFMA fragment load
//   hit different banks.
// * The output tile is staged through LDS and written with 16-byte row-contiguous
//   stores.  Tiles are handed to XCDs in contiguous ranges (m fastest), so the
//   workgroups of one XCD share the W0 rows of a column tile in L2.
// * When the tiles alone cannot cover the 256 CUs (short, wide layers), K is
//   split over S workgroups that write fp32 partials (split 0 adds t U^T; all
//   apply s), and a small kernel adds them in split order.  Deterministic.

#include <stdlib.h>

#include "aq_internal.h"
#include "device_common.h"

namespace aq {

namespace {
constexpr int BK = 64;
enum { EPI_PLAIN = 0, EPI_RECON = 1, EPI_PARTIAL = 2 };
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
  float *part;             // [S][M][ldp] fp32 partials (EPI_PARTIAL)
  const uint16_t *t;
  int ldx, ldy, ldt, ldp, M, K, nblk, ntm, ntiles, S, kchunk, vec_store;
  int raw;                 // EPI_PARTIAL without s and t U^T (the rank-r pass)
  PfBlk b[kMaxBlocks];
};

__device__ __forceinline__ bf16x8 load_u8(const PfBlk &B, int n, int j) {
  // U[n, j .. j+7], zero beyond r
  if (B.ufast) return j < B.r ? as_bf16x8(ld16(B.U + (size_t)n * B.r + j)) : zero_bf16x8();
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

// One 16-byte-per-lane direct load into LDS: lane l of the instruction writes
// bytes [16 l, 16 l + 16) of the 1 KiB at `lds`.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, uint16_t *lds, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, off, 0, 0, 0);
}

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256, 1) void k_gemm_bf16(const PfArgs a) {
  constexpr int WM = BM / 2, WN = BN / 2;          // wave tile
  constexpr int TM = WM / 32, TN = WN / 32;        // 32x32 MFMA tiles per wave
  constexpr int STAGE = (BM + BN) * BK;            // elements per LDS stage
  // Two stages as two distinct LDS objects: the compiler can then tell that the
  // direct loads in flight into one stage never alias the fragment reads of the
  // other, and does not wait for them before reading.
  __shared__ __attribute__((aligned(1024))) uint16_t lds0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t lds1[STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lhi = lane >> 5;
  const int unit = xcd_contiguous_tile(blockIdx.x, a.ntiles * a.S);
  if (unit < 0) return;
  const int tile = unit / a.S, p = unit - tile * a.S;
  int bi = 0;
  if (a.nblk > 1 && tile >= a.b[1].tile0) bi = 1;
  if (a.nblk > 2 && tile >= a.b[2].tile0) bi = 2;
  const PfBlk B = bi == 0 ? a.b[0] : (bi == 1 ? a.b[1] : a.b[2]);

  const int tin = tile - B.tile0;
  const int tn = tin / a.ntm, tm = tin - tn * a.ntm;
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = a.M, K = a.K;
  const int kbeg = p * a.kchunk;
  const int kend = min(K, kbeg + a.kchunk);
  const int nk = (kend - kbeg + BK - 1) / BK;

  // Buffer resources over this tile's rows of x and W.
  const int mrows = min(BM, M - m0), nrows = min(BN, B.N - n0);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x + (size_t)m0 * a.ldx, (uint32_t)(((mrows - 1) * a.ldx + K) * 2));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(B.W + (size_t)n0 * K, nrows > 0 ? (uint32_t)nrows * K * 2 : 0u);

  // Loader: instruction j of this wave fills 8 rows (1 KiB) of a stage; lane l
  // takes row 8 q + l / 8 and chunk position l % 8, which holds global chunk
  // (l % 8) ^ (row mod 8).
  const int lrow = lane >> 3, lslot = lane & 7;
  auto issue = [&](int slice, uint16_t *stage) {
    const int k0 = kbeg + slice * BK;
    uint16_t *As = stage, *Bs = stage + BM * BK;
#pragma unroll
    for (int j = 0; j < BM / 32; ++j) {
      const int q = wave * (BM / 32) + j, row = 8 * q + lrow;
      const int kk = k0 + 8 * (lslot ^ (row & 7));
      const int off = (slice < nk && kk < kend) ? (row * a.ldx + kk) * 2 : kOOB;
      lds_load16(rx, As + q * 512, off);
    }
#pragma unroll
    for (int j = 0; j < BN / 32; ++j) {
      const int q = wave * (BN / 32) + j, row = 8 * q + lrow;
      const int kk = k0 + 8 * (lslot ^ (row & 7));
      const int off = (slice < nk && kk < kend) ? (row * K + kk) * 2 : kOOB;
      lds_load16(rw, Bs + q * 512, off);
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  auto compute = [&](const uint16_t *stage) {
    const uint16_t *As = stage, *Bs = stage + BM * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = 2 * kk + lhi;          // 16-byte chunk of the 64-wide row
      bf16x8 af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WM + i * 32 + l32;
        af[i] = as_bf16x8(*reinterpret_cast<const uint4 *>(As + row * BK + 8 * (c ^ (row & 7))));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wn * WN + j * 32 + l32;
        bf[j] = as_bf16x8(*reinterpret_cast<const uint4 *>(Bs + row * BK + 8 * (c ^ (row & 7))));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };

  // Slice s lives in stage s % 2.  The loads of slice s + 1 are in flight while
  // slice s is multiplied; past the last slice the loads are out of range (no
  // memory traffic, zeros into an unused stage).
  issue(0, lds0);
  for (int s = 0; s < nk; s += 2) {
    __builtin_amdgcn_s_waitcnt(0);       // this wave's loads of slice s have landed
    __syncthreads();                     // ... and everyone's; slice s - 1 consumed
    issue(s + 1, lds1);
    compute(lds0);
    if (s + 1 >= nk) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    issue(s + 2, lds0);
    compute(lds1);
  }
  __builtin_amdgcn_s_waitcnt(0);         // drain the (out-of-range) tail loads

  // ---- epilogue.  MFMA 32x32 output layout: lane holds column (lane % 32) and
  // rows 8 (v / 4) + 4 (lane / 32) + (v % 4), v = 0..15.
  if (EPI != EPI_PLAIN && !a.raw) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn * WN + j * 32 + l32;
      const float sv = n < B.N ? bf2f(B.s[n]) : 0.f;
#pragma unroll
      for (int i = 0; i < TM; ++i) acc[i][j] *= sv;
    }
    if (EPI == EPI_RECON || p == 0) {
      for (int jc = 0; jc < B.r; jc += 16) {
        const int jj = jc + 8 * lhi;
        bf16x8 ta[TM], ub[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int m = m0 + wm * WM + i * 32 + l32;
          ta[i] = m < M ? as_bf16x8(ld16(a.t + (size_t)m * a.ldt + B.tcol + jj)) : zero_bf16x8();
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = n0 + wn * WN + j * 32 + l32;
          ub[j] = n < B.N ? load_u8(B, n, jj) : zero_bf16x8();
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[i], ub[j], acc[i][j], 0, 0, 0);
      }
    }
  }

  if (EPI == EPI_PARTIAL) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 32 + l32;
        if (n >= B.Nst) continue;            // padding columns carry zeros
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + wm * WM + i * 32 + 8 * (v >> 2) + 4 * lhi + (v & 3);
          if (m < M) a.part[((size_t)p * M + m) * a.ldp + B.col + n] = acc[i][j][v];
        }
      }
    return;
  }

  // Stage the bf16 tile through LDS, half a tile (one wave row) at a time, then
  // write rows with 16-byte stores.
  const int nst = min(BN, B.Nst - n0);
#pragma unroll 1
  for (int h = 0; h < 2; ++h) {
    __syncthreads();                     // previous users of lds0 are done
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int ml = i * 32 + 8 * (v >> 2) + 4 * lhi + (v & 3);
            const int nl = wn * WN + j * 32 + l32;
            lds0[ml * BN + nl] = f2bf(acc[i][j][v]);
          }
    }
    __syncthreads();
    for (int c = tid; c < WM * (BN / 8); c += 256) {
      const int ml = c / (BN / 8), nc = (c - ml * (BN / 8)) * 8;
      const int m = m0 + h * WM + ml;
      if (m >= M || nc >= nst) continue;
      uint16_t *dst = a.y + (size_t)m * a.ldy + B.col + n0 + nc;
      const uint16_t *src = lds0 + ml * BN + nc;
      if (a.vec_store && nc + 8 <= nst) {
        *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
      } else {
        for (int e = 0; e < 8 && nc + e < nst; ++e) dst[e] = src[e];
      }
    }
  }
}

// y = bf16(sum of the S fp32 partials, in split order); also folds the split
// partials of the rank-r pass into the bf16 t buffer.
__global__ __launch_bounds__(256) void k_prefill_reduce(const float *part, int S, int M, int ldp,
                                                        int ncols, uint16_t *y, int ldy) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)M * ncols) return;
  const int m = (int)(i / ncols), n = (int)(i - (long)m * ncols);
  float sum = 0.f;
  for (int q = 0; q < S; ++q) sum += part[((size_t)q * M + m) * ldp + n];
  y[(size_t)m * ldy + n] = f2bf(sum);
}

// ---------------------------------------------------------------- host side

namespace {

struct TileCfg {
  int BM, BN, S;
};

static int env_int(const char *name, int dflt) {
  const char *v = getenv(name);
  return v && *v ? atoi(v) : dflt;
}

int count_tiles(const Recon &rq, int BM, int BN, bool tpass) {
  const int ntm = (int)((rq.M + BM - 1) / BM);
  int t = 0;
  for (int b = 0; b < rq.nblk; ++b) {
    const int64_t N = tpass ? (rq.blk[b].r + 15) / 16 * 16 : rq.blk[b].N;
    if (N == 0) continue;
    t += (int)((N + BN - 1) / BN) * ntm;
  }
  return t;
}

// Output tile and K split of the main pass.  Measured on MI355X over the
// Gemma-3-1B and large-decoder prefill shapes, 128 x 128 tiles were fastest in
// every case (two workgroups per CU); K is split when the tiles cover fewer than
// two workgroups per CU, as long as each split keeps >= 1024 K values.
TileCfg choose(const Recon &rq) {
  TileCfg best = {128, 128, 1};
  const int tiles = count_tiles(rq, 128, 128, false);
  if (tiles > 0 && tiles < 2 * kNumCU) {
    const int S = (2 * kNumCU + tiles - 1) / tiles;
    const int smax = rq.K / 1024 > 1 ? (int)(rq.K / 1024) : 1;
    best.S = S < smax ? S : smax;
  }
  // Tuning overrides (profiling sweeps).
  const int bm = env_int("AQ_PREFILL_BM", 0), bn = env_int("AQ_PREFILL_BN", 0);
  const int so = env_int("AQ_PREFILL_S", 0);
  if ((bm == 128 || bm == 256) && (bn == 128 || bn == 256) && !(bm == 256 && bn == 256))
    best.BM = bm, best.BN = bn;
  if (so >= 1) best.S = so;
  return best;
}

}  // namespace

void plan_prefill(const Recon &rq, PrefillPlan *pl) {
  int c = 0;
  for (int b = 0; b < rq.nblk; ++b) {
    pl->tcol[b] = c;
    c += (int)((rq.blk[b].r + 15) / 16 * 16);
  }
  pl->ldt = c;
  const TileCfg tc = choose(rq);
  pl->BM = tc.BM;
  pl->BN = tc.BN;
  pl->S = tc.S;
  // Rank-r pass: 64 x 128 tiles over t's columns (a narrow output, so small
  // tiles keep enough workgroups busy); K is split only when it is long, and
  // then a small kernel folds the fp32 partials.
  pl->tBM = 64;
  pl->tBN = 128;
  pl->tS = 1;
  if (c > 0) {
    const int kslices = (int)((rq.K + BK - 1) / BK);
    pl->tS = (kslices + 35) / 36;                            // <= 36 K slices per split
    const int to = env_int("AQ_TPASS_S", 0);
    if (to >= 1) pl->tS = to;
  }
  size_t bytes = (size_t)rq.M * c * 2;
  bytes = (bytes + 255) / 256 * 256;
  pl->tpart_off = bytes;
  if (pl->tS > 1) bytes += ((size_t)pl->tS * rq.M * c * 4 + 255) / 256 * 256;
  pl->part_off = bytes;
  if (pl->S > 1) bytes += (size_t)pl->S * rq.M * rq.Ntot * 4;
  pl->ws_bytes = bytes > 0 ? kWsReserved + bytes : 0;
}

template <int EPI>
static void launch_tile(int BM, int BN, const PfArgs &a, int grid, hipStream_t st) {
  if (BM == 64) {
    if constexpr (EPI != EPI_RECON)
      hipLaunchKernelGGL((k_gemm_bf16<64, 128, EPI>), dim3(grid), dim3(256), 0, st, a);
    return;
  }
  if (BM == 256 && BN == 128)
    hipLaunchKernelGGL((k_gemm_bf16<256, 128, EPI>), dim3(grid), dim3(256), 0, st, a);
  else if (BM == 128 && BN == 256)
    hipLaunchKernelGGL((k_gemm_bf16<128, 256, EPI>), dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_gemm_bf16<128, 128, EPI>), dim3(grid), dim3(256), 0, st, a);
}

static hipError_t run(PfArgs &a, int BM, int BN, int epi, hipStream_t st) {
  a.ntm = (a.M + BM - 1) / BM;
  int t0 = 0;
  for (int b = 0; b < a.nblk; ++b) {
    a.b[b].tile0 = t0;
    a.b[b].ntn = (a.b[b].Nst + BN - 1) / BN;
    t0 += a.b[b].ntn * a.ntm;
  }
  a.ntiles = t0;
  if (t0 == 0) return hipSuccess;
  const int units = t0 * a.S;
  const int grid = 8 * ((units + 7) / 8);
  switch (epi) {
    case EPI_PLAIN: launch_tile<EPI_PLAIN>(BM, BN, a, grid, st); break;
    case EPI_RECON: launch_tile<EPI_RECON>(BM, BN, a, grid, st); break;
    default: launch_tile<EPI_PARTIAL>(BM, BN, a, grid, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const Recon &rq, const PrefillPlan &pl, void *ws, hipStream_t st) {
  char *scratch = ws ? (char *)ws + kWsReserved : nullptr;
  uint16_t *tbuf = pl.ldt > 0 ? (uint16_t *)scratch : nullptr;
  PfArgs a = {};
  a.x = (const uint16_t *)rq.x;
  a.ldx = (int)rq.ldx;
  a.M = (int)rq.M;
  a.K = (int)rq.K;

  // pass 1: t = x Vt^T for every block with r > 0 (columns padded to 16 with
  // zeros), split along K into fp32 partials when that fills more CUs.
  if (pl.ldt > 0) {
    PfArgs t = a;
    t.y = tbuf;
    t.ldy = pl.ldt;
    t.S = pl.tS;
    int tkc = (int)((rq.K + pl.tS - 1) / pl.tS);
    t.kchunk = (tkc + BK - 1) / BK * BK;
    t.vec_store = 1;
    t.raw = 1;
    t.part = pl.tS > 1 ? (float *)(scratch + pl.tpart_off) : nullptr;
    t.ldp = pl.ldt;
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
    hipError_t e = run(t, pl.tBM, pl.tBN, pl.tS > 1 ? EPI_PARTIAL : EPI_PLAIN, st);
    if (e != hipSuccess) return e;
    if (pl.tS > 1) {
      const long n = (long)rq.M * pl.ldt;
      hipLaunchKernelGGL(k_prefill_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                         (const float *)t.part, pl.tS, (int)rq.M, pl.ldt, pl.ldt, tbuf, pl.ldt);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }

  // pass 2: y = s * (x W0^T) + t U^T
  a.y = (uint16_t *)rq.y;
  a.ldy = (int)rq.ldy;
  a.t = tbuf;
  a.ldt = pl.ldt;
  a.S = pl.S;
  int kc = (int)((rq.K + pl.S - 1) / pl.S);
  a.kchunk = (kc + BK - 1) / BK * BK;
  a.nblk = rq.nblk;
  a.part = pl.S > 1 ? (float *)(scratch + pl.part_off) : nullptr;
  a.ldp = (int)rq.Ntot;
  a.vec_store = ((uintptr_t)rq.y % 16 == 0) && (rq.ldy % 8 == 0);
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
    if (P.col % 8) a.vec_store = 0;
  }
  hipError_t e = run(a, pl.BM, pl.BN, pl.S > 1 ? EPI_PARTIAL : EPI_RECON, st);
  if (e != hipSuccess || pl.S == 1) return e;
  const long n = (long)rq.M * rq.Ntot;
  hipLaunchKernelGGL(k_prefill_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     (const float *)a.part, pl.S, (int)rq.M, (int)rq.Ntot, (int)rq.Ntot, a.y,
                     (int)rq.ldy);
  return hipGetLastError();
}

}  // namespace aq
