// Streaming reconstruction for small batches (M <= 64 tokens), bf16 in, fp32
// accumulation, bf16 out.
//
// What it computes ("How attnquant works", section "The reconstruction identity";
// "Execution paths", section "The GEMM formulation" for the row-batch form and
// the Q/K/V and gate/up batching):
//     y[m, col_b + n] = s_b[n] * (x[m] . W0_b[n]) + sum_j U_b[n, j] * (x[m] . Vt_b[j])
// for every block b of a (possibly fused) dispatch.
//
// Design (MI355X / gfx950):
// * At decode the arithmetic intensity is ~1-16 flop/byte, so the kernel is
//   bound by HBM: every byte of W0 is read exactly once, with 16-byte loads.
// * The weights are the MFMA B operand and the tokens the A operand of
//   v_mfma_f32_16x16x32_bf16: one 16-row group of W0 x 32 K-values per
//   instruction, tokens padded to 16 (rows of x beyond M are zero registers, not
//   loads).  A lane loads 16 contiguous bytes of one row; four lanes cover 64
//   contiguous bytes.  No cross-lane reduction is needed and no bf16 -> fp32
//   conversion runs on the VALU.
// * The concatenated down-contraction of the pages ("one x @ [W0^T, V]") is
//   realised by treating the block's Vt rows as extra 16-row groups that the
//   workgroup streams alongside its W0 rows: the workgroup obtains the partial
//   t = x Vt^T over its own K range and applies U in its epilogue, so t never
//   leaves the chip.  Vt is small and is served from L2 to the workgroups that
//   share it.
// * Each workgroup (4 waves) owns NG row groups (vg of Vt, NG - vg of W0) and one
//   K range; its waves interleave over that range in 128-value steps and their
//   partial sums are added in LDS in a fixed wave order.  When one row tile is
//   split over S workgroups along K (to fill 256 CUs on short, wide layers), each
//   split stores its fp32 partial y, and the last split to finish (an atomic
//   arrival counter; no workgroup ever waits) adds the partials in split order and
//   writes bf16 y.  The result is therefore deterministic.  The splits of one
//   tile are placed on one XCD so that the partials stay in one L2.

#include <stdlib.h>

#include "aq_internal.h"
#include "device_common.h"

namespace aq {

struct DecBlk {
  const uint16_t *W0, *s, *U, *Vt;
  int N, r, col, tile0, vg, ufast;
};

struct DecArgs {
  const uint16_t *x;
  uint16_t *y;
  float *part;          // [S][M][Ntot] fp32 partials (S > 1)
  unsigned *counters;   // [ntiles] arrival counters, zero between calls
  int ldx, ldy, M, K, Ntot;
  int nblk, ntiles, S, kchunk;
  DecBlk b[kMaxBlocks];
};

template <int MT, int NG>
__global__ __launch_bounds__(256, 2) void k_decode_bf16(const DecArgs a) {
  __shared__ float red[NG * MT * 256];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j16 = lane & 15, g = lane >> 4;

  // Workgroup -> (row tile, K split).  Ids go to XCDs round-robin, so the S splits
  // of tile t all carry ids = xcd(t) (mod 8).
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int tl = slot / a.S, p = slot - tl * a.S;
  const int tile = tl * 8 + xcd;
  if (tile >= a.ntiles) return;

  int bi = 0;
  if (a.nblk > 1 && tile >= a.b[1].tile0) bi = 1;
  if (a.nblk > 2 && tile >= a.b[2].tile0) bi = 2;
  const DecBlk B = bi == 0 ? a.b[0] : (bi == 1 ? a.b[1] : a.b[2]);

  const int vg = B.vg, wg = NG - vg;
  const int row0 = (tile - B.tile0) * 16 * wg;
  const int K = a.K;
  const int kbeg = p * a.kchunk;
  const int kend = min(K, kbeg + a.kchunk);
  const int nsteps = (kend - kbeg + 127) >> 7;

  const uint16_t *rp[NG];
  bool rok[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    if (gi < vg) {
      const int j = gi * 16 + j16;
      rok[gi] = j < B.r;
      rp[gi] = B.Vt + (size_t)(rok[gi] ? j : 0) * K;
    } else {
      const int n = row0 + (gi - vg) * 16 + j16;
      rok[gi] = n < B.N;
      rp[gi] = B.W0 + (size_t)(rok[gi] ? n : 0) * K;
    }
  }
  const uint16_t *xp[MT];
  bool xok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + j16;
    xok[mt] = m < a.M;
    xp[mt] = a.x + (size_t)(xok[mt] ? m : 0) * a.ldx;
  }

  f32x4 acc[NG][MT];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[gi][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int st = wave; st < nsteps; st += 4) {
    const int k0 = kbeg + st * 128 + 8 * g;
    bf16x8 xf[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kk = k0 + 32 * s;
        xf[mt][s] = (xok[mt] && kk < kend) ? as_bf16x8(ld16(xp[mt] + kk)) : zero_bf16x8();
      }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      bf16x8 wf[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kk = k0 + 32 * s;
        wf[s] = (rok[gi] && kk < kend) ? as_bf16x8(ld16(rp[gi] + kk)) : zero_bf16x8();
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[gi][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[mt][s], wf[s], acc[gi][mt], 0, 0, 0);
    }
  }

  // Add the four waves' partial sums in wave order 0, 1, 2, 3 (deterministic).
  // Layout: red[((gi * MT + mt) * 4 + v) * 64 + lane] holds the MFMA output
  // element (row m = 16 mt + 4 (lane / 16) + v, column = lane % 16 of group gi).
#pragma unroll 1
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int idx = ((gi * MT + mt) * 4 + v) * 64 + lane;
            red[idx] = (w == 0) ? acc[gi][mt][v] : red[idx] + acc[gi][mt][v];
          }
    }
    __syncthreads();
  }

  // Epilogue: y_p = s * z_p + U t_p for this K range.
  const int Rv = min(16 * wg, B.N - row0);
  const int r = B.r;
  const int nout = a.M * Rv;
  for (int o = tid; o < nout; o += 256) {
    const int nl = o % Rv, m = o / Rv;
    const int n = row0 + nl;
    const int mt = m >> 4, i = m & 15, vz = i & 3, lb = (i >> 2) << 4;
    const float z = red[(((vg + (nl >> 4)) * MT + mt) * 4 + vz) * 64 + lb + (nl & 15)];
    float yv = bf2f(B.s[n]) * z;
    const uint16_t *u = B.U + (size_t)n * r;
    const float *tb = red + (size_t)(mt * 4 + vz) * 64 + lb;   // t group gv at + gv*MT*256
    if (B.ufast) {
      for (int j0 = 0; j0 < r; j0 += 8) {
        const uint4 uv = ld16(u + j0);
        const uint32_t w4[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int j = j0 + q;
          const float uj = bf2f((uint16_t)(w4[q >> 1] >> ((q & 1) * 16)));
          yv += uj * tb[(j >> 4) * MT * 256 + (j & 15)];
        }
      }
    } else {
      for (int j = 0; j < r; ++j) yv += bf2f(u[j]) * tb[(j >> 4) * MT * 256 + (j & 15)];
    }
    if (a.S == 1)
      a.y[(size_t)m * a.ldy + B.col + n] = f2bf(yv);
    else
      a.part[((size_t)p * a.M + m) * a.Ntot + B.col + n] = yv;
  }

  if (a.S > 1) {
    // Publish this split's partial; the last split to arrive finishes the tile.
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = atomicAdd(&a.counters[tile], 1u);
      s_last = (prev == (unsigned)(a.S - 1));
    }
    __syncthreads();
    if (s_last) {
      __threadfence();
      for (int o = tid; o < nout; o += 256) {
        const int nl = o % Rv, m = o / Rv;
        const size_t c = (size_t)B.col + row0 + nl;
        float sum = 0.f;
        for (int q = 0; q < a.S; ++q)
          sum += __builtin_nontemporal_load(&a.part[((size_t)q * a.M + m) * a.Ntot + c]);
        a.y[(size_t)m * a.ldy + c] = f2bf(sum);
      }
      if (tid == 0) atomicExch(&a.counters[tile], 0u);
    }
  }
}

// ---------------------------------------------------------------- host side

static int env_int(const char *name, int dflt) {
  const char *v = getenv(name);
  return v && *v ? atoi(v) : dflt;
}

static int max_ng(int MT) { return MT == 1 ? 10 : (MT == 2 ? 8 : 6); }

bool plan_decode(const Recon &rq, DecodePlan *pl) {
  if (rq.dt != AQ_BF16 || rq.M < 1 || rq.M > kDecodeMaxM) return false;
  const int M = (int)rq.M, K = (int)rq.K;
  pl->MT = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  int vgmax = 0;
  for (int b = 0; b < rq.nblk; ++b) {
    pl->vg[b] = (int)((rq.blk[b].r + 15) / 16);
    vgmax = vgmax > pl->vg[b] ? vgmax : pl->vg[b];
  }
  const int ngmax = max_ng(pl->MT);
  if (vgmax + 1 > ngmax) return false;          // rank too large for this kernel

  // Tuning override (profiling sweeps): AQ_DECODE_NG, AQ_DECODE_S.
  int NG = env_int("AQ_DECODE_NG", 0);
  int S = env_int("AQ_DECODE_S", 0);
  if (NG < vgmax + 1 || NG > ngmax || (NG & 1)) NG = 0;

  auto tiles_for = [&](int ng) {
    int t = 0;
    for (int b = 0; b < rq.nblk; ++b) {
      const int rows = 16 * (ng - pl->vg[b]);
      t += (int)((rq.blk[b].N + rows - 1) / rows);
    }
    return t;
  };
  if (!NG) {
    // Largest row tile (least Vt re-reading) that still yields >= 2 workgroups
    // per CU once K is split into ranges of >= 512 values.
    const int smax = K / 512 > 1 ? K / 512 : 1;
    NG = ngmax;
    while (NG - 2 >= vgmax + 1 && tiles_for(NG) * smax < 2 * kNumCU) NG -= 2;
  }
  const int ntiles = tiles_for(NG);
  if (S <= 0) {
    const int smax = K / 512 > 1 ? K / 512 : 1;
    S = (4 * kNumCU + ntiles - 1) / ntiles;
    S = S < 1 ? 1 : (S > smax ? smax : S);
  }
  int kchunk = (K + S - 1) / S;
  kchunk = (kchunk + 127) / 128 * 128;
  S = (K + kchunk - 1) / kchunk;

  pl->NG = NG;
  pl->S = S;
  pl->kchunk = kchunk;
  pl->ntiles = ntiles;
  int t0 = 0;
  for (int b = 0; b < rq.nblk; ++b) {
    const int rows = 16 * (NG - pl->vg[b]);
    pl->tile0[b] = t0;
    pl->ntile[b] = (int)((rq.blk[b].N + rows - 1) / rows);
    t0 += pl->ntile[b];
  }
  pl->ws_counters = ((size_t)ntiles * 4 + 255) / 256 * 256;
  pl->ws_partials = S > 1 ? (size_t)S * M * rq.Ntot * 4 : 0;
  return true;
}

template <int MT, int NG>
static void launch_one(const DecArgs &a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((k_decode_bf16<MT, NG>), dim3(grid), dim3(256), 0, st, a);
}

template <int MT>
static bool launch_ng(const DecArgs &a, int NG, int grid, hipStream_t st) {
  switch (NG) {
    case 2: launch_one<MT, 2>(a, grid, st); return true;
    case 4: launch_one<MT, 4>(a, grid, st); return true;
    case 6: launch_one<MT, 6>(a, grid, st); return true;
    case 8:
      if constexpr (MT <= 2) { launch_one<MT, 8>(a, grid, st); return true; }
      return false;
    case 10:
      if constexpr (MT == 1) { launch_one<MT, 10>(a, grid, st); return true; }
      return false;
  }
  return false;
}

hipError_t launch_decode(const Recon &rq, const DecodePlan &pl, void *ws, hipStream_t st) {
  DecArgs a = {};
  a.x = (const uint16_t *)rq.x;
  a.y = (uint16_t *)rq.y;
  a.counters = (unsigned *)ws;
  a.part = pl.S > 1 ? (float *)((char *)ws + pl.ws_counters) : nullptr;
  a.ldx = (int)rq.ldx;
  a.ldy = (int)rq.ldy;
  a.M = (int)rq.M;
  a.K = (int)rq.K;
  a.Ntot = (int)rq.Ntot;
  a.nblk = rq.nblk;
  a.ntiles = pl.ntiles;
  a.S = pl.S;
  a.kchunk = pl.kchunk;
  for (int b = 0; b < rq.nblk; ++b) {
    const Proj &P = rq.blk[b];
    DecBlk &d = a.b[b];
    d.W0 = (const uint16_t *)P.W0;
    d.s = (const uint16_t *)P.s;
    d.U = (const uint16_t *)P.U;
    d.Vt = (const uint16_t *)P.Vt;
    d.N = (int)P.N;
    d.r = (int)P.r;
    d.col = (int)P.col;
    d.tile0 = pl.tile0[b];
    d.vg = pl.vg[b];
    d.ufast = (P.r % 8 == 0) && (((uintptr_t)P.U & 15) == 0);
  }
  const int grid = 8 * ((pl.ntiles + 7) / 8) * pl.S;
  bool ok = false;
  switch (pl.MT) {
    case 1: ok = launch_ng<1>(a, pl.NG, grid, st); break;
    case 2: ok = launch_ng<2>(a, pl.NG, grid, st); break;
    case 4: ok = launch_ng<4>(a, pl.NG, grid, st); break;
  }
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace aq
