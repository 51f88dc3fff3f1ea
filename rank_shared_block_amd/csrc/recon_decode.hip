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
// * Loads go through buffer resources: rows past N, K past the end of the range
//   and tokens past M fall outside the resource and read as zero, so the loop is
//   branch-free and every fragment of a step is requested at once; two steps are
//   in flight per wave (two register sets used in turn).
// * Each workgroup (WAVES = 4 or 8 waves) owns NG row groups (vg of Vt, NG - vg
//   of W0) and one K range; its waves interleave over that range and their
//   partial sums are added in LDS in a fixed wave order.  When a row tile is
//   split over S workgroups along K (short, wide layers need it to fill 256 CUs),
//   each split writes its fp32 partial y to the workspace and a second small
//   kernel adds the S partials in split order.  The kernel boundary publishes the
//   partials; a device-scope fence per workgroup would write back and invalidate
//   the whole L2 each time, which costs far more than the extra launch.  The
//   result is deterministic.

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
  int ldx, ldy, M, K, Ntot;
  int nblk, ntiles, S, kchunk;
  DecBlk b[kMaxBlocks];
};

// MT: 16-token groups; NG: 16-row groups per workgroup; WAVES: waves per
// workgroup.  A step covers KS = 4 / MT chunks of 32 K-values, so that the
// fragments of two steps fit the register budget of two waves per SIMD.
template <int MT, int NG, int WAVES>
__global__ __launch_bounds__(64 * WAVES, WAVES >= 8 ? 1 : 2) void k_decode_bf16(const DecArgs a) {
  constexpr int KS = 4 / MT;
  constexpr int KSTEP = 32 * KS;
  constexpr int NT = 64 * WAVES;
  constexpr int SLOT = NG * MT * 256;             // floats per wave's partial sums
  __shared__ float red[WAVES * SLOT];
  __shared__ float tsum[16 * MT * 16 * (NG - 1)];  // reduced t: [token][rank]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j16 = lane & 15, g = lane >> 4;

  const int unit = xcd_contiguous_tile(blockIdx.x, a.ntiles * a.S);
  if (unit < 0) return;
  const int tile = unit / a.S, p = unit - tile * a.S;

  int bi = 0;
  if (a.nblk > 1 && tile >= a.b[1].tile0) bi = 1;
  if (a.nblk > 2 && tile >= a.b[2].tile0) bi = 2;
  const DecBlk B = bi == 0 ? a.b[0] : (bi == 1 ? a.b[1] : a.b[2]);

  const int vg = B.vg, wg = NG - vg;
  const int row0 = (tile - B.tile0) * 16 * wg;
  const int K = a.K;
  const int kbeg = p * a.kchunk;
  const int kend = min(K, kbeg + a.kchunk);
  const int nsteps = (kend - kbeg + KSTEP - 1) / KSTEP;

  // One buffer resource per operand: rows past the valid range fall outside it,
  // and so do K chunks past this range (offset kOOB).
  const int Rv = min(16 * wg, B.N - row0);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(B.W0 + (size_t)row0 * K, (uint32_t)Rv * K * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(B.Vt, (uint32_t)B.r * K * 2);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)((a.M - 1) * a.ldx + K) * 2);
  int roff[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi)
    roff[gi] = (gi < vg ? gi * 16 + j16 : (gi - vg) * 16 + j16) * K * 2;
  int xoff[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + j16;
    xoff[mt] = m < a.M ? m * a.ldx * 2 : kOOB;
  }

  // Epilogue mapping: thread tid owns output row nl = tid % Rv and tokens
  // m = tid / Rv, tid / Rv + tpr, ...  Its s value and (for r <= 16) its U row are
  // requested now, so that their latency hides under the main loop.
  const int r = B.r;
  const int tpr = NT / Rv;                       // threads per output row (>= 1)
  const int nl_e = tid % Rv, m_e0 = tid / Rv;
  const bool epi = m_e0 < tpr && m_e0 < a.M;
  const int n_e = row0 + nl_e;
  const float s_e = epi ? bf2f(B.s[n_e]) : 0.f;
  uint4 u_pre0 = make_uint4(0, 0, 0, 0), u_pre1 = make_uint4(0, 0, 0, 0);
  const bool upre = B.ufast && r <= 16;
  if (epi && upre && r > 0) {
    u_pre0 = ld16(B.U + (size_t)n_e * r);
    if (r > 8) u_pre1 = ld16(B.U + (size_t)n_e * r + 8);
  }

  f32x4 acc[NG][MT];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[gi][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto fetch = [&](int st, bf16x8 (&xd)[MT][KS], bf16x8 (&wd)[NG][KS]) {
    const int k0 = kbeg + st * KSTEP + 8 * g;
    int koff[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) koff[s] = (st < nsteps && k0 + 32 * s < kend) ? (k0 + 32 * s) * 2 : kOOB;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        wd[gi][s] = bload16(gi < vg ? rv : rw, koff[s] == kOOB ? kOOB : roff[gi] + koff[s]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        xd[mt][s] = bload16(rx, (xoff[mt] == kOOB || koff[s] == kOOB) ? kOOB : xoff[mt] + koff[s]);
  };
  auto compute = [&](const bf16x8 (&xd)[MT][KS], const bf16x8 (&wd)[NG][KS]) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[gi][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xd[mt][s], wd[gi][s], acc[gi][mt], 0, 0, 0);
  };

  // Software pipeline with two register sets used in turn (no register copies,
  // so no wait on loads still in flight).  The scheduling barriers keep the
  // compiler from sinking the next step's loads down to their uses.  Past the
  // last step the offsets are out of range: the extra loads return zeros
  // without touching memory.
  bf16x8 xa[MT][KS], wa[NG][KS], xb[MT][KS], wb[NG][KS];
  fetch(wave, xa, wa);
  for (int st = wave; st < nsteps; st += 2 * WAVES) {
    fetch(st + WAVES, xb, wb);
    __builtin_amdgcn_sched_barrier(0);
    compute(xa, wa);
    __builtin_amdgcn_sched_barrier(0);
    if (st + WAVES >= nsteps) break;
    fetch(st + 2 * WAVES, xa, wa);
    __builtin_amdgcn_sched_barrier(0);
    compute(xb, wb);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Every wave stores its partial sums in its own LDS slot; after one barrier
  // they are added in wave order (deterministic).  Slot layout:
  // [((gi * MT + mt) * 4 + v) * 64 + lane] is the MFMA output element
  // (token 16 mt + 4 (lane / 16) + v, row lane % 16 of group gi).
  {
    float *slot = red + wave * SLOT;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) slot[((gi * MT + mt) * 4 + v) * 64 + lane] = acc[gi][mt][v];
  }
  __syncthreads();
  auto red_at = [&](int gi, int m, int c) {       // sum over waves: group gi, token m, column c
    const int idx = ((gi * MT + (m >> 4)) * 4 + (m & 3)) * 64 + (((m & 15) >> 2) << 4) + c;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += red[w * SLOT + idx];
    return v;
  };
  // t[m][j] for this K range, once per workgroup.
  for (int e = tid; e < a.M * r; e += NT) {
    const int m = e / r, j = e - m * r;
    tsum[m * 16 * (NG - 1) + j] = red_at(j >> 4, m, j & 15);
  }
  __syncthreads();

  // Epilogue: y_p = s * z_p + U t_p over this K range.
  if (epi) {
    const uint16_t *u = B.U + (size_t)n_e * r;
    for (int m = m_e0; m < a.M; m += tpr) {
      const float z = red_at(vg + (nl_e >> 4), m, nl_e & 15);
      const float *tm = tsum + m * 16 * (NG - 1);
      float lr = 0.f;
      if (upre) {
        const uint32_t w8[8] = {u_pre0.x, u_pre0.y, u_pre0.z, u_pre0.w, u_pre1.x, u_pre1.y, u_pre1.z, u_pre1.w};
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (j < r) lr += bf2f((uint16_t)(w8[j >> 1] >> ((j & 1) * 16))) * tm[j];
      } else if (B.ufast) {
        for (int j0 = 0; j0 < r; j0 += 8) {
          const uint4 uv = ld16(u + j0);
          const uint32_t w4[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
          for (int q = 0; q < 8; ++q) lr += bf2f((uint16_t)(w4[q >> 1] >> ((q & 1) * 16))) * tm[j0 + q];
        }
      } else {
        for (int j = 0; j < r; ++j) lr += bf2f(u[j]) * tm[j];
      }
      const float yv = s_e * z + lr;
      if (a.S == 1)
        a.y[(size_t)m * a.ldy + B.col + n_e] = f2bf(yv);
      else
        a.part[((size_t)p * a.M + m) * a.Ntot + B.col + n_e] = yv;
    }
  }
}

// y = bf16(sum over the S splits, in split order) for the split-K case.
__global__ __launch_bounds__(256) void k_decode_reduce(const float *part, int S, int M, int Ntot,
                                                       uint16_t *y, int ldy) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int m = blockIdx.y;
  if (n >= Ntot) return;
  float sum = 0.f;
  for (int q = 0; q < S; ++q) sum += part[((size_t)q * M + m) * Ntot + n];
  y[(size_t)m * ldy + n] = f2bf(sum);
}

// ---------------------------------------------------------------- host side

static int env_int(const char *name, int dflt) {
  const char *v = getenv(name);
  return v && *v ? atoi(v) : dflt;
}

// Largest row-group count per workgroup: the fragments of two steps
// (2 * 4 * KS * (NG + MT) VGPRs) plus NG * MT * 4 accumulators must fit the
// 256 registers of a wave at two waves per SIMD.
// LDS: WAVES * NG * MT KiB of partials must leave room for two workgroups per CU.
static int max_ng(int MT) { return MT == 1 ? 4 : (MT == 2 ? 6 : 3); }

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
  // 32-bit buffer offsets: the row tile and Vt must stay below 2^31 bytes.
  if ((int64_t)16 * ngmax * K * 2 >= (int64_t(1) << 31)) return false;

  auto tiles_for = [&](int ng) {
    int t = 0;
    for (int b = 0; b < rq.nblk; ++b) {
      const int rows = 16 * (ng - pl->vg[b]);
      t += (int)((rq.blk[b].N + rows - 1) / rows);
    }
    return t;
  };
  const int ngmin = vgmax + 1 > 2 ? vgmax + 1 : 2;

  // Defaults, from sweeps over the Gemma-3-1B and large-decoder decode shapes on
  // MI355X: 4 waves per workgroup; the largest row tile (least re-reading of Vt)
  // that still gives >= 384 work units once K is split; K split only into
  // ranges of >= 2304 values (a split costs fp32 partials and a reduce launch).
  constexpr int kUnits = 384;
  const int smax = K / 2304 > 1 ? K / 2304 : 1;
  int NG = ngmax;
  while (NG - 1 >= ngmin && tiles_for(NG) * smax < kUnits) NG -= 1;
  int ntiles = tiles_for(NG);
  int WAVES = 4;
  int S = (kUnits + ntiles - 1) / ntiles;
  S = S < 1 ? 1 : (S > smax ? smax : S);
  // Tuning overrides (profiling sweeps): AQ_DECODE_NG, AQ_DECODE_S, AQ_DECODE_WAVES.
  const int ng_o = env_int("AQ_DECODE_NG", 0), s_o = env_int("AQ_DECODE_S", 0);
  const int w_o = env_int("AQ_DECODE_WAVES", 0);
  if (ng_o >= ngmin && ng_o <= ngmax) NG = ng_o;
  if (s_o >= 1) S = s_o;
  if (w_o == 4 || (pl->MT == 1 && w_o == 8)) WAVES = w_o;
  ntiles = tiles_for(NG);

  int kchunk = (K + S - 1) / S;
  kchunk = (kchunk + 127) / 128 * 128;
  S = (K + kchunk - 1) / kchunk;

  pl->NG = NG;
  pl->S = S;
  pl->WAVES = WAVES;
  pl->kchunk = kchunk;
  pl->ntiles = ntiles;
  int t0 = 0;
  for (int b = 0; b < rq.nblk; ++b) {
    const int rows = 16 * (NG - pl->vg[b]);
    pl->tile0[b] = t0;
    pl->ntile[b] = (int)((rq.blk[b].N + rows - 1) / rows);
    t0 += pl->ntile[b];
  }
  pl->ws_bytes = S > 1 ? kWsReserved + (size_t)S * M * rq.Ntot * 4 : 0;
  return true;
}

template <int MT, int NG, int WAVES>
static void launch_one(const DecArgs &a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((k_decode_bf16<MT, NG, WAVES>), dim3(grid), dim3(64 * WAVES), 0, st, a);
}

template <int MT, int WAVES>
static bool launch_ng(const DecArgs &a, int NG, int grid, hipStream_t st) {
  switch (NG) {
    case 2: launch_one<MT, 2, WAVES>(a, grid, st); return true;
    case 3: launch_one<MT, 3, WAVES>(a, grid, st); return true;
    case 4:
      if constexpr (MT < 4) { launch_one<MT, 4, WAVES>(a, grid, st); return true; }
      return false;
    case 5:
      if constexpr (MT == 2) { launch_one<MT, 5, WAVES>(a, grid, st); return true; }
      return false;
    case 6:
      if constexpr (MT == 2) { launch_one<MT, 6, WAVES>(a, grid, st); return true; }
      return false;
  }
  return false;
}

template <int MT>
static bool launch_w(const DecArgs &a, int NG, int WAVES, int grid, hipStream_t st) {
  if constexpr (MT == 1) {
    if (WAVES == 8) return launch_ng<1, 8>(a, NG, grid, st);
  }
  return WAVES == 4 ? launch_ng<MT, 4>(a, NG, grid, st) : false;
}

hipError_t launch_decode(const Recon &rq, const DecodePlan &pl, void *ws, hipStream_t st) {
  DecArgs a = {};
  a.x = (const uint16_t *)rq.x;
  a.y = (uint16_t *)rq.y;
  a.part = pl.S > 1 ? (float *)((char *)ws + kWsReserved) : nullptr;
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
  const int units = pl.ntiles * pl.S;
  const int grid = 8 * ((units + 7) / 8);
  bool ok = false;
  switch (pl.MT) {
    case 1: ok = launch_w<1>(a, pl.NG, pl.WAVES, grid, st); break;
    case 2: ok = launch_w<2>(a, pl.NG, pl.WAVES, grid, st); break;
    case 4: ok = launch_w<4>(a, pl.NG, pl.WAVES, grid, st); break;
  }
  if (!ok) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.S == 1) return e;
  dim3 rg((unsigned)((rq.Ntot + 255) / 256), (unsigned)rq.M);
  hipLaunchKernelGGL(k_decode_reduce, rg, dim3(256), 0, st, (const float *)a.part, pl.S, a.M,
                     a.Ntot, a.y, a.ldy);
  return hipGetLastError();
}

}  // namespace aq
