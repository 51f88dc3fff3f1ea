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
//   v_mfma_f32_16x16x32_bf16: one 16-row group of weights x 32 K-values per
//   instruction, tokens padded to 16 (rows of x beyond M are zero registers, not
//   loads).  A lane loads 16 contiguous bytes of one row; four lanes cover 64
//   contiguous bytes.  No cross-lane reduction is needed and no bf16 -> fp32
//   conversion runs on the VALU.
// * The pages' concatenated down-contraction ("one x @ [W0^T, V]") is a stack of
//   16-row groups: the W0 rows of every block and the r rows of its Vt.  A
//   workgroup streams NG groups over one K range; its waves interleave over that
//   range and their partial sums are added in LDS in a fixed wave order.
// * Loads go through buffer resources: rows past the end, K past the end of the
//   range and tokens past M fall outside the resource and read as zero, so the
//   loop is branch-free and every fragment of a step is requested at once; two
//   steps are in flight per wave (two register sets used in turn).
//
// Two ways to meet the rank-r term, chosen per dispatch by the host:
// * fused (one kernel): each workgroup's tile holds vg groups of Vt next to its
//   W0 groups, so the workgroup gets t = x Vt^T itself and applies s and U in its
//   epilogue; t never leaves the chip.  The price is that every workgroup streams
//   the whole Vt (served from L2): cheap while the tiles outnumber r heavily,
//   ruinous for long K and large r, where it can double the load traffic.
// * split (two kernels): Vt rows form tiles of their own, read exactly once, and
//   K may be split over S workgroups to fill 256 CUs.  Every tile writes its fp32
//   partial (z for W0 rows, t for Vt rows) to the workspace; a combine kernel then
//   forms y = s * sum_p z_p + U (sum_p t_p) in split order.  The kernel boundary
//   publishes the partials; a device-scope fence per workgroup would write back
//   and invalidate the whole L2 each time, which costs far more than the launch.
// Both are deterministic.

#include <limits.h>

#include "aq_internal.h"
#include "device_common.h"

namespace aq {

// One segment of stacked rows.  Fused mode: a block (W0 rows plus vg groups of
// its Vt per tile, s and U for the epilogue).  Split mode: either the W0 rows or
// the Vt rows of a block (vg = 0), written as partials at column `col`.
struct alignas(64) DecSeg {
  const uint16_t *W0, *s, *U, *Vt;
  int N, r, col, vg, ufast, rows, pad[2];
};
static_assert(sizeof(DecSeg) == 64, "one scalar load per segment");
typedef int i32x16 __attribute__((ext_vector_type(16)));

// The first 88 bytes hold everything a workgroup needs before it can pick its
// segment (two scalar cache lines, loaded in one batch); the segment table
// follows and is read once, with one dynamic offset.
struct DecArgs {
  int ntiles, S, K, kchunk;
  int M, ldx, ldy, Wp;
  int tile0[kMaxSegs];  // first tile of each segment; unused entries INT_MAX
  int pad0, pad1;
  const uint16_t *x;
  uint16_t *y;
  float *part;          // split mode: [S][M][Wp] fp32 partials
  DecSeg g[kMaxSegs];
};
static_assert(sizeof(int) * (8 + kMaxSegs + 2) == 64, "header layout");

// MT: 16-token groups; NG: 16-row groups per workgroup; WAVES: waves per
// workgroup; PART: split mode (partials out) instead of the fused epilogue.
// A step covers KS = 4 / MT chunks of 32 K-values, so that the fragments of two
// steps fit the register budget of two waves per SIMD.
template <int MT, int NG, int WAVES, bool PART>
__global__ __launch_bounds__(64 * WAVES, (WAVES >= 8 || (MT == 1 && NG >= 5)) ? 1 : 2) void k_decode_bf16(
    const DecArgs a) {
  constexpr int KS = 4 / MT;
  constexpr int KSTEP = 32 * KS;
  constexpr int NT = 64 * WAVES;
  constexpr int SLOT = NG * MT * 256;             // floats per wave's partial sums
  constexpr int TSUM = PART ? 1 : 16 * MT * 16 * (NG - 1);
  __shared__ float red[WAVES * SLOT];
  __shared__ __attribute__((aligned(16))) float tsum[TSUM];   // fused: reduced t, [token][rank]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const int j16 = lane & 15, g = lane >> 4;

  // Kernel arguments live in memory: request the header in one batch, then the
  // segment, so that a workgroup waits for two scalar round trips, not one per
  // field (the compiler would otherwise load each field at its first use).
  const int ntiles = a.ntiles, nsplit = a.S, K = a.K, kchunk = a.kchunk;
  int t0s[kMaxSegs];
#pragma unroll
  for (int i = 0; i < kMaxSegs; ++i) t0s[i] = a.tile0[i];
  const uint16_t *const xptr = a.x;
  const int Mtok = a.M, ldx = a.ldx;
  asm volatile("" ::"s"(ntiles), "s"(nsplit), "s"(K), "s"(kchunk), "s"(Mtok), "s"(ldx), "s"(t0s[1]),
               "s"(t0s[2]), "s"(t0s[3]), "s"(t0s[4]), "s"(t0s[5]), "s"(xptr));

  const int unit = xcd_contiguous_tile(blockIdx.x, ntiles * nsplit);
  if (unit < 0) return;
  const int tile = unit / nsplit, p = unit - tile * nsplit;

  int bi = 0;
#pragma unroll
  for (int i = 1; i < kMaxSegs; ++i) bi += tile >= t0s[i] ? 1 : 0;
  // The whole 64-byte segment entry as one scalar load.
  const i32x16 sraw = *reinterpret_cast<const i32x16 *>(&a.g[bi]);
  auto ptr_at = [&](int i) {   // global-memory pointers: loads through them stay global loads
    const uint64_t v = ((uint64_t)(uint32_t)sraw[2 * i + 1] << 32) | (uint32_t)sraw[2 * i];
    return (const uint16_t *)(const __attribute__((address_space(1))) uint16_t *)v;
  };
  struct {
    const uint16_t *W0, *s, *U, *Vt;
    int N, r, col, vg, ufast, rows;
  } const B = {ptr_at(0), ptr_at(1), ptr_at(2), ptr_at(3), sraw[8], sraw[9], sraw[10], sraw[11], sraw[12], sraw[13]};
  int tile0 = t0s[0];
#pragma unroll
  for (int i = 1; i < kMaxSegs; ++i) tile0 = bi == i ? t0s[i] : tile0;

  // A tile holds B.rows rows (any count up to 16 x its W0 groups): row groups
  // past them lie outside the W0 resource and cost no memory traffic.
  const int vg = PART ? 0 : B.vg;
  const int row0 = (tile - tile0) * B.rows;
  const int kbeg = p * kchunk;
  const int kend = min(K, kbeg + kchunk);
  const int nsteps = (kend - kbeg + KSTEP - 1) / KSTEP;

  // One buffer resource per operand: rows past the valid range fall outside it,
  // and so do K chunks past this range (offset kOOB).
  const int Rv = min(B.rows, B.N - row0);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(B.W0 + (size_t)row0 * K, (uint32_t)Rv * K * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(B.Vt, PART ? 0u : (uint32_t)B.r * K * 2);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(xptr, (uint32_t)((Mtok - 1) * ldx + K) * 2);
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

  // Fused epilogue mapping: thread tid owns output row nl = tid % Rv and tokens
  // m = tid / Rv, tid / Rv + tpr, ...  Its s value and (for r <= 16) its U row are
  // requested now, by every thread (row n_e < N always) and with no branch, so
  // that nothing waits for them before the main loop: their latency hides under
  // it.  s stays raw bf16 until the epilogue.
  const int r = PART ? 0 : B.r;
  const int tpr = NT / Rv;                       // threads per output row (>= 1)
  const int nl_e = tid % Rv, m_e0 = tid / Rv;
  const bool epi = !PART && m_e0 < tpr && m_e0 < a.M;
  const int n_e = row0 + nl_e;
  uint16_t s_raw = 0;
  if constexpr (!PART) s_raw = B.s[n_e];
  uint4 u_pre0 = make_uint4(0, 0, 0, 0), u_pre1 = make_uint4(0, 0, 0, 0);
  const bool upre = B.ufast && r <= 16;
  if (upre && r > 0) {
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
  // compiler from sinking the next step's loads down to their uses.  A wave
  // fetches exactly its own steps: a load past the last one would return zeros
  // without touching memory, but it still queues behind every load the CU has
  // in flight, and the epilogue would wait for it.  The branches are uniform.
  const int nmine = wave < nsteps ? (nsteps - 1 - wave) / WAVES + 1 : 0;
  bf16x8 xa[MT][KS], wa[NG][KS], xb[MT][KS], wb[NG][KS];
  if (nmine > 0) fetch(wave, xa, wa);
  int i = 0;
  for (; i + 2 < nmine; i += 2) {
    fetch(wave + (i + 1) * WAVES, xb, wb);
    __builtin_amdgcn_sched_barrier(0);
    compute(xa, wa);
    __builtin_amdgcn_sched_barrier(0);
    fetch(wave + (i + 2) * WAVES, xa, wa);
    __builtin_amdgcn_sched_barrier(0);
    compute(xb, wb);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (i + 1 < nmine) {
    fetch(wave + (i + 1) * WAVES, xb, wb);
    __builtin_amdgcn_sched_barrier(0);
    compute(xa, wa);
    __builtin_amdgcn_sched_barrier(0);
    compute(xb, wb);
  } else if (i < nmine) {
    compute(xa, wa);
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

  if constexpr (PART) {
    // Split mode: this tile's rows over this K range, as fp32 partials.
    float *dst = a.part + (size_t)p * a.M * a.Wp + B.col + row0;
    for (int e = tid; e < a.M * Rv; e += NT) {
      const int m = e / Rv, nl = e - m * Rv;
      dst[(size_t)m * a.Wp + nl] = red_at(nl >> 4, m, nl & 15);
    }
    return;
  }

  // t[m][j] over the whole K, once per workgroup.
  for (int e = tid; e < a.M * r; e += NT) {
    const int m = e / r, j = e - m * r;
    tsum[m * 16 * (NG - 1) + j] = red_at(j >> 4, m, j & 15);
  }
  __syncthreads();

  // Fused epilogue: y = s * z + U t.
  if (epi) {
    const float s_e = bf2f(s_raw);
    const uint16_t *u = B.U + (size_t)n_e * r;
    for (int m = m_e0; m < a.M; m += tpr) {
      const float z = red_at(vg + (nl_e >> 4), m, nl_e & 15);
      const float *tm = tsum + m * 16 * (NG - 1);
      float lr = 0.f;
      if (upre) {
        // All 16 t values in four 16-byte LDS reads, requested together; terms
        // past r are dropped by a select (their LDS words were never written).
        // Per-term conditional reads would serialise 16 LDS round trips.
        const uint32_t w8[8] = {u_pre0.x, u_pre0.y, u_pre0.z, u_pre0.w, u_pre1.x, u_pre1.y, u_pre1.z, u_pre1.w};
        const float4 *t4 = reinterpret_cast<const float4 *>(tm);
        const float4 q0 = t4[0], q1 = t4[1], q2 = t4[2], q3 = t4[3];
        const float tv[16] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w,
                              q2.x, q2.y, q2.z, q2.w, q3.x, q3.y, q3.z, q3.w};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float term = bf2f((uint16_t)(w8[j >> 1] >> ((j & 1) * 16))) * tv[j];
          lr += j < r ? term : 0.f;
        }
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
      a.y[(size_t)m * a.ldy + B.col + n_e] = f2bf(s_e * z + lr);
    }
  }
}

// Split mode, second kernel: y[m, col + n] = bf16(s[n] * Z[m, n] + U[n] . T[m])
// with Z = sum_p z_p and T = sum_p t_p added in split order.  Workgroup
// (chunk, m) owns 256 output columns of one block for one token m, so every
// token runs in parallel; T[m] of its block is folded into LDS first.
struct CombBlk {
  const uint16_t *s, *U;
  int N, r, col, tcol, chunk0, ufast;
};

struct CombArgs {
  const float *part;
  uint16_t *y;
  int S, M, Wp, ldy, nblk;
  CombBlk b[kMaxBlocks];
};

__global__ __launch_bounds__(256) void k_decode_combine(const CombArgs a) {
  __shared__ __attribute__((aligned(16))) float T[AQ_MAX_RANK];
  const int chunk = blockIdx.x, m = blockIdx.y, tid = threadIdx.x;
  int bi = 0;
  if (a.nblk > 1 && chunk >= a.b[1].chunk0) bi = 1;
  if (a.nblk > 2 && chunk >= a.b[2].chunk0) bi = 2;
  const CombBlk B = bi == 0 ? a.b[0] : (bi == 1 ? a.b[1] : a.b[2]);
  const int r = B.r;
  const size_t pstride = (size_t)a.M * a.Wp;
  const float *row = a.part + (size_t)m * a.Wp;

  // This thread's s and (for r <= 32) U row are requested together with the
  // partials, before the barrier, so that the kernel waits for memory once.
  const int n = (chunk - B.chunk0) * 256 + tid;
  const bool live = n < B.N;
  const int nc = live ? n : B.N - 1;
  const uint16_t s_raw = B.s[nc];
  const uint16_t *u = B.U + (size_t)nc * r;
  const bool upre = B.ufast && r <= 32;
  uint4 ur[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) ur[q] = (upre && 8 * q < r) ? ld16(u + 8 * q) : make_uint4(0, 0, 0, 0);
  // The partials of this thread's column (z) and, for threads below r, of one
  // rank (t) are requested eight splits at a time, both before either is
  // added up (in split order): one memory round trip per eight splits, not one
  // per split and partial.
  float z = 0.f, tj = 0.f;
  const bool has_t = tid < r;
  const float *zp = row + B.col + nc, *tp = row + B.tcol + (has_t ? tid : 0);
  for (int q0 = 0; q0 < a.S; q0 += 8) {
    float zv[8], tv8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool in = q0 + e < a.S;
      zv[e] = in ? zp[(size_t)(q0 + e) * pstride] : 0.f;
      tv8[e] = in && has_t ? tp[(size_t)(q0 + e) * pstride] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (q0 + e < a.S) {
        z += zv[e];
        tj += tv8[e];
      }
  }
  if (has_t) T[tid] = tj;
  for (int j = tid + 256; j < r; j += 256) {   // ranks past 256 threads (not reached for r <= 256)
    float v = 0.f;
    for (int q = 0; q < a.S; ++q) v += row[q * pstride + B.tcol + j];
    T[j] = v;
  }
  __syncthreads();
  if (!live) return;

  const float sn = bf2f(s_raw);
  float lr = 0.f;
  if (upre) {
    // r is a multiple of 8 here: whole float4s of T, terms in rank order.
    const uint32_t w16[16] = {ur[0].x, ur[0].y, ur[0].z, ur[0].w, ur[1].x, ur[1].y, ur[1].z, ur[1].w,
                              ur[2].x, ur[2].y, ur[2].z, ur[2].w, ur[3].x, ur[3].y, ur[3].z, ur[3].w};
    const float4 *t4 = reinterpret_cast<const float4 *>(T);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (4 * q < r) {
        const float4 t = t4[q];
        lr += bf2f((uint16_t)w16[2 * q]) * t.x;
        lr += bf2f((uint16_t)(w16[2 * q] >> 16)) * t.y;
        lr += bf2f((uint16_t)w16[2 * q + 1]) * t.z;
        lr += bf2f((uint16_t)(w16[2 * q + 1] >> 16)) * t.w;
      }
    }
  } else if (B.ufast) {
    for (int j0 = 0; j0 < r; j0 += 8) {
      const uint4 uv = ld16(u + j0);
      const uint32_t w4[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) lr += bf2f((uint16_t)(w4[q >> 1] >> ((q & 1) * 16))) * T[j0 + q];
    }
  } else {
    for (int j = 0; j < r; ++j) lr += bf2f(u[j]) * T[j];
  }
  a.y[(size_t)m * a.ldy + B.col + n] = f2bf(sn * z + lr);
}

// The combine for launches that would need more than 2048 one-token
// workgroups (the large-decoder gate/up at 32 tokens: 168 chunks x 32 tokens,
// each re-reading its 256 U rows from L2): workgroup (chunk, g) takes tokens
// 4 g .. 4 g + 3, so each U row is read a quarter as often.  The partials go
// through one buffer resource, the token and split in the uniform scalar
// offset, so the loads of every token share one address register (with
// 64-bit addresses per load the kernel ran at two waves per SIMD and lost).
// Same sums in the same order as k_decode_combine.
__global__ __launch_bounds__(256) void k_decode_combine4(const CombArgs a) {
  constexpr int TG = 4;
  __shared__ __attribute__((aligned(16))) float T[TG][AQ_MAX_RANK];
  const int chunk = blockIdx.x, m0 = blockIdx.y * TG, tid = threadIdx.x;
  int bi = 0;
  if (a.nblk > 1 && chunk >= a.b[1].chunk0) bi = 1;
  if (a.nblk > 2 && chunk >= a.b[2].chunk0) bi = 2;
  const CombBlk B = bi == 0 ? a.b[0] : (bi == 1 ? a.b[1] : a.b[2]);
  const int r = B.r, S = a.S, M = a.M, Wp = a.Wp;
  const int n = (chunk - B.chunk0) * 256 + tid;
  const bool live = n < B.N;
  const int nc = live ? n : B.N - 1;
  const uint16_t s_raw = B.s[nc];
  const uint16_t *u = B.U + (size_t)nc * r;
  const bool upre = B.ufast && r <= 32;
  uint4 ur[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) ur[q] = (upre && 8 * q < r) ? ld16(u + 8 * q) : make_uint4(0, 0, 0, 0);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.part, (uint32_t)((size_t)S * M * Wp * 4));
  const int vz = (B.col + nc) * 4, vt = (B.tcol + (tid < r ? tid : 0)) * 4;
  const bool has_t = tid < r;
  float z[TG], tj[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) z[t] = tj[t] = 0.f;
  for (int q0 = 0; q0 < S; q0 += 4) {
    float zv[TG][4], tv[TG][4];
#pragma unroll
    for (int t = 0; t < TG; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool in = m0 + t < M && q0 + e < S;
        const int so = in ? ((q0 + e) * M + m0 + t) * Wp * 4 : 0;
        zv[t][e] = in ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, vz, so, 0)) : 0.f;
        tv[t][e] = in && has_t ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, vt, so, 0)) : 0.f;
      }
#pragma unroll
    for (int t = 0; t < TG; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (q0 + e < S) {
          z[t] += zv[t][e];
          tj[t] += tv[t][e];
        }
  }
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    if (has_t) T[t][tid] = tj[t];
    for (int j = tid + 256; j < r && m0 + t < M; j += 256) {   // ranks past 256 threads (not reached for r <= 256)
      float v = 0.f;
      for (int q = 0; q < S; ++q) v += a.part[((size_t)q * M + m0 + t) * Wp + B.tcol + j];
      T[t][j] = v;
    }
  }
  __syncthreads();
  if (!live) return;
  const float sn = bf2f(s_raw);
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    const int m = m0 + t;
    if (m >= M) break;
    float lr = 0.f;
    if (upre) {
      const uint32_t w16[16] = {ur[0].x, ur[0].y, ur[0].z, ur[0].w, ur[1].x, ur[1].y, ur[1].z, ur[1].w,
                                ur[2].x, ur[2].y, ur[2].z, ur[2].w, ur[3].x, ur[3].y, ur[3].z, ur[3].w};
      const float4 *t4 = reinterpret_cast<const float4 *>(T[t]);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (4 * q < r) {
          const float4 v = t4[q];
          lr += bf2f((uint16_t)w16[2 * q]) * v.x;
          lr += bf2f((uint16_t)(w16[2 * q] >> 16)) * v.y;
          lr += bf2f((uint16_t)w16[2 * q + 1]) * v.z;
          lr += bf2f((uint16_t)(w16[2 * q + 1] >> 16)) * v.w;
        }
      }
    } else if (B.ufast) {
      for (int j0 = 0; j0 < r; j0 += 8) {
        const uint4 uv = ld16(u + j0);
        const uint32_t w4[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) lr += bf2f((uint16_t)(w4[q >> 1] >> ((q & 1) * 16))) * T[t][j0 + q];
      }
    } else {
      for (int j = 0; j < r; ++j) lr += bf2f(u[j]) * T[t][j];
    }
    a.y[(size_t)m * a.ldy + B.col + n] = f2bf(sn * z[t] + lr);
  }
}

// ---------------------------------------------------------------- host side

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
  const int ngmax_f = pl->MT == 1 ? 5 : ngmax;    // fused tiles: one more group at 16 tokens
  const int ngmin = vgmax + 1 > 2 ? vgmax + 1 : 2;

  // Cost model (microseconds), fitted to sweeps over the Gemma-3-1B and
  // large-decoder decode shapes on MI355X.  A dispatch lasts as long as its
  // most loaded CU: ceil(units / 256) work units in turn, each paying a fixed
  // ~0.8 us (argument loads, first-load latency, epilogue) plus its bytes at
  // the ~21.5 GB/s that one CU sustains when all 256 stream at once.  Vt rows
  // re-read by every fused tile come from L2 and count 0.7 of a W0 row.  Split
  // mode adds the combine launch (~3.7 us with its graph node).  Tiles hold any
  // number of rows up to what the compiled tile holds, so that 2 x 6912 rows
  // become 256 tiles of 54 (one per CU) and a 1536-row QKV 221 tiles of 7.
  constexpr double kUnit = 0.8, kRate = 21500.0, kVtW = 0.7, kComb = 3.7;
  auto rounds = [](long units) { return (double)((units + kNumCU - 1) / kNumCU); };
  auto tiles_of = [&](int R, bool with_vt) {
    long t = 0;
    for (int b = 0; b < rq.nblk; ++b) {
      t += (rq.blk[b].N + R - 1) / R;
      if (with_vt && rq.blk[b].r > 0) t += (rq.blk[b].r + R - 1) / R;
    }
    return t;
  };
  int Rf = 0;
  double best_f = 1e30;
  for (int R = 4; R <= 16 * (ngmax_f - vgmax); ++R) {
    const double c = rounds(tiles_of(R, false)) * (kUnit + (R + kVtW * 16 * vgmax) * K * 2.0 / kRate);
    if (c < best_f - 1e-9) { best_f = c; Rf = R; }
  }
  int Rs = 16, Ss = 1;
  double best_s = 1e30;
  const int smax = K / 256 > 1 ? (K / 256 < 16 ? K / 256 : 16) : 1;
  // A workgroup with four or more 16-row groups streams faster than one with
  // fewer (more rows' loads in flight per wave), which the model, linear in
  // rows, does not see.  Where there are at least 64 tiles of 64 rows, the
  // split search takes only such tiles: on the large-decoder QKV, 27.3 us
  // (67 rows, K in two) against 29.9 (three groups) at 32 tokens, and o 14.8
  // against 16.1 at one.  Fewer tiles than that (the Gemma-3-1B QKV, o, down)
  // would need very short K ranges to fill the CUs, which measured slower.
  const int rlo = (ngmax >= 4 && tiles_of(64, true) >= 64) ? 49 : 8;
  auto search_split = [&](int smin) {
    for (int R = rlo; R <= 16 * ngmax; ++R) {
      const long t = tiles_of(R, true);
      for (int sc = smin; sc <= smax; ++sc) {
        const int kc = ((K + sc - 1) / sc + 127) / 128 * 128;
        const int sr = (K + kc - 1) / kc;
        if (sr != sc) continue;
        const double c = rounds(t * sr) * (kUnit + (double)R * kc * 2.0 / kRate) + kComb;
        if (c < best_s - 1e-9) { best_s = c; Rs = R; Ss = sr; }
      }
    }
  };
  search_split(1);
  // One token, K unsplit over more than two rounds of units: the model's
  // rounds are synchronous, but the units are not, and shorter ones (K in
  // three or more ranges) let the CUs that stream faster take more of them --
  // the large-decoder gate/up (2 x 21504 x 5376) 81 us against 91 with the
  // model's 757 unsplit units of 57 rows (weights beyond the Infinity Cache).
  // At 16 and 32 tokens the unsplit plans measured best.
  if (pl->MT == 1 && Ss == 1 && tiles_of(Rs, true) > 2L * kNumCU && smax >= 3) {
    best_s = 1e30;
    search_split(3);
  }
  bool split = best_s < best_f;

  // Plan overrides (tests, aq_debug_force_plan): split (0/1), rows per tile,
  // W0 groups per tile (rows = 16 x groups), K splits, waves.
  const int sp_o = debug_knob(AQ_DBG_DECODE_SPLIT, -1);
  if (sp_o == 1 || (sp_o == 0 && Rf > 0)) split = sp_o == 1;
  int R = split ? Rs : Rf, S = split ? Ss : 1;
  const int rmax = split ? 16 * ngmax : 16 * (ngmax_f - vgmax);
  const int ng_o = debug_knob(AQ_DBG_DECODE_NG, 0);
  if (ng_o >= (split ? 1 : ngmin) && ng_o <= (split ? ngmax : ngmax_f)) R = 16 * (ng_o - (split ? 0 : vgmax));
  const int r_o = debug_knob(AQ_DBG_DECODE_ROWS, 0);
  if (r_o >= 1 && r_o <= rmax) R = r_o;
  if (split) {
    const int s_o = debug_knob(AQ_DBG_DECODE_S, 0);
    if (s_o >= 1) S = s_o;
  }
  if (R < 1) return false;
  int NG = split ? (R + 15) / 16 : vgmax + (R + 15) / 16;
  if (!split && NG < ngmin) NG = ngmin;
  if (NG > (split ? ngmax : ngmax_f)) return false;
  int WAVES = 4;
  const int w_o = debug_knob(AQ_DBG_DECODE_WAVES, 0);
  if (w_o == 4 || (pl->MT == 1 && w_o == 8)) WAVES = w_o;

  int kchunk = (K + S - 1) / S;
  kchunk = (kchunk + 127) / 128 * 128;
  S = (K + kchunk - 1) / kchunk;
  // 32-bit buffer offsets: one tile's rows must stay below 2^31 bytes.
  if ((int64_t)16 * NG * K * 2 >= (int64_t(1) << 31)) return false;

  pl->split = split;
  pl->NG = NG;
  pl->S = S;
  pl->WAVES = WAVES;
  pl->kchunk = kchunk;
  int t0 = 0, nseg = 0, tcol = (int)rq.Ntot;
  for (int b = 0; b < rq.nblk; ++b) {
    const Proj &P = rq.blk[b];
    pl->seg[nseg++] = DecodeSeg{b, 0, t0, (int)((P.N + R - 1) / R), R};
    t0 += pl->seg[nseg - 1].ntile;
    if (!split) continue;
    pl->tcol[b] = tcol;
    if (P.r > 0) {
      pl->seg[nseg++] = DecodeSeg{b, 1, t0, (int)((P.r + R - 1) / R), R};
      t0 += pl->seg[nseg - 1].ntile;
      tcol += (int)P.r;
    }
  }
  pl->nseg = nseg;
  pl->ntiles = t0;
  pl->Wp = tcol;
  pl->ws_bytes = split ? kWsReserved + (size_t)S * M * tcol * 4 : 0;
  return true;
}

template <int MT, int NG, int WAVES, bool PART>
static void launch_one(const DecArgs &a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((k_decode_bf16<MT, NG, WAVES, PART>), dim3(grid), dim3(64 * WAVES), 0, st, a);
}

template <int MT, int WAVES, bool PART>
static bool launch_ng(const DecArgs &a, int NG, int grid, hipStream_t st) {
  switch (NG) {
    case 1:
      if constexpr (PART) { launch_one<MT, 1, WAVES, PART>(a, grid, st); return true; }
      return false;
    case 2: launch_one<MT, 2, WAVES, PART>(a, grid, st); return true;
    case 3: launch_one<MT, 3, WAVES, PART>(a, grid, st); return true;
    case 4:
      if constexpr (MT < 4) { launch_one<MT, 4, WAVES, PART>(a, grid, st); return true; }
      return false;
    case 5:
      if constexpr (MT == 2 || (MT == 1 && !PART && WAVES == 4)) { launch_one<MT, 5, WAVES, PART>(a, grid, st); return true; }
      return false;
    case 6:
      if constexpr (MT == 2) { launch_one<MT, 6, WAVES, PART>(a, grid, st); return true; }
      return false;
  }
  return false;
}

template <int MT, bool PART>
static bool launch_w(const DecArgs &a, int NG, int WAVES, int grid, hipStream_t st) {
  if constexpr (MT == 1) {
    if (WAVES == 8) return launch_ng<1, 8, PART>(a, NG, grid, st);
  }
  return WAVES == 4 ? launch_ng<MT, 4, PART>(a, NG, grid, st) : false;
}

template <bool PART>
static bool launch_mt(const DecArgs &a, const DecodePlan &pl, int grid, hipStream_t st) {
  switch (pl.MT) {
    case 1: return launch_w<1, PART>(a, pl.NG, pl.WAVES, grid, st);
    case 2: return launch_w<2, PART>(a, pl.NG, pl.WAVES, grid, st);
    case 4: return launch_w<4, PART>(a, pl.NG, pl.WAVES, grid, st);
  }
  return false;
}

hipError_t launch_decode(const Recon &rq, const DecodePlan &pl, void *ws, hipStream_t st) {
  DecArgs a = {};
  a.x = (const uint16_t *)rq.x;
  a.y = (uint16_t *)rq.y;
  a.part = pl.split ? (float *)((char *)ws + kWsReserved) : nullptr;
  a.ldx = (int)rq.ldx;
  a.ldy = (int)rq.ldy;
  a.M = (int)rq.M;
  a.K = (int)rq.K;
  a.Wp = pl.Wp;
  a.ntiles = pl.ntiles;
  a.S = pl.S;
  a.kchunk = pl.kchunk;
  for (int i = 0; i < kMaxSegs; ++i) a.tile0[i] = i < pl.nseg ? pl.seg[i].tile0 : INT_MAX;
  for (int i = 0; i < pl.nseg; ++i) {
    const DecodeSeg &sg = pl.seg[i];
    const Proj &P = rq.blk[sg.b];
    DecSeg &d = a.g[i];
    d.rows = sg.rows;
    if (!pl.split) {
      d.W0 = (const uint16_t *)P.W0;
      d.s = (const uint16_t *)P.s;
      d.U = (const uint16_t *)P.U;
      d.Vt = (const uint16_t *)P.Vt;
      d.N = (int)P.N;
      d.r = (int)P.r;
      d.col = (int)P.col;
      d.vg = pl.vg[sg.b];
      d.ufast = (P.r % 8 == 0) && (((uintptr_t)P.U & 15) == 0);
    } else {
      d.W0 = (const uint16_t *)(sg.isVt ? P.Vt : P.W0);
      d.N = (int)(sg.isVt ? P.r : P.N);
      d.col = sg.isVt ? pl.tcol[sg.b] : (int)P.col;
    }
  }
  const int units = pl.ntiles * pl.S;
  const int grid = 8 * ((units + 7) / 8);
  const bool ok = pl.split ? launch_mt<true>(a, pl, grid, st) : launch_mt<false>(a, pl, grid, st);
  if (!ok) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !pl.split) return e;

  CombArgs c = {};
  c.part = a.part;
  c.y = a.y;
  c.S = pl.S;
  c.M = a.M;
  c.Wp = pl.Wp;
  c.ldy = a.ldy;
  c.nblk = rq.nblk;
  int chunks = 0;
  for (int b = 0; b < rq.nblk; ++b) {
    const Proj &P = rq.blk[b];
    CombBlk &d = c.b[b];
    d.s = (const uint16_t *)P.s;
    d.U = (const uint16_t *)P.U;
    d.N = (int)P.N;
    d.r = (int)P.r;
    d.col = (int)P.col;
    d.tcol = pl.tcol[b];
    d.chunk0 = chunks;
    d.ufast = (P.r % 8 == 0) && (((uintptr_t)P.U & 15) == 0);
    chunks += (int)((P.N + 255) / 256);
  }
  if ((long)chunks * c.M > 2048 && (size_t)pl.S * c.M * c.Wp * 4 < (size_t(1) << 31))
    hipLaunchKernelGGL(k_decode_combine4, dim3(chunks, (c.M + 3) / 4), dim3(256), 0, st, c);
  else
    hipLaunchKernelGGL(k_decode_combine, dim3(chunks, c.M), dim3(256), 0, st, c);
  return hipGetLastError();
}

}  // namespace aq
