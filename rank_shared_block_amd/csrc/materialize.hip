// Effective-weight materialisation: W_eff = diag(s) W0 + U Vt, fp32 accumulation,
// one rounding to the storage dtype.  "Execution paths", section
// "Precompute-outside" (rebuilt once at load); "How attnquant works", section
// "The reconstruction identity".
//
// bf16 kernel (gfx950):
// * Streaming W0 in and W_eff out is the bound (2 + 2 bytes per element); the
//   rank-r product costs 2 r flop per element, which at r = 64 would exceed the
//   fp32 VALU roofline, so it runs on v_mfma_f32_32x32x16_bf16.
// * A workgroup owns a block of 64 columns and a range of rows, taken 128 rows
//   (32 per wave) at a time.  The Vt block [r, 64] is staged once in LDS
//   transposed (64 columns x r ranks, rank-contiguous) and is the A operand
//   (8 consecutive ranks of one column per lane); U rows are the B operand
//   (8 consecutive ranks of one row per lane, one 16-byte load).  The result
//   comes out transposed: a lane holds one output row and, per group of four
//   accumulator values, 4 consecutive output columns.  W0 comes in and W_eff
//   goes out as whole 128-byte row pieces (16 bytes per lane) through an LDS
//   tile, where the product meets W0 in the accumulator layout.
// * Many small workgroups (four per CU) keep enough loads in flight to hide the
//   memory latency without software pipelining.
// * diag(s) W0 is added in fp32 with one fused multiply-add per element; with
//   r = 0 (or U = Vt = 0) the accumulator is +0 and the result is one rounding of
//   the exact product s * w, i.e. bit-exact.
//
// fp32 kernel: one thread per element, rank loop in fp32 FMAs, then one fused
// multiply-add with s * w.

#include "aq_internal.h"
#include "device_common.h"
#include "fp4_block.h"

namespace aq {

struct MatArgs {
  const void *W0, *s, *U, *Vt;
  void *out;
  int N, K, r, ldw, rows_per_wg, ufast;
};

// RJ: 16-rank steps (r <= 16 RJ).
template <int RJ>
__global__ __launch_bounds__(256, 4) void k_materialize_bf16(const MatArgs a) {
  constexpr int CB = 64;                    // columns per workgroup
  constexpr int RB = 128;                   // rows per step (32 per wave)
  constexpr int RP = 16 * RJ + 8;           // LDS row (one column of Vt, rank-contiguous), padded
  constexpr int WP = CB + 8;                // LDS row of the W0 / W_eff tile, padded
  __shared__ __attribute__((aligned(16))) uint16_t vts[CB * RP];
  __shared__ __attribute__((aligned(16))) uint16_t wt[RB * WP];
  const uint16_t *W0 = (const uint16_t *)a.W0, *S = (const uint16_t *)a.s;
  const uint16_t *U = (const uint16_t *)a.U, *Vt = (const uint16_t *)a.Vt;
  uint16_t *out = (uint16_t *)a.out;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int K = a.K, r = a.r, N = a.N;
  const int cb0 = blockIdx.x * CB;
  const int ncol = min(CB, K - cb0);        // a multiple of 8 (K % 8 == 0)
  const int nb = blockIdx.y * a.rows_per_wg, ne = min(N, nb + a.rows_per_wg);

  // Stage Vt[:, cb0 : cb0 + 64] transposed (zeros past r or K): thread i reads
  // 8 columns of one rank row and writes them to 8 LDS rows.
  for (int i = tid; i < 16 * RJ * (CB / 8); i += 256) {
    const int j = i % (16 * RJ), c = (i / (16 * RJ)) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j < r && c < ncol) v = ld16(Vt + (size_t)j * K + cb0 + c);
    const uint32_t q4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) vts[(c + q) * RP + j] = (uint16_t)(q4[q >> 1] >> ((q & 1) * 16));
  }
  __syncthreads();

  // A operands: column tile t (columns 32 t + lane % 32), rank step kk.
  bf16x8 av[2][RJ];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int kk = 0; kk < RJ; ++kk)
      av[t][kk] = as_bf16x8(*reinterpret_cast<const uint4 *>(&vts[(32 * t + l32) * RP + 16 * kk + 8 * hi]));

  // W0 in and W_eff out move as whole 128-byte row pieces: thread i handles the
  // 16-byte chunks i, i + 256, ... of the 128 x 64 step tile (8 per row),
  // through the LDS tile wt; the MFMA result meets W0 there, in its own layout.
  for (int n0 = nb; n0 < ne; n0 += RB) {
    const int nrow = min(RB, ne - n0);
    uint4 wv[RB * CB / 8 / 256];
#pragma unroll
    for (int q = 0; q < RB * CB / 8 / 256; ++q) {
      const int c = tid + 256 * q, row = c >> 3, col = (c & 7) * 8;
      wv[q] = row < nrow && col < ncol ? ld16(W0 + (size_t)(n0 + row) * K + cb0 + col) : make_uint4(0, 0, 0, 0);
    }
    // This lane's output row (its s, and its U row as the B operand).
    const int rl = 32 * wave + l32, n = n0 + rl;
    const bool rowok = rl < nrow;
    const uint16_t s_raw = S[rowok ? n : n0];   // branch-free: converted at its use
    bf16x8 bu[RJ];
#pragma unroll
    for (int kk = 0; kk < RJ; ++kk) {
      const int j = 16 * kk + 8 * hi;
      if (!rowok || j >= r) {
        bu[kk] = zero_bf16x8();
      } else if (a.ufast) {
        bu[kk] = as_bf16x8(ld16(U + (size_t)n * r + j));
      } else {
        uint16_t v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = (j + q < r) ? U[(size_t)n * r + j + q] : (uint16_t)0;
        uint4 u;
        u.x = v[0] | ((uint32_t)v[1] << 16);
        u.y = v[2] | ((uint32_t)v[3] << 16);
        u.z = v[4] | ((uint32_t)v[5] << 16);
        u.w = v[6] | ((uint32_t)v[7] << 16);
        bu[kk] = as_bf16x8(u);
      }
    }
#pragma unroll
    for (int q = 0; q < RB * CB / 8 / 256; ++q) {
      const int c = tid + 256 * q, row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<uint4 *>(&wt[row * WP + col]) = wv[q];
    }
    // acc[t]: column 32 t + 8 (v / 4) + 4 hi + (v % 4) of row n.  Every lane
    // takes part in the MFMAs (they read all lanes' operands).
    f32x16 acc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[t][v] = 0.f;
    if (r > 0) {
#pragma unroll
      for (int kk = 0; kk < RJ; ++kk)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[t][kk], bu[kk], acc[t], 0, 0, 0);
    }
    __syncthreads();                        // the W0 tile is in LDS
    // w_eff = s * w + acc, in place: every lane reads and writes only its own
    // 4-column groups of its own row.
    const float sv = bf2f(s_raw);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 *p = reinterpret_cast<uint2 *>(&wt[rl * WP + 32 * t + 8 * g + 4 * hi]);
        const uint2 w = *p;
        uint2 o;
        o.x = f2bf(fmaf(sv, bf2f((uint16_t)w.x), acc[t][4 * g + 0])) |
              ((uint32_t)f2bf(fmaf(sv, bf2f((uint16_t)(w.x >> 16)), acc[t][4 * g + 1])) << 16);
        o.y = f2bf(fmaf(sv, bf2f((uint16_t)w.y), acc[t][4 * g + 2])) |
              ((uint32_t)f2bf(fmaf(sv, bf2f((uint16_t)(w.y >> 16)), acc[t][4 * g + 3])) << 16);
        *p = o;
      }
    __syncthreads();                        // W_eff tile complete
#pragma unroll
    for (int q = 0; q < RB * CB / 8 / 256; ++q) {
      const int c = tid + 256 * q, row = c >> 3, col = (c & 7) * 8;
      if (row < nrow && col < ncol)
        *reinterpret_cast<uint4 *>(out + (size_t)(n0 + row) * a.ldw + cb0 + col) =
            *reinterpret_cast<const uint4 *>(&wt[row * WP + col]);
    }
    __syncthreads();                        // wt is reused by the next step
  }
}

// Ranks above 64: same arithmetic, Vt operand gathered per row block.
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

// ---- many projections per launch (load time) ----------------------------------
//
// The whole model's W_eff in a few launches instead of one per projection: a
// work unit is one 128-row x 64-column tile of a shared block W0 together with
// every output of its run (consecutive items that name the same W0, i.e. the
// layers of one band, up to kMatRunMax of them): the W0 tile is read from HBM
// once and each output's W_eff tile is formed from it with the same arithmetic
// and summation order as k_materialize_bf16 (so the bits are identical).  Units
// are numbered run by run, row block by row block, column blocks fastest, and
// remapped so that each XCD takes a contiguous range: the units that share a U
// row block or a run's Vt share one L2.  Optionally each output's largest
// magnitude (bits 0..14 of the rounded bf16 values, an exact integer maximum)
// is folded into amax[] with one atomic maximum per unit and output, which lets
// the FP4 pack skip its own pass over W_eff.
struct MatBOut {
  const uint16_t *s, *U, *Vt;
  uint16_t *w;               // W_eff (kMatStore), or the FP4 codes [N, K/2] (kMatPack)
  uint8_t *scales;           // kMatPack: the block scales [N, K/16]
  float *gscale;             // kMatPack: the global scale
  int r, ldw;
};
struct MatBRun {
  const uint16_t *W0;
  int N, K, colblocks, unit0, out0, nout;
};
struct MatBatchArgs {
  int nrun, nunits, amax0, ufast_all, steps;
  unsigned *amax;          // NULL: no maxima; else amax[amax0 + output index]
  MatBRun run[kMatBatchRuns];
  MatBOut out[kMatBatchOuts];
};
static_assert(sizeof(MatBatchArgs) <= 3584, "kernel arguments stay well inside 4 KiB");

// What a launch does with each W_eff tile: store it (bf16; with amax set, the
// maxima too), only fold its largest magnitude into amax, or encode it as
// block-16 FP4 with the global scale that amax gives (the tile is the same
// one, value for value, that kMatStore writes).
enum { kMatStore = 0, kMatMax = 1, kMatPack = 2 };

template <int RJ, int MODE>
__global__ __launch_bounds__(256, 3) void k_materialize_batch(const MatBatchArgs a) {
  constexpr int CB = 64, RB = 128;
  constexpr int RP = 16 * RJ + 8, WP = CB + 8;
  constexpr int NQ = RB * CB / 8 / 256;     // 16-byte W0 chunks per thread and step
  __shared__ __attribute__((aligned(16))) uint16_t vts[kMatRunMax][CB * RP];
  __shared__ __attribute__((aligned(16))) uint16_t wt[RB * WP];
  __shared__ unsigned red[4][kMatRunMax];
  const int unit = xcd_contiguous_tile((int)blockIdx.x, a.nunits);
  if (unit < 0) return;
  int ri = 0;
  for (int i = 1; i < a.nrun; ++i)
    if (unit >= a.run[i].unit0) ri = i;
  const MatBRun &R = a.run[ri];
  const int u = unit - R.unit0;
  const int K = R.K, N = R.N, nout = R.nout;
  // a unit: one 64-column block and a.steps row steps of 128 rows
  const int cb0 = (u % R.colblocks) * CB, g0 = (u / R.colblocks) * RB * a.steps;
  const int gend = min(N, g0 + RB * a.steps);
  const int ncol = min(CB, K - cb0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // W0 tile of a step, as 16-byte chunks (zeros past N and K)
  uint4 wv[NQ];
  auto load_w0 = [&](int n0) __attribute__((always_inline)) {
    const int nrow = min(RB, gend - n0);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int c = tid + 256 * q, row = c >> 3, col = (c & 7) * 8;
      wv[q] = row < nrow && col < ncol ? ld16(R.W0 + (size_t)(n0 + row) * K + cb0 + col) : make_uint4(0, 0, 0, 0);
    }
  };
  load_w0(g0);
  // Each output's Vt[:, cb0 : cb0 + 64], transposed (zeros past r or K), once
  // per unit: every row step uses it.
  for (int o = 0; o < nout; ++o) {
    const MatBOut &O = a.out[R.out0 + o];
    for (int i = tid; i < 16 * RJ * (CB / 8); i += 256) {
      const int j = i % (16 * RJ), c = (i / (16 * RJ)) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (j < O.r && c < ncol) v = ld16(O.Vt + (size_t)j * K + cb0 + c);
      const uint32_t q4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) vts[o][(c + q) * RP + j] = (uint16_t)(q4[q >> 1] >> ((q & 1) * 16));
    }
  }

  // Each output's largest |W_eff| before rounding: rounding to bf16 is
  // monotone and symmetric, so one rounding of that maximum is the largest
  // rounded magnitude (one max per element instead of a max over bits).
  float amx[kMatRunMax];
#pragma unroll
  for (int o = 0; o < kMatRunMax; ++o) amx[o] = 0.f;
  float gq[kMatRunMax];                     // kMatPack: each output's global scale
#pragma unroll
  for (int o = 0; o < kMatRunMax; ++o) gq[o] = 1.f;
  if constexpr (MODE == kMatPack) {
#pragma unroll
    for (int o = 0; o < kMatRunMax; ++o) {
      if (o >= nout) break;
      gq[o] = fp4_global_scale(a.amax[a.amax0 + R.out0 + o]);
      if (u == 0 && tid == 0) *a.out[R.out0 + o].gscale = gq[o];
    }
  }
  for (int n0 = g0; n0 < gend; n0 += RB) {
    const int nrow = min(RB, gend - n0);
    // This lane's output row: its s and U row (the B operand) per output.
    const int rl = 32 * wave + l32, n = n0 + rl;
    const bool rowok = rl < nrow;
    uint16_t s_raw[kMatRunMax];
    bf16x8 bu[kMatRunMax][RJ];
#pragma unroll
    for (int o = 0; o < kMatRunMax; ++o) {
      const MatBOut &O = a.out[R.out0 + (o < nout ? o : 0)];
      s_raw[o] = O.s[rowok ? n : n0];
#pragma unroll
      for (int kk = 0; kk < RJ; ++kk) {
        const int j = 16 * kk + 8 * hi;
        if (o >= nout || !rowok || j >= O.r) {
          bu[o][kk] = zero_bf16x8();
        } else if (a.ufast_all) {
          bu[o][kk] = as_bf16x8(ld16(O.U + (size_t)n * O.r + j));
        } else {
          uint16_t v[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] = (j + q < O.r) ? O.U[(size_t)n * O.r + j + q] : (uint16_t)0;
          uint4 w;
          w.x = v[0] | ((uint32_t)v[1] << 16);
          w.y = v[2] | ((uint32_t)v[3] << 16);
          w.z = v[4] | ((uint32_t)v[5] << 16);
          w.w = v[6] | ((uint32_t)v[7] << 16);
          bu[o][kk] = as_bf16x8(w);
        }
      }
    }
    __syncthreads();                        // the previous step's stores have read wt (and Vt is staged)
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int c = tid + 256 * q, row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<uint4 *>(&wt[row * WP + col]) = wv[q];
    }
    if (n0 + RB < gend) load_w0(n0 + RB);   // the next step's W0 tile, in flight during this step
    __syncthreads();
    // This lane's W0 values, in the accumulator layout (see below).
    uint2 w0[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) w0[t][g] = *reinterpret_cast<const uint2 *>(&wt[rl * WP + 32 * t + 8 * g + 4 * hi]);

#pragma unroll
    for (int o = 0; o < kMatRunMax; ++o) {
      if (o >= nout) break;
      const MatBOut &O = a.out[R.out0 + o];
      // acc[t]: column 32 t + 8 (v / 4) + 4 hi + (v % 4) of row n, as in
      // k_materialize_bf16 (same operands, same order of the rank steps).
      f32x16 acc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[t][v] = 0.f;
      if (O.r > 0) {
#pragma unroll
        for (int kk = 0; kk < RJ; ++kk)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const bf16x8 av = as_bf16x8(*reinterpret_cast<const uint4 *>(&vts[o][(32 * t + l32) * RP + 16 * kk + 8 * hi]));
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bu[o][kk], acc[t], 0, 0, 0);
          }
      }
      __syncthreads();                      // every lane is done reading wt
      const float sv = bf2f(s_raw[o]);
      float m = amx[o];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint2 w = w0[t][g];
          const float v0 = fmaf(sv, bf2f((uint16_t)w.x), acc[t][4 * g + 0]);
          const float v1 = fmaf(sv, bf2f((uint16_t)(w.x >> 16)), acc[t][4 * g + 1]);
          const float v2 = fmaf(sv, bf2f((uint16_t)w.y), acc[t][4 * g + 2]);
          const float v3 = fmaf(sv, bf2f((uint16_t)(w.y >> 16)), acc[t][4 * g + 3]);
          m = fmaxf(fmaxf(fmaxf(m, fabsf(v0)), fmaxf(fabsf(v1), fabsf(v2))), fabsf(v3));
          if constexpr (MODE != kMatMax) {
            // one rounding to bf16 each (round to nearest even; the hardware
            // conversion, two values per instruction)
            const f32x2 lo2 = {v0, v1}, hi2 = {v2, v3};
            *reinterpret_cast<uint2 *>(&wt[rl * WP + 32 * t + 8 * g + 4 * hi]) =
                make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(lo2, bf16x2)),
                           __builtin_bit_cast(uint32_t, __builtin_convertvector(hi2, bf16x2)));
          }
        }
      amx[o] = m;                           // rows and columns past the tile hold exact zeros
      if constexpr (MODE == kMatStore) {
        __syncthreads();                    // W_eff tile complete
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int c = tid + 256 * q, row = c >> 3, col = (c & 7) * 8;
          if (row < nrow && col < ncol)
            *reinterpret_cast<uint4 *>(O.w + (size_t)(n0 + row) * O.ldw + cb0 + col) =
                *reinterpret_cast<const uint4 *>(&wt[row * WP + col]);
        }
      } else if constexpr (MODE == kMatPack) {
        __syncthreads();                    // W_eff tile complete
        // 128 rows x four 16-column blocks: two blocks per thread, each read
        // from the tile as 32 bytes, encoded, one 8-byte code store and one
        // scale byte (K is a multiple of 16, so every block is whole)
        const int kb = K >> 4;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int bi = 2 * tid + h2, row = bi >> 2, col = (bi & 3) * 16;
          if (row < nrow && col < ncol) {
            const uint4 v0 = *reinterpret_cast<const uint4 *>(&wt[row * WP + col]);
            const uint4 v1 = *reinterpret_cast<const uint4 *>(&wt[row * WP + col + 8]);
            const uint32_t qv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            uint32_t lo, hb, sf;
            pack_block16(qv, gq[o], lo, hb, sf);
            const size_t n = (size_t)(n0 + row);
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint8_t *>(O.w) + n * (size_t)(K >> 1) + (cb0 + col) / 2) =
                make_uint2(lo, hb);
            O.scales[n * kb + (cb0 + col) / 16] = (uint8_t)sf;
          }
        }
      }
    }
  }
  if (MODE != kMatPack && a.amax) {
#pragma unroll
    for (int o = 0; o < kMatRunMax; ++o) {
      unsigned m = f2bf(amx[o]) & 0x7FFFu;   // the rounded maximum's magnitude bits
#pragma unroll
      for (int sh = 32; sh > 0; sh >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, sh));
      if (lane == 0) red[wave][o] = m;
    }
    __syncthreads();
    if (tid < nout) {
      const unsigned m = max(max(red[0][tid], red[1][tid]), max(red[2][tid], red[3][tid]));
      atomicMax(a.amax + a.amax0 + R.out0 + tid, m);
    }
  }
}

__global__ __launch_bounds__(256) void k_fill_u32(unsigned *p, int n, unsigned v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

int matb_rank_steps(int64_t r) { return r <= 16 ? 1 : (r <= 32 ? 2 : 4); }

hipError_t launch_materialize_batch(int n, const MatItem *it, unsigned *amax, hipStream_t st, int mode) {
  // Row steps per work unit: 128-row steps with the next W0 tile in flight;
  // longer units keep the pipeline full, shorter ones fill the CUs' last round.
  int steps = debug_knob(AQ_DBG_MAT_STEPS, 3);
  if (steps < 1 || steps > 8) steps = 3;
  if (amax && mode != kMatPack) {
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, amax, n, 0u);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int i = 0;
  while (i < n) {
    // One launch: whole runs (consecutive items on one W0, at most kMatRunMax
    // per run) while they fit in the argument block; the rank steps of the
    // largest rank of the launch.
    MatBatchArgs a = {};
    a.amax = amax;
    a.amax0 = i;
    a.ufast_all = 1;
    a.steps = steps;
    int nout = 0, units = 0, rj = 1;
    while (i + nout < n && a.nrun < kMatBatchRuns) {
      const MatItem &f = it[i + nout];
      int len = 1;
      while (len < kMatRunMax && i + nout + len < n) {
        const MatItem &g = it[i + nout + len];
        if (g.W0 != f.W0 || g.N != f.N || g.K != f.K) break;
        ++len;
      }
      if (nout + len > kMatBatchOuts) break;
      MatBRun &R = a.run[a.nrun++];
      R.W0 = (const uint16_t *)f.W0;
      R.N = (int)f.N;
      R.K = (int)f.K;
      R.colblocks = (int)((f.K + 63) / 64);
      R.unit0 = units;
      R.out0 = nout;
      R.nout = len;
      units += R.colblocks * (int)((f.N + 128 * steps - 1) / (128 * steps));
      for (int o = 0; o < len; ++o) {
        const MatItem &g = it[i + nout + o];
        MatBOut &O = a.out[nout + o];
        O.s = (const uint16_t *)g.s;
        O.U = (const uint16_t *)g.U;
        O.Vt = (const uint16_t *)g.Vt;
        O.w = (uint16_t *)(mode == kMatPack ? (void *)g.packed : g.w);
        O.scales = (uint8_t *)g.scales;
        O.gscale = g.gscale;
        O.r = (int)g.r;
        O.ldw = (int)g.ldw;
        if (!(g.r % 8 == 0 && ((uintptr_t)g.U & 15) == 0)) a.ufast_all = 0;
        const int q = matb_rank_steps(g.r);
        rj = q > rj ? q : rj;
      }
      nout += len;
    }
    a.nunits = units;
    const dim3 grid((unsigned)(8 * ((units + 7) / 8)));
#define AQ_MATB(M)                                                          \
  if (mode == M) {                                                          \
    if (rj == 1)                                                            \
      hipLaunchKernelGGL((k_materialize_batch<1, M>), grid, dim3(256), 0, st, a); \
    else if (rj == 2)                                                       \
      hipLaunchKernelGGL((k_materialize_batch<2, M>), grid, dim3(256), 0, st, a); \
    else                                                                    \
      hipLaunchKernelGGL((k_materialize_batch<4, M>), grid, dim3(256), 0, st, a); \
  }
    AQ_MATB(kMatStore)
    AQ_MATB(kMatMax)
    AQ_MATB(kMatPack)
#undef AQ_MATB
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    i += nout;
  }
  return hipSuccess;
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
  if (p.r <= 64) {
    // 64-column blocks; row ranges sized for about four workgroups per CU,
    // at least one 32-row block per wave.
    const int colblocks = (int)((K + 63) / 64);
    long rows = (p.N * colblocks + 4 * kNumCU - 1) / (4 * kNumCU);
    rows = (rows + 127) / 128 * 128;
    if (rows < 128) rows = 128;
    a.rows_per_wg = (int)rows;
    const long nrb = (p.N + rows - 1) / rows;
    dim3 grid((unsigned)colblocks, (unsigned)nrb);
    if (p.r <= 16)
      hipLaunchKernelGGL((k_materialize_bf16<1>), grid, dim3(256), 0, st, a);
    else if (p.r <= 32)
      hipLaunchKernelGGL((k_materialize_bf16<2>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((k_materialize_bf16<4>), grid, dim3(256), 0, st, a);
  } else {
    // Row blocks sized for about two workgroups per CU.
    const int colblocks = (int)((K + 127) / 128);
    long rows = (p.N * colblocks + 2 * kNumCU - 1) / (2 * kNumCU);
    rows = (rows + 31) / 32 * 32;
    if (rows < 32) rows = 32;
    a.rows_per_wg = (int)rows;
    const long nrb = (p.N + rows - 1) / rows;
    const unsigned gy = (unsigned)(nrb < 65535 ? nrb : 65535);
    dim3 grid((unsigned)colblocks, gy);
    hipLaunchKernelGGL(k_materialize_bf16_highrank, grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace aq
