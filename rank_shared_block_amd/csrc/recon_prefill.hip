// Tiled MFMA reconstruction for large batches (prefill), bf16 in, fp32
// accumulation, bf16 out.
//
// What it computes ("How attnquant works", section "The reconstruction identity";
// "Execution paths", section "The GEMM formulation"):
//     t                 = x Vt_b^T                       (rank-r down-projection)
//     y[:, col_b + n]   = s_b[n] * (x W0_b^T)[:, n] + (t U_b^T)[:, n]
// The pages run this as stock GEMMs (one over [W0^T, V], one block-diagonal
// up-projection) plus an elementwise combine.  Here:
// * where one round of tiles covers the output (few, latency-bound tiles) and
//   r <= 64, each tile computes its own rows of t: its block's Vt rows ride in
//   every LDS stage next to its W0 rows (the concatenated [W0^T, V] GEMM per
//   tile), and t goes from the accumulators to LDS, never to memory;
// * else the rank-r pass, t = x [Vt_q; Vt_k; ...]^T for every block of the
//   dispatch, is the same GEMM on small tiles.  Where its tiles fit in the CU
//   slots the main pass leaves free, it runs in the first workgroups of the
//   main pass's own launch: they publish t (bf16) with device-coherent stores
//   and count themselves in the workspace; the main tiles wait for the count
//   only before they first read t, near the end of their K loop.  Otherwise it
//   is a launch of its own, K-split over enough workgroups for long K, with a
//   small kernel folding the fp32 partials (in split order) into the bf16 t
//   buffer;
// * the main pass: the W0 contraction, then an in-register epilogue: acc *= s[n]
//   once, then acc += t U^T as further MFMA k-steps over rank chunks that were
//   loaded into the LDS ring like K slices (t where x goes, U where W0 goes),
//   then one rounding to bf16.  t is an MFMA operand and so held in bf16;
//   everything else is fp32 until the final store.
//
// GEMM design (gfx950, measured: v_mfma_f32_32x32x16_bf16 sustains ~2.2 PFLOP/s
// over the chip, LDS reads > 180 B/clk/CU):
// * BM x BN output tile per workgroup of NW = 4 or 8 waves in a 2 x (NW / 2)
//   grid of wave tiles of 32x32 MFMA tiles (128 x 64 per wave in the large
//   shapes).  The main loop of those is bound by issuing the global -> LDS
//   loads, so the largest dispatches use 256 x 256 with eight waves: one
//   workgroup per CU, two waves per SIMD, a third fewer bytes per flop than
//   256 x 128.
// * K in slices of 32 or 64 through a ring of NST LDS stages, NST - 1 slices in
//   flight while one is multiplied; the loads of a slice are spread over the
//   MFMAs of the step.  Each stage is its own LDS object and the ring is
//   unrolled, so the compiler can see that the loads landing in one stage never
//   alias the fragment reads of another and does not wait for them.  With eight
//   waves each step's barrier sits before its last k-step and the next slice's
//   first fragments are read under that k-step's MFMAs.
// * Operands go global -> LDS directly (buffer_load ... lds, 16 bytes per lane):
//   no staging registers; rows or K past the end fall outside the buffer
//   resource and land in LDS as zeros.
// * 16-byte chunks of an LDS row are XOR-swizzled by row, so the 16 rows read
//   by 16 lanes of one fragment load cover all 64 banks once.
// * Each wave stages its output block through a free LDS stage, 32 rows at a
//   time, and writes it with 16-byte row-contiguous stores one round late.
//   Tiles are handed to XCDs in contiguous ranges (m fastest), so the
//   workgroups of one XCD share the W0 rows of a column tile in L2.
// * When the tiles cannot cover the 256 CUs (long K, few tiles), K is split
//   over S workgroups that write fp32 partials (all apply s; split 0 adds t U^T,
//   or with the rank-r pass in the same launch every split adds the rank term
//   of its own K range), and a small kernel adds them in split order.
//   Deterministic.

#include <type_traits>

#include "aq_internal.h"
#include "device_common.h"
#include "handoff.h"

namespace aq {

namespace {
// MODE_SELF: MODE_RECON for tiles that also compute their own rows of t
// (their Vt rows ride in every LDS stage next to the W0 rows).
enum { MODE_RECON = 0, MODE_PART = 1, MODE_RAW = 2, MODE_SELF = 3 };
}  // namespace

struct PfBlk {
  const uint16_t *W, *s, *U, *Vt;   // Vt: MODE_SELF only
  int N;       // valid rows of W (output columns computed)
  int Nst;     // output columns stored (>= N: padding columns are stored as 0)
  int r, col, tcol, ntn, tile0, ufast;
};

struct PfArgs {
  const uint16_t *x;
  uint16_t *y;
  float *part;             // [S][M][ldp] fp32 partials (MODE_PART, MODE_RAW)
  const uint16_t *t;       // bf16 [M][ldt] (MODE_RECON, MODE_PART)
  int ldx, ldy, ldt, ldp, M, K, nblk, ntm, ntiles, S, kchunk, vec_store;
  // Rank-r pass run by the first tgrid workgroups of the main-pass launch
  // (0: none): they publish t with device-coherent stores (coherent = 1 in
  // their arguments) and count themselves in the workspace; the main units
  // that need t wait for them before they first read t (handoff.h).
  int tgrid, coherent;
  HandoffWait hw;
  // tsplit: t is kept per K range (t_p = x_p Vt_p^T, bf16, at t + p * tstride)
  // and every K-split unit p adds t_p U^T to its partial (the rank term is
  // linear in K, so the fold of the partials sums it); the rank-r tiles write
  // t_p the same way (y + p * tstride).
  int tsplit;
  // tparts: with the main pass unsplit, t may still be kept as tparts per-K-range
  // parts (the rank-r tiles split K so that they finish well before the main
  // tiles); every main unit then adds (sum_p t_p) U^T, each part as more rank
  // chunks.  1 otherwise.
  int tparts;
  long tstride;
  unsigned *sync;
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

// s_waitcnt with vmcnt <= n and no wait on the other counters (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt 7, lgkmcnt 15).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// Workgroup barrier without a memory fence: the stage ring orders LDS itself
// (explicit vmcnt waits for the direct loads; fragment reads are consumed by the
// MFMAs before the barrier).  The memory clobber keeps the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Workgroups per CU a tile shape is built for: two when its LDS ring fits in
// half of the 160 KiB (registers are then capped at 256 per lane).
template <int BM, int BN, int BK, int NST, int RT = 0>
constexpr int gemm_occupancy() { return (BM + BN + RT) * BK * 2 * NST + BN * 4 <= 80 * 1024 ? 2 : 1; }

// NW waves per workgroup in a 2 x (NW / 2) grid: four (one or two workgroups
// per CU) or eight (one workgroup per CU, two waves per SIMD, for 256 x 256
// tiles: the same 128 x 64 wave tile as 256 x 128 with four waves, with a
// third fewer bytes loaded per flop).
template <int BM, int BN, int BK, int NST, int MODE, int NW>
__device__ __attribute__((always_inline)) inline void gemm_tile(const PfArgs &a, const int unit, uint16_t *const st0,
                                                               uint16_t *const st1, uint16_t *const st2,
                                                               uint16_t *const st3, float *const s_lds) {
  // Waves in a 2 x (NW / 2) grid, or NW x 1 where BN does not split into
  // 32-multiples over NW / 2 wave columns (BN = 96).
  constexpr int WGM = (BN / (NW / 2)) % 32 == 0 ? 2 : NW;
  constexpr int WGN = NW / WGM;                    // waves along N
  constexpr int WM = BM / WGM, WN = BN / WGN;      // wave tile
  constexpr int TM = WM / 32, TN = WN / 32;        // 32x32 MFMA tiles per wave
  constexpr bool SELF = MODE == MODE_SELF;
  constexpr int RT = SELF ? 64 : 0;                // Vt rows per stage (the tile's own t, r <= 64)
  constexpr int TNT = SELF ? RT / WGN / 32 : 0;    // 32x32 t tiles per wave
  constexpr int STAGE = (BM + BN + RT) * BK;       // bf16 elements per LDS stage
  constexpr int CPR = BK / 8;                      // 16-byte chunks per LDS row
  constexpr int RPL = 64 / CPR;                    // rows per 1 KiB load
  constexpr int LA = BM / (NW * RPL), LB = BN / (NW * RPL);   // loads per wave per stage
  constexpr int LT = RT / (NW * RPL);
  constexpr int LPS = LA + LB + LT;
  static_assert(!SELF || (NW == 4 && TNT >= 1 && LT * NW * RPL == RT), "own-t tiles: four waves, 64 Vt rows");
  static_assert(!SELF || 64 / BK <= (64 * (BN + 8) <= (BM + BN + RT) * BK ? NST - 1 : NST - 2),
                "own-t tiles: every rank chunk of t rides the ring");
  static_assert(BM % 64 == 0 && BN % 32 == 0 && WM % 32 == 0, "tile must be a multiple of 64 x 32");
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(WN % 32 == 0 && LA * NW * RPL == BM && LB * NW * RPL == BN, "wave tiles and loads must divide the tile");
  static_assert(BK == 32 || BK == 64, "K slice of 32 or 64");
  static_assert(NST >= 2 && NST <= 4, "2 to 4 LDS stages");

  // wave is read back from lane 0 so that the compiler knows it is uniform: the
  // LDS address of a direct load (M0) is per wave.
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, lhi = lane >> 5;
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

  // Swizzle: chunk c of LDS row R sits at position c ^ sw(R), with
  // sw(R) = (R / 4) mod 4 for 4-chunk rows and (R / 2) mod 8 for 8-chunk rows,
  // so the 16 rows that 16 lanes of a fragment load read cover all 64 banks
  // once.  Loader: load j of this wave fills RPL rows (1 KiB) of a stage; lane
  // l writes row RPL q + l / CPR at position l % CPR.
  auto sw = [](int R) { return CPR == 4 ? (R >> 2) & 3 : (R >> 1) & 7; };
  const int lrow = lane / CPR, lpos = lane % CPR;
  int aoff[LA], boff[LB], achk[LA], bchk[LB];
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int row = (wave * LA + j) * RPL + lrow;
    aoff[j] = row * a.ldx * 2;
    achk[j] = lpos ^ sw(row);
  }
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int row = (wave * LB + j) * RPL + lrow;
    boff[j] = row * K * 2;
    bchk[j] = lpos ^ sw(BM + row);
  }
  int voff[LT > 0 ? LT : 1], vchk[LT > 0 ? LT : 1];
#pragma unroll
  for (int j = 0; j < LT; ++j) {
    const int row = (wave * LT + j) * RPL + lrow;
    voff[j] = row * K * 2;
    vchk[j] = lpos ^ sw(BM + BN + row);
  }
  // The epilogue's rank-r term (see below) needs the tile's rows of t and U.
  // They ride on the slices issued past the end of the ring (nkp .. nkp +
  // NST - 2, never multiplied): rank chunk c (ranks BK c .. BK c + BK - 1) as
  // slice nkp + c, t rows where x rows go and U rows where W rows go, so that
  // their latency hides under the last steps.  Ranks past r16 (t) or r (U) and
  // rows past M or N read as zero; U takes this path only with 16-byte aligned
  // rows (ufast).
  // With t in parts (tparts > 1), rank chunk c is chunk c % nchunk1 of part
  // c / nchunk1: the parts are summed by the same MFMAs.
  // MODE_SELF: no t in memory (its rank chunk's t rows are written from
  // registers after the K loop).
  const bool addu = MODE != MODE_RAW && (MODE == MODE_RECON || SELF || p == 0 || a.tsplit) && B.r > 0;
  const uint16_t *const tbase = a.t + (a.tsplit ? (size_t)p * a.tstride : 0);
  const int r16 = (B.r + 15) & ~15;
  const int tparts = MODE == MODE_RAW || SELF ? 1 : a.tparts;
  const int nchunk1 = (r16 + BK - 1) / BK;         // rank chunks per part of t
  const __amdgpu_buffer_rsrc_t rt = make_rsrc(
      tbase + (size_t)m0 * a.ldt,
      addu && !SELF ? (uint32_t)(((size_t)(tparts - 1) * a.tstride + (size_t)mrows * a.ldt) * 2) : 0u);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(SELF ? B.Vt : a.x, SELF && B.r > 0 ? (uint32_t)(B.r * K * 2) : 0u);
  const __amdgpu_buffer_rsrc_t ru =
      make_rsrc(B.U + (size_t)n0 * B.r, addu && nrows > 0 && B.ufast ? (uint32_t)(nrows * B.r * 2) : 0u);
  auto part_of = [&](int c) __attribute__((always_inline)) { return tparts == 1 ? 0 : c / nchunk1; };
  auto eoff_a = [&](int d, int c) __attribute__((always_inline)) {
    const int pe = part_of(c);
    const int row = (wave * LA + d) * RPL + lrow, col = BK * (c - pe * nchunk1) + 8 * achk[d];
    // rows past M stay out of range also where another part follows
    return col < r16 && row < mrows ? (int)(pe * a.tstride + row * a.ldt + B.tcol + col) * 2 : kOOB;
  };
  auto eoff_b = [&](int d, int c) __attribute__((always_inline)) {
    const int row = (wave * LB + d) * RPL + lrow, col = BK * (c - part_of(c) * nchunk1) + 8 * bchk[d];
    return col < B.r ? (row * B.r + col) * 2 : kOOB;
  };

  // Every load is issued (an out-of-range offset for K past the range or a
  // slice past the last), selected without branches, so that the number of
  // loads per stage is fixed and the compiler's wait counting stays exact.
  // Load d of a stage: d < LA an x (A) block, else a W (B) block; with
  // ech >= 0 the blocks of rank chunk ech instead.
  auto dma = [&](int d, int k0, int klim, int ech, uint16_t *stage) __attribute__((always_inline)) {
    if (d < LA) {
      const int kk = k0 + 8 * achk[d];
      const int off = kk < klim ? aoff[d] + kk * 2 : kOOB;
      lds_load16(ech >= 0 ? rt : rx, stage + (wave * LA + d) * 512, ech >= 0 ? eoff_a(d, ech) : off);
    } else if (d >= LA + LB) {          // Vt rows (MODE_SELF); none in a rank chunk
      const int kk = k0 + 8 * vchk[d - LA - LB];
      const int off = kk < klim && ech < 0 ? voff[d - LA - LB] + kk * 2 : kOOB;
      lds_load16(rv, stage + (BM + BN) * BK + (wave * LT + d - LA - LB) * 512, off);
    } else {
      const int kk = k0 + 8 * bchk[d - LA];
      const int off = kk < klim ? boff[d - LA] + kk * 2 : kOOB;
      lds_load16(ech >= 0 ? ru : rw, stage + BM * BK + (wave * LB + d - LA) * 512, ech >= 0 ? eoff_b(d - LA, ech) : off);
    }
  };
  auto issue = [&](int slice, uint16_t *stage) __attribute__((always_inline)) {
    const int k0 = kbeg + slice * BK, klim = slice < nk ? kend : -1;
#pragma unroll
    for (int d = 0; d < LPS; ++d) dma(d, k0, klim, -1, stage);
  };

  const int wm = wave / WGN, wn = wave % WGN;
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  // MODE_SELF: this wave's block of t = x Vt^T (rows as acc, ranks wn * 32 ..)
  constexpr int TNT1 = TNT > 0 ? TNT : 1;
  f32x16 acct[TM][TNT1];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TNT1; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acct[i][j][v] = 0.f;

  // Fragment reads: lane (l32, lhi) reads row R = base + l32 at chunk
  // 2 kk + lhi; every base is a multiple of 32, so sw(R) = sw(l32).
  const int swz = sw(l32);
  const int arow = (wm * WM + l32) * BK, brow = (BM + wn * WN + l32) * BK;
  auto frags = [&](const uint16_t *stage, int kk, bf16x8 (&af)[TM], bf16x8 (&bf)[TN]) __attribute__((always_inline)) {
    const int c = 8 * ((2 * kk + lhi) ^ swz);
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = as_bf16x8(*reinterpret_cast<const uint4 *>(stage + arow + i * 32 * BK + c));
#pragma unroll
    for (int j = 0; j < TN; ++j) bf[j] = as_bf16x8(*reinterpret_cast<const uint4 *>(stage + brow + j * 32 * BK + c));
  };
  const int vrow = (BM + BN + wn * (RT / WGN) + l32) * BK;
  auto tfrags = [&](const uint16_t *stage, int kk, bf16x8 (&tf)[TNT1]) __attribute__((always_inline)) {
    const int c = 8 * ((2 * kk + lhi) ^ swz);
#pragma unroll
    for (int j = 0; j < TNT; ++j) tf[j] = as_bf16x8(*reinterpret_cast<const uint4 *>(stage + vrow + j * 32 * BK + c));
  };

  // One step of the ring: multiply the stage `cur` while the loads of slice
  // `nslice` into `next` go out.  The loads are spread over the MFMA stream (a
  // group of TN MFMAs per slot, KK * TM slots) instead of being issued in one
  // burst: the texture unit takes 16 cycles per 1 KiB load, and a wave whose
  // load cannot issue stalls its MFMAs too.  The fragments of k-step kk + 1 are
  // read while k-step kk is multiplied.
  constexpr int KK = BK / 16, SLOTS = KK * TM;
  const int nkp = (nk + NST - 1) / NST * NST;    // slices past nk are zeros
  // rank chunks of the epilogue (MODE_SELF: the one it computes, r <= 64)
  const int nchunk = SELF ? (nchunk1 < 64 / BK ? nchunk1 : 64 / BK) : nchunk1 * tparts;
  // ... riding on the tail slices (all but the last, or all but the last two
  // when the output block needs two stages for staging)
  constexpr int ESLOTS = WGM * 32 * (BN + 8) <= STAGE ? NST - 1 : NST - 2;
  const int nech = addu ? min(nchunk, ESLOTS) : 0;
  // TAIL: the step may issue a slice past nkp (a rank chunk); only the last
  // NST steps can, so the others are compiled without that selection.
  auto step = [&](auto tail, int nslice, uint16_t *next, const uint16_t *cur) __attribute__((always_inline)) {
    const int k0 = kbeg + nslice * BK, klim = nslice < nk ? kend : -1;
    const int ech = decltype(tail)::value && nslice >= nkp && nslice - nkp < nech ? nslice - nkp : -1;
    bf16x8 fa[2][TM], fb[2][TN], ft[2][TNT1];
    frags(cur, 0, fa[0], fb[0]);
    if constexpr (SELF) tfrags(cur, 0, ft[0]);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (kk + 1 < KK) {
        frags(cur, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
        if constexpr (SELF) tfrags(cur, kk + 1, ft[(kk + 1) & 1]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        // W rows are the A operand and x rows the B operand, so that the
        // result comes out transposed: a lane holds 4 consecutive output
        // columns of one output row per group of 4 values.
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kk & 1][j], fa[kk & 1][i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < TNT; ++j)
          acct[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ft[kk & 1][j], fa[kk & 1][i], acct[i][j], 0, 0, 0);
        const int t = kk * TM + i;
#pragma unroll
        for (int d = t * LPS / SLOTS; d < (t + 1) * LPS / SLOTS; ++d) dma(d, k0, klim, ech, next);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // The same step with the next slice's barrier inside it (NST >= 3): before
  // the last k-step, wait for this wave's loads of the next slice and for its
  // own reads of `cur`, pass the barrier (everyone's loads of the next slice
  // have landed and everyone is done reading `cur`), then read the next
  // slice's first fragments (`nxt`, into f0) while the last k-step's MFMAs
  // run.  So neither the barrier nor the first fragment reads after it leave
  // the MFMA pipes idle.  The loads issued in this step go into the stage of
  // slice s - 1, which everyone finished reading before the previous step's
  // barrier.
  constexpr int PA = ((KK - 1) * TM * LPS) / SLOTS;  // loads issued before the barrier
  // Used with eight waves (two per SIMD of one workgroup, whose barrier waits
  // took ~20% of the loop); four-wave shapes measured no better with it.
  constexpr bool kSplitBar = NST >= 3 && NW == 8;
  auto step2 = [&](auto tail, int nslice, uint16_t *next, const uint16_t *cur, const uint16_t *nxt,
                   bf16x8(&f0a)[TM], bf16x8(&f0b)[TN]) __attribute__((always_inline)) {
    const int k0 = kbeg + nslice * BK, klim = nslice < nk ? kend : -1;
    const int ech = decltype(tail)::value && nslice >= nkp && nslice - nkp < nech ? nslice - nkp : -1;
    // The carried fragments were requested a k-step ago: wait for them before
    // requesting more, so that the first MFMAs do not wait for the new reads
    // (across the loop's back edge the compiler would wait for all of them).
    // As a builtin, so that the compiler's own wait counting sees it.
    __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0) only
    bf16x8 fa[2][TM], fb[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[0][i] = f0a[i];
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[0][j] = f0b[j];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (kk + 1 < KK) frags(cur, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
      if (kk == KK - 1) {
        wait_vmcnt<(NST - 3) * LPS + PA>();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        ring_barrier();
        frags(nxt, 0, f0a, f0b);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kk & 1][j], fa[kk & 1][i], acc[i][j], 0, 0, 0);
        const int t = kk * TM + i;
#pragma unroll
        for (int d = t * LPS / SLOTS; d < (t + 1) * LPS / SLOTS; ++d) dma(d, k0, klim, ech, next);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Slice s lives in stage s % NST.  At step s: wait until this wave's loads of
  // slice s have landed (the NST - 2 younger slices may still be in flight),
  // then a barrier (everyone's have landed, and everyone is done with slice
  // s - 1), then slice s is multiplied while the loads of slice s + NST - 1 go
  // into the stage of slice s - 1.  Past the last slice the loads are out of
  // range (zeros, no memory traffic), which keeps the wait counts uniform.
  // The ring is written out per stage count with the stage objects named, so
  // that the compiler keeps their distinct alias scopes and adds no waits.
#define AQ_STEP(tail, slice, next, cur)      \
  wait_vmcnt<(NST - 2) * LPS>();             \
  ring_barrier();                            \
  step(tail, (slice) + NST - 1, next, cur);
#define AQ_STEP2(tail, slice, next, cur, nxt) step2(tail, (slice) + NST - 1, next, cur, nxt, f0a, f0b);
#define AQ_GROUP(tail, s)                       \
  if constexpr (NST == 2) {                     \
    AQ_STEP(tail, s, st1, st0)                  \
    AQ_STEP(tail, s + 1, st0, st1)              \
  } else if constexpr (NST == 3 && !kSplitBar) { \
    AQ_STEP(tail, s, st2, st0)                  \
    AQ_STEP(tail, s + 1, st0, st1)              \
    AQ_STEP(tail, s + 2, st1, st2)              \
  } else if constexpr (NST == 3) {              \
    AQ_STEP2(tail, s, st2, st0, st1)            \
    AQ_STEP2(tail, s + 1, st0, st1, st2)        \
    AQ_STEP2(tail, s + 2, st1, st2, st0)        \
  } else if constexpr (!kSplitBar) {            \
    AQ_STEP(tail, s, st3, st0)                  \
    AQ_STEP(tail, s + 1, st0, st1)              \
    AQ_STEP(tail, s + 2, st1, st2)              \
    AQ_STEP(tail, s + 3, st2, st3)              \
  } else {                                      \
    AQ_STEP2(tail, s, st3, st0, st1)            \
    AQ_STEP2(tail, s + 1, st0, st1, st2)        \
    AQ_STEP2(tail, s + 2, st1, st2, st3)        \
    AQ_STEP2(tail, s + 3, st2, st3, st0)        \
  }
  // The epilogue's s values (BN <= 256: one per thread) are requested now and
  // kept raw in a register, so that their latency hides under the main loop;
  // nothing waits for them before the epilogue.
  // Every thread loads (clamped index, no branch: a load under a branch would
  // be waited for where the branch joins).
  uint16_t s_raw = 0;
  if constexpr (MODE != MODE_RAW) s_raw = B.s[min(n0 + min(tid, BN - 1), B.N - 1)];
  issue(0, st0);                         // slices 0 .. NST - 2 ahead of the loop
  if constexpr (NST > 2) issue(1, st1);
  if constexpr (NST > 3) issue(2, st2);
  bf16x8 f0a[TM], f0b[TN];               // first fragments of the next slice (split barrier)
  if constexpr (kSplitBar) {
    wait_vmcnt<(NST - 2) * LPS>();
    ring_barrier();
    frags(st0, 0, f0a, f0b);
  }
  for (int s = 0; s < nkp - NST; s += NST) {
    AQ_GROUP(std::false_type{}, s)
  }
  // t is read from the last group on (rank chunks riding on the ring, then the
  // epilogue): with the rank-r pass in this launch, wait for its workgroups.
  if (MODE != MODE_RAW && addu && a.tgrid > 0) {
    // Bounded: the rank-r workgroups were dispatched before every main one and
    // need no other workgroup to finish, so the count arrives (a wait that
    // reaches the bound all the same goes on and sets the flag word that
    // aq_workspace_check reports).  The workgroup barrier after it orders
    // every wave's reads of t behind the acquire.
    if (tid == 0) handoff_wait(a.sync, a.hw, (int)blockIdx.x & 7, handoff_poll(a.sync));
    ring_barrier();
  }
  // Every K range holds at least one slice (K >= 1), so nkp >= NST.  The last
  // group runs unconditionally: a branch around it would put a join between
  // the last MFMAs and the epilogue's first reads of their results.
  AQ_GROUP(std::true_type{}, nkp - NST)
#undef AQ_GROUP
#undef AQ_STEP2
#undef AQ_STEP
  __builtin_amdgcn_s_waitcnt(0);         // drain the (out-of-range) tail loads

  // ---- epilogue.  MFMA 32x32 output layout with W as the A operand: lane
  // holds output row m = mbase + lane % 32 and output columns n = nbase +
  // 8 (v / 4) + 4 (lane / 32) + (v % 4), v = 0..15.
  // First acc *= s, once per accumulator.  The rank-r term w = t U^T is one
  // more contraction, over r instead of K, that adds straight into acc: rank
  // chunk c < NST - 1 sits in stage c laid out like a K slice (it came with the
  // tail of the ring), so it is multiplied like one more K slice, with the
  // same fragment reads and MFMAs.  Chunks that did not fit in the ring, and U
  // rows that are not 16-byte aligned, are read from global memory per 32-row
  // round into 16 fresh accumulators that are added at the end.  Then, one
  // 32-row block of each wave row per round, y is written: fp32 partials
  // directly, bf16 through LDS (8 bytes per lane and column group).  The
  // rank-r pass (MODE_RAW) writes acc itself (no s, no w).
  constexpr int OP = BN + 8;                     // staging row pitch (bank spread, 16-byte rows)
  // Output staging: wave row 0's 32 rows in ost0, wave row 1's in ost1 (the
  // last stage holds both when it can, else the last two stages); with NW wave
  // rows, row w's in the last stage at 32 w rows.
  static_assert(32 * OP <= STAGE && ESLOTS >= 1, "staging and one rank chunk must fit");
  static_assert(WGM == 2 || WGM * 32 * OP <= STAGE, "four wave rows stage in one LDS stage");
  uint16_t *const slast = NST == 2 ? st1 : (NST == 3 ? st2 : st3);
  uint16_t *const sprev = NST == 2 ? st0 : (NST == 3 ? st1 : st2);
  uint16_t *const ost0 = ESLOTS == NST - 1 ? slast : sprev;
  uint16_t *const ost1 = ESLOTS == NST - 1 ? slast + 32 * OP : slast;
  const bool fp32_out = MODE == MODE_PART || (MODE == MODE_RAW && a.part);
  // fp32 rows of 4 columns as one 16-byte store where every row and block
  // start is 16-byte aligned
  const bool part_vec = ((a.ldp | B.col) & 3) == 0;
  const int nst = min(BN, B.Nst - n0);
  if (MODE != MODE_RAW)
    if (tid < BN) s_lds[tid] = n0 + tid < B.N ? bf2f(s_raw) : 0.f;
  __syncthreads();                       // s_lds, and every wave's last loads, are in
  if constexpr (SELF) {
    // This wave's block of t, rounded to bf16, goes where the rank chunks'
    // t rows sit (chunk c = ranks BK c .. in stage c, x rows, same swizzle);
    // U came with the ring.  Lane: row wm * WM + 32 i + l32, ranks
    // wn * RT / WGN + 32 jt + 8 g + 4 lhi + (0..3).
    if (addu) {
#pragma unroll
      for (int jt = 0; jt < TNT; ++jt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int j0 = wn * (RT / WGN) + jt * 32 + 8 * g, c = j0 / BK;
          if (c >= nchunk) continue;
          uint16_t *const stc = c == 0 ? st0 : st1;
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const int R = wm * WM + i * 32 + l32;
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            const bf16x4 h = {(__bf16)acct[i][jt][4 * g + 0], (__bf16)acct[i][jt][4 * g + 1],
                              (__bf16)acct[i][jt][4 * g + 2], (__bf16)acct[i][jt][4 * g + 3]};
            *reinterpret_cast<uint2 *>(stc + R * BK + 8 * (((j0 % BK) / 8) ^ sw(R)) + 4 * lhi) =
                __builtin_bit_cast(uint2, h);
          }
        }
    }
    __syncthreads();
  }

  if constexpr (MODE != MODE_RAW) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 sc = *reinterpret_cast<const float4 *>(s_lds + wn * WN + j * 32 + 8 * g + 4 * lhi);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          acc[i][j][4 * g + 0] *= sc.x;
          acc[i][j][4 * g + 1] *= sc.y;
          acc[i][j][4 * g + 2] *= sc.z;
          acc[i][j][4 * g + 3] *= sc.w;
        }
      }
  }
  // Rank chunks in the ring (16-byte aligned U rows): k-steps past r16 hold
  // zeros and are skipped.
  const bool ring_rank = addu && B.ufast;
  if (ring_rank) {
#pragma unroll
    for (int c = 0; c < ESLOTS; ++c) {
      if (c >= nech) break;
      const uint16_t *stc = c == 0 ? st0 : (c == 1 ? st1 : st2);
      const int kmax = min(KK, (r16 - BK * (c - part_of(c) * nchunk1)) / 16);
      bf16x8 fa[2][TM], fb[2][TN];
      frags(stc, 0, fa[0], fb[0]);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk >= kmax) break;
        if (kk + 1 < KK) frags(stc, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kk & 1][j], fa[kk & 1][i], acc[i][j], 0, 0, 0);
      }
    }
  }
  // Rank chunks left for the per-round path.
  const int cfirst = ring_rank ? nech : 0;
  const bool wround = addu && cfirst < nchunk;

  // Per-round rank-r fragments (this lane's 8 ranks at column col): t from
  // stage c for chunks c < nech, else from global memory; U from global memory.
  auto tfrag_lds = [&](const uint16_t *stc, int i, int kk) __attribute__((always_inline)) {
    return as_bf16x8(*reinterpret_cast<const uint4 *>(stc + arow + i * 32 * BK + 8 * ((2 * kk + lhi) ^ swz)));
  };
  auto tfrag_glb = [&](int i, int pe, int col) __attribute__((always_inline)) {
    const int m = m0 + wm * WM + i * 32 + l32;
    return m < M && col < r16 ? as_bf16x8(ld16(tbase + pe * a.tstride + (size_t)m * a.ldt + B.tcol + col))
                              : zero_bf16x8();
  };
  auto ufrag_glb = [&](int j, int col) __attribute__((always_inline)) {
    const int n = n0 + wn * WN + j * 32 + l32;
    return n < B.N ? load_u8(B, n, col) : zero_bf16x8();
  };

  // Column blocks per round of the per-round rank-r path: every block's MFMA
  // chain at once where the registers allow, else two at a time.
  constexpr int JH = (gemm_occupancy<BM, BN, BK, NST, RT>() == 1 && TM * TN <= 8) ? TN : (TN >= 2 ? 2 : 1);
  // bf16 output: each wave stages its 32 x WN block of a round in LDS and
  // stores it itself as 16-byte row pieces, one round late: the staged block
  // of round i - 1 is read back before round i is computed (LDS operations of
  // one wave complete in order, so round i's writes land after those reads),
  // and stored after round i's writes, so no wait sits between an LDS access
  // and its use, and no workgroup barrier is needed.
  constexpr int NSC = WN / 16;                     // 16-byte pieces per lane and round
  uint16_t *const ost = WGM == 2 ? (wm ? ost1 : ost0) : slast + wm * 32 * OP;
  uint4 pend[NSC];
  auto stage_read = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NSC; ++q) {
      const int c = lane + 64 * q, rl = c / (WN / 8), nc = wn * WN + (c - rl * (WN / 8)) * 8;
      pend[q] = *reinterpret_cast<const uint4 *>(ost + rl * OP + nc);
    }
  };
  auto stage_store = [&](int i) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NSC; ++q) {
      const int c = lane + 64 * q, rl = c / (WN / 8), nc = wn * WN + (c - rl * (WN / 8)) * 8;
      const int mr = m0 + wm * WM + i * 32 + rl;
      if (mr >= M || nc >= nst) continue;
      uint16_t *dst = a.y + (MODE == MODE_RAW && a.tsplit ? (size_t)p * a.tstride : 0) + (size_t)mr * a.ldy + B.col + n0 + nc;
      if (a.coherent) {
        // device-coherent 4-byte stores (the reader may sit on another XCD)
        unsigned *d4 = reinterpret_cast<unsigned *>(dst);
        __hip_atomic_store(d4 + 0, pend[q].x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(d4 + 1, pend[q].y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(d4 + 2, pend[q].z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(d4 + 3, pend[q].w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else if (a.vec_store && nc + 8 <= nst) {
        *reinterpret_cast<uint4 *>(dst) = pend[q];
      } else {
        const uint32_t wv[4] = {pend[q].x, pend[q].y, pend[q].z, pend[q].w};
        for (int e = 0; e < 8 && nc + e < nst; ++e) dst[e] = (uint16_t)(wv[e >> 1] >> (16 * (e & 1)));
      }
    }
  };
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + wm * WM + i * 32 + l32;
    if (!fp32_out && i > 0) {
      stage_read();
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j0 = 0; j0 < TN; j0 += JH) {
      f32x16 w[JH];
#pragma unroll
      for (int q = 0; q < JH; ++q)
#pragma unroll
        for (int v = 0; v < 16; ++v) w[q][v] = 0.f;
      if (wround) {
        for (int c = cfirst; c < nchunk; ++c) {
          const int pe = part_of(c), cc = c - pe * nchunk1;
          const int kmax = min(KK, (r16 - BK * cc) / 16);
          const uint16_t *stc = c == 0 ? st0 : (c == 1 ? st1 : st2);
          for (int kk = 0; kk < kmax; ++kk) {
            const int col = BK * cc + 16 * kk + 8 * lhi;
            const bf16x8 tb = c < nech ? tfrag_lds(stc, i, kk) : tfrag_glb(i, pe, col);
#pragma unroll
            for (int q = 0; q < JH; ++q)
              w[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ufrag_glb(j0 + q, col), tb, w[q], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < JH; ++q) {
        const int j = j0 + q;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int nl = wn * WN + j * 32 + 8 * g + 4 * lhi;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = acc[i][j][4 * g + e] + w[q][4 * g + e];
          if (fp32_out) {
            if (m < M) {
              float *dst = a.part + ((size_t)p * M + m) * a.ldp + B.col + n0 + nl;
              if (part_vec && nl + 4 <= nst) {
                *reinterpret_cast<float4 *>(dst) = make_float4(o[0], o[1], o[2], o[3]);
              } else {
                for (int e = 0; e < 4 && nl + e < nst; ++e) dst[e] = o[e];
              }
            }
          } else {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            const bf16x4 h = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
            *reinterpret_cast<uint2 *>(ost + l32 * OP + nl) = __builtin_bit_cast(uint2, h);
          }
        }
      }
    }
    if (!fp32_out && i > 0) stage_store(i - 1);
  }
  if (!fp32_out) {
    stage_read();
    stage_store(TM - 1);
  }
}

// Rank-r pass tile shape run inside a main-pass launch: 64 x 64 (128 x 128
// with eight waves) over 64-wide K slices, in as many stages as the main
// shape has (its stages fit in the main shape's); ok is false where the main
// shape has none.  (Tiles as tall as the main tile were tried: they take
// nearly as long as a main tile, which then waits for t.)
template <int BM, int BN, int BK, int NST, int NW>
struct TPass {
  static constexpr bool ok = (NW == 8 && BM == 256 && BN == 256 && BK == 32 && NST == 4) ||
                             (NW == 4 && ((BM == 256 && BN == 128) || (BM == 128 && (BN == 128 || BN == 96) && NST == 4) ||
                                          (BM == 64 && BN == 64 && BK == 64)));
  static constexpr int tBM = NW == 8 ? 128 : 64, tBN = tBM, tBK = 64, tNST = NST;
};

// The main pass (MODE_RECON / MODE_PART) or the rank-r pass (MODE_RAW), one
// tile (and K range) per workgroup.  With tgrid > 0 the first tgrid workgroups
// run the rank-r pass tiles described by tp instead (over the same K ranges as
// the main pass under a K split).
template <int BM, int BN, int BK, int NST, int MODE, int NW>
__global__ __launch_bounds__(64 * NW, (gemm_occupancy<BM, BN, BK, NST, MODE == MODE_SELF ? 64 : 0>())) void k_gemm_bf16(
    const PfArgs a, const PfArgs tp) {
  constexpr int STAGE = (BM + BN + (MODE == MODE_SELF ? 64 : 0)) * BK;
  // Each stage is its own LDS object; unused ones are a token size.
  __shared__ __attribute__((aligned(1024))) uint16_t st0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t st1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t st2[NST > 2 ? STAGE : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t st3[NST > 3 ? STAGE : 8];
  __shared__ float s_lds[BN];
  using T = TPass<BM, BN, BK, NST, NW>;
  if constexpr (MODE != MODE_RAW && MODE != MODE_SELF && T::ok) {
    static_assert((T::tBM + T::tBN) * T::tBK <= STAGE && T::tNST <= NST, "rank-r stages must fit");
    if ((int)blockIdx.x < a.tgrid) {
      const int u = xcd_contiguous_tile(blockIdx.x, tp.ntiles * tp.S);
      if (u >= 0) gemm_tile<T::tBM, T::tBN, T::tBK, T::tNST, MODE_RAW, NW>(tp, u, st0, st1, st2, st3, s_lds);
      // every wave's coherent t stores are complete, then one arrival that
      // releases them at agent scope (the readers may sit on other XCDs)
      __builtin_amdgcn_s_waitcnt(0);
      ring_barrier();
      if (threadIdx.x == 0) handoff_arrive(a.sync);
      return;
    }
  }
  const int unit = xcd_contiguous_tile((int)blockIdx.x - a.tgrid, a.ntiles * a.S);
  if (unit < 0) return;
  gemm_tile<BM, BN, BK, NST, MODE, NW>(a, unit, st0, st1, st2, st3, s_lds);
}

// y = bf16(sum of the S fp32 partials, in split order); also folds the split
// partials of the rank-r pass into the bf16 t buffer.
__global__ __launch_bounds__(256) void k_prefill_reduce(const float *part, int S, int M, int ldp,
                                                        int ncols, uint16_t *y, int ldy) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)M * ncols) return;
  const int m = (int)(i / ncols), n = (int)(i - (long)m * ncols);
  // Eight partials requested at once, then added in split order: one memory
  // round trip per eight splits instead of one per split.
  float sum = 0.f;
  for (int q0 = 0; q0 < S; q0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = q0 + u < S ? part[((size_t)(q0 + u) * M + m) * ldp + n] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (q0 + u < S) sum += v[u];
  }
  y[(size_t)m * ldy + n] = f2bf(sum);
}

// ---------------------------------------------------------------- host side

namespace {

struct TileCfg {
  int BM, BN, BK, NST, S, NW;
};

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

// Compiled main-pass tile shapes: BM x BN output, BK-wide K slices through NST
// LDS stages; workgroups resident per CU follow from the LDS ring.
struct Cand {
  int BM, BN, BK, NST, NW;
};
static const Cand kCands[] = {{128, 128, 64, 4, 4}, {256, 128, 32, 3, 4}, {256, 128, 64, 3, 4}, {256, 256, 32, 4, 4},
                               {256, 256, 64, 2, 4}, {256, 256, 32, 4, 8}, {256, 256, 64, 2, 8}, {128, 256, 64, 3, 4},
                               {128, 128, 64, 2, 4}, {128, 256, 32, 3, 4}, {128, 128, 32, 4, 4}, {64, 64, 64, 4, 4},
                               {64, 128, 64, 4, 4},  {128, 64, 64, 4, 4},  {128, 128, 64, 3, 4},  {128, 96, 64, 4, 4},
                               {128, 96, 64, 3, 4}};

// Main-pass tile and K split.  The tile comes from a cost model fitted to
// sweeps over the Gemma-3-1B and large-decoder prefill shapes on MI355X: a
// dispatch takes ceil(tiles / slots) rounds on the CUs, and a tile takes
// (K / 32) x (time per 32-wide K slice) + (prologue and epilogue).  Measured
// per-slice times (us): 256 x 256 with eight waves 0.85 (one per CU); 256 x 128
// with 32-wide slices 0.89 when two share a CU, 0.71 alone; 256 x 128 with
// 64-wide slices 0.52 (one per CU); 128 x 128 0.35 (one per CU).
// * up to 16 tiles of 128 x 128, or K <= 2048 and at most one round of 64 x 64
//   tiles (the Gemma-3-1B QKV and o projections at M = 512): 64 x 64 tiles,
//   four stages, no K split (they cover four times as many CUs, and a tile's
//   K loop, bound by load latency there, runs a quarter of the bytes);
// * K <= 2048 and at most one round of 128 x 128 tiles: where they cover
//   more than half of the CUs and r <= 64 (the Gemma-3-1B QKV and o
//   projections at M = 2048), tiles with 64-wide slices that compute their own
//   rows of t, 128 x 96 where those still fit in one round (o), else 128 x 128
//   in three stages (QKV); otherwise 128 x 128 with 32-wide slices, two
//   workgroups per CU, so that the rank-r pass tiles fit beside them in the
//   same launch (fewer tiles: M = 1024 measured faster so);
// * else, for K >= 8192 where 256 x 128 tiles K-split in S >= 2 ranges of
//   >= 4096 fill at least 80% of the CUs in one round, those;
// * else the cheapest of the four by the model; 128 x 128 splits long K
//   (>= 4096) when its tiles cover at most half of the CUs (ranges >= 2048),
//   else becomes 128 x 96 (four waves in a column) where those still fit in
//   one round and cover more CUs (Gemma-3-1B down at M = 2048: 192 tiles
//   instead of 144, 61 us instead of 70).
struct Est {
  TileCfg tc;
  int slots;
  double step_us, step_alone_us, epi_us;
};
static const Est kEst[] = {{{256, 256, 32, 4, 1, 8}, kNumCU, 0.85, 0.85, 5.0},
                           {{256, 128, 32, 3, 1, 4}, 2 * kNumCU, 0.89, 0.71, 5.0},
                           {{256, 128, 64, 3, 1, 4}, kNumCU, 0.52, 0.52, 5.0},
                           {{128, 128, 64, 4, 1, 4}, kNumCU, 0.35, 0.35, 3.0}};

TileCfg choose(const Recon &rq) {
  const int t128 = count_tiles(rq, 128, 128, false);
  int rmax = 0;
  for (int b = 0; b < rq.nblk; ++b) rmax = rq.blk[b].r > rmax ? (int)rq.blk[b].r : rmax;
  const bool own_t = rmax <= 64 && debug_knob(AQ_DBG_PREFILL_SELF, 1) != 0;
  TileCfg tc = {128, 128, 64, 4, 1, 4};
  if (t128 <= 16 || (rq.K <= 2048 && count_tiles(rq, 64, 64, false) <= kNumCU)) {
    tc = {64, 64, 64, 4, 1, 4};
  } else if (rq.K <= 2048 && t128 <= kNumCU) {
    if (own_t && 2 * t128 > kNumCU)
      tc = count_tiles(rq, 128, 96, false) <= kNumCU ? TileCfg{128, 96, 64, 4, 1, 4} : TileCfg{128, 128, 64, 3, 1, 4};
    else
      tc = {128, 128, 32, 4, 1, 4};
  } else {
    double best = 1e30;
    for (const Est &e : kEst) {
      const int t = count_tiles(rq, e.tc.BM, e.tc.BN, false);
      const double step = t <= kNumCU ? e.step_alone_us : e.step_us;
      const double cost = (double)((t + e.slots - 1) / e.slots) * ((double)rq.K / 32.0 * step + e.epi_us);
      if (cost < best) best = cost, tc = e.tc;
    }
    // Long K (>= 8192) with few 256 x 128 tiles: those tiles, K split so that
    // the units fill at least 80% of the CUs in one round (ranges >= 4096):
    // the large-decoder down at M = 512 (K = 21504, 84 tiles, S = 3) 146 us
    // against 178 for one round of 240 unsplit 128 x 96 tiles (weights not in
    // the Infinity Cache).
    const int t256 = count_tiles(rq, 256, 128, false);
    const int s256 = t256 > 0 ? kNumCU / t256 : 0, s256max = (int)(rq.K / 4096);
    const int sl = s256 < s256max ? s256 : s256max;
    if (rq.K >= 8192 && sl >= 2 && 10 * t256 * sl >= 8 * kNumCU) {
      tc = {256, 128, 64, 3, sl, 4};
    } else if (tc.BM == 128 && rq.K >= 4096 && 2 * t128 <= kNumCU) {
      const int S = kNumCU / t128, smax = (int)(rq.K / 2048);
      tc.S = S < smax ? S : smax;
    } else if (tc.BM == 128 && tc.BN == 128 && t128 < kNumCU && count_tiles(rq, 128, 96, false) <= kNumCU) {
      tc = {128, 96, 64, 4, 1, 4};
    }
  }
  // Plan overrides (tests, aq_debug_force_plan): BM/BN/BK/NST/W pick a compiled
  // shape, S the K split.
  const int bm = debug_knob(AQ_DBG_PREFILL_BM, 0), bn = debug_knob(AQ_DBG_PREFILL_BN, 0);
  const int bk = debug_knob(AQ_DBG_PREFILL_BK, 0), ns = debug_knob(AQ_DBG_PREFILL_NST, 0);
  const int nw = debug_knob(AQ_DBG_PREFILL_W, 4);
  for (const Cand &c : kCands)
    if (c.BM == bm && c.BN == bn && (bk == 0 || c.BK == bk) && (ns == 0 || c.NST == ns) && c.NW == nw) {
      tc.BM = c.BM, tc.BN = c.BN, tc.BK = c.BK, tc.NST = c.NST, tc.NW = c.NW;
      break;
    }
  const int so = debug_knob(AQ_DBG_PREFILL_S, 0);
  if (so >= 1) tc.S = so;
  return tc;
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
  pl->BK = tc.BK;
  pl->NST = tc.NST;
  pl->S = tc.S;
  pl->NW = tc.NW;
  pl->tBM = 64;
  pl->tBN = 64;
  pl->tS = 1;
  // The rank-r pass runs inside the main-pass launch (its tiles first, see
  // k_gemm_bf16) when the main pass has no K split, its tile shape has a
  // rank-r tile shape that fits its LDS stages (the shapes TPass lists), a
  // main tile is at least four rank-r tiles (so that t is ready before the
  // main tiles reach their epilogue, also with the rank-r pass's K unsplit),
  // and the rank-r tiles fit in the slots that the main pass's last round
  // leaves free (else they would push main tiles into another round): one
  // launch, its ramp and the fold of a K split less.
  const bool fusable =
      (tc.NW == 8 && tc.BM == 256 && tc.BN == 256 && tc.BK == 32 && tc.NST == 4) ||
      (tc.NW == 4 && ((tc.BM == 256 && tc.BN == 128) || (tc.BM == 128 && (tc.BN == 128 || tc.BN == 96) && tc.NST == 4) ||
                      (tc.BM == 64 && tc.BN == 64 && tc.BK == 64)));
  // Under a main-pass K split the rank-r tiles run over the same K ranges and
  // keep one t per range (each main unit adds its own range's rank term).
  // A main tile smaller than four rank-r tiles (64 x 64) takes about as long
  // as one: there the rank-r tiles split K into parts (kept apart, summed by
  // the main tiles' epilogue MFMAs) so that each runs at most half as many K
  // slices as a main tile and t is ready before the main tiles need it.
  const int to = debug_knob(AQ_DBG_TPASS_S, 0);
  pl->fuse = 0;
  pl->tparts = 1;
  // The tile shapes chosen for one round of few, latency-bound tiles with
  // K <= 2048 compute their own rows of t: the Vt rows of their block (r <= 64)
  // ride in every LDS stage as 64 more B rows, so t never goes through memory
  // and no tile waits for another; the extra MFMAs cost little where each K
  // slice waits for its loads anyway (with long K they do not: down at
  // M = 2048 took 79 us so against 61 with the rank-r pass).
  int rmax = 0;
  for (int b = 0; b < rq.nblk; ++b) rmax = rq.blk[b].r > rmax ? (int)rq.blk[b].r : rmax;
  const bool self_tile = tc.NW == 4 && ((tc.BM == 64 && tc.BN == 64 && tc.BK == 64 && tc.NST == 4) ||
                                         (tc.BM == 128 && tc.BN == 128 && tc.BK == 32 && tc.NST == 4) ||
                                         (tc.BM == 128 && tc.BN == 128 && tc.BK == 64 && tc.NST == 3) ||
                                         (tc.BM == 128 && tc.BN == 96 && tc.BK == 64 && tc.NST >= 3));
  pl->self = c > 0 && self_tile && tc.S == 1 && rq.K <= 2048 && rmax <= 64 && to <= 1 &&
             debug_knob(AQ_DBG_PREFILL_SELF, 1) != 0;
  if (c > 0 && !pl->self && fusable && to <= 1 && debug_knob(AQ_DBG_PREFILL_FUSE, 1) != 0) {
    const int tb = tc.NW == 8 ? 128 : 64;              // the shape TPass gives
    const int slots = kNumCU * ((tc.BM + tc.BN) * tc.BK * 2 * tc.NST <= 80 * 1024 ? 2 : 1);
    const int rem = count_tiles(rq, tc.BM, tc.BN, false) * tc.S % slots;
    const bool big = tc.BM * tc.BN >= 4 * tb * tb;
    int parts = 1;
    if (!big && tc.S == 1) {
      parts = 2 * 64 / tc.BK;
      const int po = debug_knob(AQ_DBG_TPASS_PARTS, 0);
      if (po >= 1) parts = po;
      const int pmax = (int)((rq.K + 127) / 128);        // parts of >= 128 K values
      parts = parts < pmax ? parts : pmax;
      parts = parts < 8 ? parts : 8;
      // the parts' offsets stay 32-bit
      if ((double)parts * (double)rq.M * c * 2 >= 2147483648.0) parts = 1;
    }
    const int tt = count_tiles(rq, tb, tb, true) * (tc.S > 1 ? tc.S : parts);
    if ((big || parts > 1) && rem > 0 && rem + tt <= slots) {
      pl->fuse = 1;
      pl->tparts = tc.S > 1 ? 1 : parts;
      pl->tBM = pl->tBN = tb;
    }
  }
  // Else a rank-r pass of its own: 64 x 64 tiles over t's columns.  For long K
  // (> 2048) K is split so that the workgroups cover the CUs with ranges of
  // >= 768 values and the fp32 partials are folded into the bf16 t buffer by
  // the reduce kernel; for shorter K the fold costs more than the split saves
  // (sweeps over the Gemma-3-1B prefill shapes on MI355X).
  if (!pl->fuse && !pl->self && c > 0 && rq.K > 2048) {
    const int tiles = count_tiles(rq, 64, 64, true);
    int S = (kNumCU + tiles - 1) / tiles;
    const int smax = rq.K / 768 > 1 ? (int)(rq.K / 768) : 1;
    pl->tS = S < smax ? S : smax;
  }
  if (to >= 1) pl->tS = to;
  size_t bytes = pl->self ? 0 : (size_t)rq.M * c * 2 * (pl->fuse ? (pl->S > pl->tparts ? pl->S : pl->tparts) : 1);
  bytes = (bytes + 255) / 256 * 256;
  pl->tpart_off = bytes;
  if (pl->tS > 1) bytes += ((size_t)pl->tS * rq.M * c * 4 + 255) / 256 * 256;
  pl->part_off = bytes;
  if (pl->S > 1) bytes += (size_t)pl->S * rq.M * rq.Ntot * 4;
  pl->ws_bytes = bytes > 0 ? kWsReserved + bytes : 0;
}

template <int MODE>
static bool launch_tile(int BM, int BN, int BK, int NST, int NW, const PfArgs &a, const PfArgs &tp, int grid,
                        hipStream_t st) {
#define AQ_TILE(bm, bn, bk, ns, nw)                                                                   \
  if (BM == bm && BN == bn && BK == bk && NST == ns && NW == nw) {                                   \
    hipLaunchKernelGGL((k_gemm_bf16<bm, bn, bk, ns, MODE, nw>), dim3(grid), dim3(64 * nw), 0, st, a, tp); \
    return true;                                                                                      \
  }
  if constexpr (MODE == MODE_RAW) {
    AQ_TILE(64, 64, 64, 4, 4)
  } else if constexpr (MODE == MODE_SELF) {
    AQ_TILE(64, 64, 64, 4, 4)
    AQ_TILE(128, 128, 32, 4, 4)
    AQ_TILE(128, 128, 64, 3, 4)
    AQ_TILE(128, 96, 64, 4, 4)
    AQ_TILE(128, 96, 64, 3, 4)
  } else {
    AQ_TILE(256, 256, 32, 4, 4)
    AQ_TILE(256, 256, 64, 2, 4)
    AQ_TILE(256, 256, 32, 4, 8)
    AQ_TILE(256, 256, 64, 2, 8)
    AQ_TILE(256, 128, 64, 3, 4)
    AQ_TILE(128, 256, 64, 3, 4)
    AQ_TILE(128, 128, 64, 2, 4)
    AQ_TILE(128, 128, 64, 3, 4)
    AQ_TILE(128, 96, 64, 4, 4)
    AQ_TILE(128, 96, 64, 3, 4)
    AQ_TILE(128, 128, 64, 4, 4)
    AQ_TILE(256, 128, 32, 3, 4)
    AQ_TILE(128, 256, 32, 3, 4)
    AQ_TILE(128, 128, 32, 4, 4)
    AQ_TILE(64, 64, 64, 4, 4)
    AQ_TILE(64, 128, 64, 4, 4)
    AQ_TILE(128, 64, 64, 4, 4)
  }
#undef AQ_TILE
  return false;
}

static void tile_prep(PfArgs &a, int BM, int BN) {
  a.ntm = (a.M + BM - 1) / BM;
  int t0 = 0;
  for (int b = 0; b < a.nblk; ++b) {
    a.b[b].tile0 = t0;
    a.b[b].ntn = (a.b[b].Nst + BN - 1) / BN;
    t0 += a.b[b].ntn * a.ntm;
  }
  a.ntiles = t0;
}

static hipError_t run(PfArgs &a, const PfArgs &tp, int BM, int BN, int BK, int NST, int NW, int mode, hipStream_t st) {
  tile_prep(a, BM, BN);
  if (a.ntiles == 0) return hipSuccess;
  const int units = a.ntiles * a.S;
  const int grid = a.tgrid + 8 * ((units + 7) / 8);
  bool ok = false;
  switch (mode) {
    case MODE_RECON: ok = launch_tile<MODE_RECON>(BM, BN, BK, NST, NW, a, tp, grid, st); break;
    case MODE_PART: ok = launch_tile<MODE_PART>(BM, BN, BK, NST, NW, a, tp, grid, st); break;
    case MODE_SELF: ok = launch_tile<MODE_SELF>(BM, BN, BK, NST, NW, a, tp, grid, st); break;
    default: ok = launch_tile<MODE_RAW>(BM, BN, BK, NST, NW, a, tp, grid, st); break;
  }
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_prefill(const Recon &rq, const PrefillPlan &pl, void *ws, hipStream_t st) {
  char *scratch = ws ? (char *)ws + kWsReserved : nullptr;
  uint16_t *tbuf = pl.ldt > 0 ? (uint16_t *)scratch : nullptr;
  PfArgs a = {};
  a.tparts = 1;
  a.x = (const uint16_t *)rq.x;
  a.ldx = (int)rq.ldx;
  a.M = (int)rq.M;
  a.K = (int)rq.K;

  // pass 1: fp32 partials of t = x Vt^T for every block with r > 0 (columns
  // padded to 16 with zeros), then folded into the bf16 t buffer.
  PfArgs t = a;
  if (pl.ldt > 0 && !pl.self) {
    t.S = pl.tS;
    int tkc = (int)((rq.K + pl.tS - 1) / pl.tS);
    t.kchunk = (tkc + 63) / 64 * 64;
    t.S = (int)((rq.K + t.kchunk - 1) / t.kchunk);
    t.part = (float *)(scratch + pl.tpart_off);
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
    if (t.S == 1) {                  // no K split: bf16 t straight from the tile
      t.part = nullptr;
      t.y = tbuf;
      t.ldy = pl.ldt;
      t.vec_store = 1;
    }
    if (pl.fuse) {
      // run by the first workgroups of the main-pass launch (below), over the
      // main pass's K ranges (or in tparts K ranges of its own), one bf16 t
      // per range
      const int nr = pl.S > 1 ? pl.S : pl.tparts, kq = pl.S > 1 ? pl.BK : 64;
      const int kc = (int)((rq.K + nr - 1) / nr);
      t.kchunk = (kc + kq - 1) / kq * kq;
      t.S = (int)((rq.K + t.kchunk - 1) / t.kchunk);
      t.part = nullptr;
      t.y = tbuf;
      t.ldy = pl.ldt;
      t.vec_store = 1;
      t.tsplit = t.S > 1;
      t.tstride = (long)rq.M * pl.ldt;
      t.coherent = 1;
      tile_prep(t, pl.tBM, pl.tBN);
    }
    hipError_t e = pl.fuse ? hipSuccess : run(t, t, pl.tBM, pl.tBN, 64, 4, 4, MODE_RAW, st);
    if (e != hipSuccess) return e;
    if (!pl.fuse && t.S > 1) {
      const long n = (long)rq.M * pl.ldt;
      hipLaunchKernelGGL(k_prefill_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                         (const float *)t.part, t.S, (int)rq.M, pl.ldt, pl.ldt, tbuf, pl.ldt);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }

  // pass 2: y = s * (x W0^T) + t U^T
  a.y = (uint16_t *)rq.y;
  a.ldy = (int)rq.ldy;
  a.t = tbuf;
  a.ldt = pl.ldt;
  int kc = (int)((rq.K + pl.S - 1) / pl.S);
  a.kchunk = (kc + pl.BK - 1) / pl.BK * pl.BK;
  a.S = (int)((rq.K + a.kchunk - 1) / a.kchunk);
  a.nblk = rq.nblk;
  a.part = a.S > 1 ? (float *)(scratch + pl.part_off) : nullptr;
  a.ldp = (int)rq.Ntot;
  a.vec_store = ((uintptr_t)rq.y % 16 == 0) && (rq.ldy % 8 == 0);
  for (int b = 0; b < rq.nblk; ++b) {
    const Proj &P = rq.blk[b];
    PfBlk &d = a.b[b];
    d.W = (const uint16_t *)P.W0;
    d.s = (const uint16_t *)P.s;
    d.U = (const uint16_t *)P.U;
    d.Vt = (const uint16_t *)P.Vt;
    d.N = (int)P.N;
    d.Nst = (int)P.N;
    d.r = (int)P.r;
    d.col = (int)P.col;
    d.tcol = pl.tcol[b];
    d.ufast = (P.r % 8 == 0) && (((uintptr_t)P.U & 15) == 0);
    if (P.col % 8) a.vec_store = 0;
  }
  if (pl.fuse && t.ntiles > 0) {
    tile_prep(a, pl.BM, pl.BN);
    a.tgrid = 8 * ((t.ntiles * t.S + 7) / 8);
    a.sync = (unsigned *)ws;
    a.tsplit = a.S > 1;
    a.tparts = a.S > 1 ? 1 : t.S;
    a.tstride = (long)rq.M * pl.ldt;
    // The main units that wait: those of blocks with a rank-r term, every K
    // range with one t per range, else the first (it adds the rank term).
    // Every rank-r workgroup arrives (the grid is rounded up to whole XCD
    // rounds; the padding workgroups count themselves too).
    const int S = a.S;
    const bool tsplit = a.tsplit;
    auto waits = [&](int u) {
      const int tile = u / S, p = u - tile * S;
      int bi = 0;
      if (a.nblk > 1 && tile >= a.b[1].tile0) bi = 1;
      if (a.nblk > 2 && tile >= a.b[2].tile0) bi = 2;
      return a.b[bi].r > 0 && (S == 1 || tsplit || p == 0);
    };
    int nwait = 0;
    for (int u = 0; u < a.ntiles * S; ++u) nwait += waits(u) ? 1 : 0;
    if (nwait == 0) a.tgrid = 0;
    else handoff_counts(a.ntiles * S, a.tgrid, waits, &a.hw);
  }
  const int mode = pl.self ? MODE_SELF : (a.S > 1 ? MODE_PART : MODE_RECON);
  hipError_t e = run(a, t, pl.BM, pl.BN, pl.BK, pl.NST, pl.NW, mode, st);
  if (e != hipSuccess || a.S == 1) return e;
  const long n = (long)rq.M * rq.Ntot;
  hipLaunchKernelGGL(k_prefill_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     (const float *)a.part, a.S, (int)rq.M, (int)rq.Ntot, (int)rq.Ntot, a.y,
                     (int)rq.ldy);
  return hipGetLastError();
}

}  // namespace aq
