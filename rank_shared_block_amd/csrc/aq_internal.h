// Internal interface between the C-ABI front end (aq_api.hip) and the kernels.
// Host-side plan structures: everything here is validated before it is built.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/aq.h"

namespace aq {

constexpr int kMaxBlocks = 3;     // Q/K/V
constexpr int kNumCU = 256;       // MI355X: 256 CUs in 8 XCDs of 32
constexpr int kNumXCD = 8;
constexpr int kDecodeMaxM = 64;   // largest batch served by the streaming kernel

// Workspace layout shared by every call: the first kWsReserved bytes hold the
// arrival counters (zero between calls; the prefill launch that also runs the
// rank-r pass uses the first two); per-call scratch (partials, the
// rank-r activation buffer, FP4 partial maxima) starts after them, so calls of
// different kinds can share one workspace.
constexpr size_t kWsReserved = 65536;
constexpr int kMaxCounterTiles = (int)(kWsReserved / 4);

// Plan overrides set through aq_debug_force_plan (thread-local, for tests that
// force one kernel variant).  Returns dflt while the knob is unset, so without
// those calls a plan depends only on the call's arguments.
int debug_knob(aq_debug_knob k, int dflt);

// Hand-off words in the reserved workspace region (handoff.h): [0] arrivals of
// the workgroups that compute t, [1] groups of waiters that have all passed,
// [2] flag set when a wait gave up (read and cleared by aq_workspace_check),
// [16 + 16 g] waiters of group g that have passed (g = 0..7, one 64-byte line
// each).  All zero between calls.
constexpr int kSyncArrive = 0, kSyncGroups = 1, kSyncFlag = 2;
constexpr int kSyncGroup0 = 16, kSyncGroupStride = 16, kHandoffGroups = 8;
constexpr int kSyncWords = kSyncGroup0 + kSyncGroupStride * kHandoffGroups;
constexpr int kHandoffSpin = 1 << 22;   // polls before a wait gives up

// One projection of a (possibly fused) dispatch, host view.
struct Proj {
  int64_t N, r;
  const void *W0, *s, *U, *Vt;
  int64_t col;   // first output column of this block inside y
};

// A validated reconstruction request.
struct Recon {
  aq_dtype dt;
  int64_t M, K, ldx, ldy, Ntot;
  const void *x;
  void *y;
  int nblk;
  Proj blk[kMaxBlocks];
};

// ---- decode (streaming, M <= kDecodeMaxM, bf16) ---------------------------
constexpr int kMaxSegs = 2 * kMaxBlocks;   // split mode: W0 rows and Vt rows per block

struct DecodeSeg {
  int b;           // block
  int isVt;        // split mode: 1 for the block's Vt rows
  int tile0, ntile;
  int rows;        // rows per tile (W0 rows in fused mode; at most 16 x the tile's W0 groups)
};

struct DecodePlan {
  int MT;          // 16-token groups: 1, 2 or 4
  int NG;          // 16-row groups per workgroup
  int split;       // 0: fused (t per workgroup, one kernel); 1: partials + combine
  int S;           // K splits across workgroups (split mode only; 1 when fused)
  int WAVES;       // waves per workgroup: 4 or 8
  int kchunk;      // K elements per split (multiple of 128)
  int ntiles;      // row tiles over all segments
  int nseg;
  DecodeSeg seg[kMaxSegs];
  int vg[kMaxBlocks];                // fused: Vt groups per tile of each block
  int tcol[kMaxBlocks];              // split: column of block b's t in a partial row
  int Wp;                            // split: partial row width (sum N + sum r)
  size_t ws_bytes;                   // total workspace bytes (0 when fused)
};
bool plan_decode(const Recon &rq, DecodePlan *pl);
hipError_t launch_decode(const Recon &rq, const DecodePlan &pl, void *ws, hipStream_t st);

// ---- prefill (MFMA tiles, bf16) ---------------------------------------------
struct PrefillPlan {
  int ldt;                          // columns of the t buffer (sum of r rounded to 16)
  int tcol[kMaxBlocks];
  int BM, BN, BK, NST, S;           // output tile, K slice, LDS stages, K splits (main pass)
  int NW;                           // waves per workgroup (main pass)
  int tBM, tBN, tS;                 // output tile and K splits of the rank-r (t) pass
  int fuse;                         // rank-r pass inside the main-pass launch
  int tparts;                       // fused, main pass unsplit: t kept in this many K-range parts
  int self;                         // main tiles compute their own rows of t (no rank-r pass)
  size_t tpart_off;                 // byte offset of the t-pass partials in the scratch
  size_t part_off;                  // byte offset of the main-pass partials in the scratch
  size_t ws_bytes;                  // total workspace bytes (reserved region + t buffer)
};
void plan_prefill(const Recon &rq, PrefillPlan *pl);
hipError_t launch_prefill(const Recon &rq, const PrefillPlan &pl, void *ws, hipStream_t st);

// ---- per-element rebuild (M <= 16, r <= 64, bf16) -----------------------------
constexpr int kRebuildMaxM = 16, kRebuildMaxRank = 64;
struct RebuildPlan {
  int rows;                    // rows per tile (at most 16 NG)
  int NG;                      // 16-row groups per tile
  int RC;                      // 32-wide rank chunks (0 for rank 0)
  int S, kchunk;               // K ranges and their length (multiple of 32)
  int ntiles;
  int tile0[kMaxBlocks];
  size_t ws_bytes;             // 0 without a K split, else reserved region + fp32 partials
};
void plan_rebuild(const Recon &rq, RebuildPlan *pl);
hipError_t launch_rebuild(const Recon &rq, const RebuildPlan &pl, void *ws, hipStream_t st);

// ---- decomposition (band mean, least squares, randomized SVD; fp64) ----------
constexpr int kMaxBandLayers = 64;
constexpr int kDecompMaxL = 256;
struct DecompArgs {
  aq_dtype dt;
  int64_t N, K, r, l;
  int q;
  const void *W, *W0;
  const double *omega;
  double *s, *U, *Vt;
};
struct DecompPlan {
  int lj;                      // compiled width of the l side (32, 64, 80, 128, 256)
  int srm, kchunk;             // K ranges of R X; columns per range
  int srt, sgram;              // N ranges of R^T Q; ranges of the Gram sums
  long nchunk;                 // rows per N range
  int jac_wgs;                 // workgroups of the grid Jacobi (0: the one-workgroup LDS kernel)
  int jac_block;               // 1: the block Jacobi instead (jac_wgs workgroups, n padded to jac_n)
  int jac_n;
  int jac_spin, jac_extra;     // its barrier's poll bound; arrivals awaited beyond the grid's
  size_t o_y1, o_y2, o_z1, o_z2, o_zp, o_yp, o_gp, o_g, o_rinv, o_scr, o_jac, o_ctr, o_lam, o_wu, o_wv;   // byte offsets
};
size_t decompose_ws_bytes(int64_t N, int64_t K, int64_t r, int64_t l, DecompPlan *pl);
hipError_t launch_decompose(const DecompArgs &d, const DecompPlan &pl, void *ws, hipStream_t st);
hipError_t launch_band_mean(aq_dtype dt, int L, const void *const *W, int64_t n, void *out, hipStream_t st);

// ---- fp32 (any M) -------------------------------------------------------------
hipError_t launch_recon_f32(const Recon &rq, hipStream_t st);

// ---- materialise ----------------------------------------------------------------
hipError_t launch_materialize(aq_dtype dt, int64_t K, const Proj &p, void *w, int64_t ldw,
                              hipStream_t st);

// Many projections per launch (bf16, r <= 64): consecutive items that name the
// same W0 (and N, K) share each read of a W0 tile, up to kMatRunMax of them.
constexpr int kMatRunMax = 2, kMatBatchRuns = 24, kMatBatchOuts = 48, kMatBatchMaxRank = 64;
struct MatItem {
  int64_t N, K, r, ldw;
  const void *W0, *s, *U, *Vt;
  void *w;                     // W_eff (mode 0)
  uint8_t *packed = nullptr, *scales = nullptr;   // the FP4 weight (mode 2)
  float *gscale = nullptr;
};
// mode 0: W_eff stored; amax NULL, or n device words that receive each W_eff's
// largest magnitude as bf16 bits (zeroed here first).  mode 1: only those
// maxima (amax required, zeroed here first), nothing stored.  mode 2: W_eff
// encoded as block-16 FP4 (K % 16 == 0) with the global scale derived from
// amax (read, not zeroed: the maxima of a mode-1 launch).
hipError_t launch_materialize_batch(int n, const MatItem *items, unsigned *amax, hipStream_t st, int mode = 0);

// ---- FP4 pack -------------------------------------------------------------------
constexpr int kFp4AmaxBlocks = 1024;
hipError_t launch_fp4(int64_t N, int64_t K, const void *w, int64_t ldw, uint8_t *packed,
                      uint8_t *scales, float *gscale, void *ws, hipStream_t st);

// Many weights per launch: the pack of each weight as above, its global scale
// from amax (bf16 bits of its largest magnitude, e.g. from
// launch_materialize_batch) or, when amax is NULL, from a batched max pass into
// the workspace (fp4_batch_ws_bytes).
constexpr int kFp4BatchItems = 64;
struct Fp4Item {
  int64_t N, K, ldw;
  const void *w;
  uint8_t *packed, *scales;
  float *gscale;
};
size_t fp4_batch_ws_bytes(int n, bool have_amax);
hipError_t launch_fp4_batch(int n, const Fp4Item *items, const unsigned *amax, void *ws, hipStream_t st);

// ---- FP4 decode GEMV --------------------------------------------------------------
struct Fp4LinPlan {
  int NG, rows, ntiles, S, kchunk;  // 16-row groups and rows per tile, tiles, K splits, K per split
  size_t ws_bytes;                  // 0 without a K split, else reserved region + fp32 partials
};
void plan_fp4_linear(int64_t M, int64_t N, int64_t K, Fp4LinPlan *pl);
hipError_t launch_fp4_linear(int64_t M, int64_t N, int64_t K, const void *x, int64_t ldx, const uint8_t *packed,
                             const uint8_t *scales, const float *gscale, void *y, int64_t ldy,
                             const Fp4LinPlan &pl, void *ws, hipStream_t st);

}  // namespace aq
