// C-ABI front end: argument validation, kernel choice by batch size and dtype,
// launch on the caller's stream.  Nothing here allocates device memory and
// nothing synchronises; argument errors are reported before any HIP call.

#include <limits.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "aq_internal.h"

// Device memory of the allocation-free entry point (aq_recon_linear_noalloc):
// one array per GPU, loaded with the code object and held until the process
// ends.  On the host the name is only a stand-in, never a device address: host
// code looks up each device's address (scratch_of_current_device) and passes
// that to kernels.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local char g_err[512] = "";

// Plan overrides (aq_debug_force_plan): unset unless a test sets them.
constexpr int kUnset = INT_MIN;
struct Knobs {
  int v[AQ_DBG_COUNT];
  Knobs() {
    for (int &x : v) x = kUnset;
  }
};
thread_local Knobs g_knobs;

aq_status fail(aq_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

constexpr int64_t kMaxDim = int64_t(1) << 24;
constexpr int64_t kMaxK = (int64_t(1) << 22) - 1;    // 32-bit buffer offsets over 256-row tiles
constexpr int64_t kMaxM = int64_t(1) << 19;
constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;
constexpr int kMaxBatchItems = 1 << 16;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

size_t esize(aq_dtype dt) { return dt == AQ_BF16 ? 2 : 4; }

// Validates a recon request and fills `rq`.  `need_ptrs` is false for the
// workspace-size query (no data pointers are inspected then).
aq_status build_recon(aq_dtype dt, int64_t M, int64_t K, const void *x, int64_t ldx,
                      const aq_proj *p, int nproj, void *y, int64_t ldy, bool need_ptrs,
                      aq::Recon *rq) {
  if (dt != AQ_F32 && dt != AQ_BF16) return fail(AQ_ERR_INVALID_ARG, "dtype %d is not AQ_F32 or AQ_BF16", (int)dt);
  if (!p) return fail(AQ_ERR_INVALID_ARG, "projection descriptor pointer is NULL");
  if (M < 0) return fail(AQ_ERR_INVALID_ARG, "M = %lld is negative", (long long)M);
  if (K < 1) return fail(AQ_ERR_SHAPE, "K = %lld must be >= 1", (long long)K);
  if (K > kMaxK) return fail(AQ_ERR_UNSUPPORTED, "K = %lld exceeds 2^22 - 1", (long long)K);
  if (M > kMaxM) return fail(AQ_ERR_UNSUPPORTED, "M = %lld exceeds 2^19", (long long)M);
  const int64_t kdiv = dt == AQ_BF16 ? 8 : 4;
  if (K % kdiv) return fail(AQ_ERR_ALIGNMENT, "K = %lld must be a multiple of %lld for this dtype", (long long)K, (long long)kdiv);
  rq->dt = dt;
  rq->M = M;
  rq->K = K;
  rq->nblk = nproj;
  int64_t col = 0;
  for (int b = 0; b < nproj; ++b) {
    const aq_proj &P = p[b];
    if (P.N < 1) return fail(AQ_ERR_SHAPE, "projection %d: N = %lld must be >= 1", b, (long long)P.N);
    if (P.N > kMaxDim) return fail(AQ_ERR_UNSUPPORTED, "projection %d: N = %lld exceeds 2^24", b, (long long)P.N);
    if (P.N * K > kMaxElems) return fail(AQ_ERR_UNSUPPORTED, "projection %d: N*K exceeds 2^31-1 elements", b);
    if (P.r < 0) return fail(AQ_ERR_SHAPE, "projection %d: rank %lld is negative", b, (long long)P.r);
    if (P.r > AQ_MAX_RANK) return fail(AQ_ERR_UNSUPPORTED, "projection %d: rank %lld exceeds the supported maximum %d", b, (long long)P.r, AQ_MAX_RANK);
    if (need_ptrs) {
      if (!P.W0 || !P.s) return fail(AQ_ERR_INVALID_ARG, "projection %d: W0 or s is NULL", b);
      if (P.r > 0 && (!P.U || !P.Vt)) return fail(AQ_ERR_INVALID_ARG, "projection %d: rank %lld but U or Vt is NULL", b, (long long)P.r);
      if (!aligned(P.W0, 16)) return fail(AQ_ERR_ALIGNMENT, "projection %d: W0 is not 16-byte aligned", b);
      if (!aligned(P.s, esize(dt))) return fail(AQ_ERR_ALIGNMENT, "projection %d: s is not naturally aligned", b);
      if (P.r > 0 && !aligned(P.Vt, 16)) return fail(AQ_ERR_ALIGNMENT, "projection %d: Vt is not 16-byte aligned", b);
      if (P.r > 0 && !aligned(P.U, esize(dt))) return fail(AQ_ERR_ALIGNMENT, "projection %d: U is not naturally aligned", b);
    }
    rq->blk[b] = aq::Proj{P.N, P.r, P.W0, P.s, P.U, P.Vt, col};
    col += P.N;
  }
  rq->Ntot = col;
  if (M == 0) return AQ_OK;
  if (ldx < K) return fail(AQ_ERR_SHAPE, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
  if (ldx > kMaxK) return fail(AQ_ERR_UNSUPPORTED, "ldx = %lld exceeds 2^22 - 1", (long long)ldx);
  if (ldx % kdiv) return fail(AQ_ERR_ALIGNMENT, "ldx = %lld must be a multiple of %lld", (long long)ldx, (long long)kdiv);
  if (ldy < col) return fail(AQ_ERR_SHAPE, "ldy = %lld < total output columns %lld", (long long)ldy, (long long)col);
  if (M * ldx > kMaxElems || M * ldy > kMaxElems) return fail(AQ_ERR_UNSUPPORTED, "x or y exceeds 2^31-1 elements");
  if (need_ptrs) {
    if (!x || !y) return fail(AQ_ERR_INVALID_ARG, "x or y is NULL");
    if (!aligned(x, 16)) return fail(AQ_ERR_ALIGNMENT, "x is not 16-byte aligned");
    if (!aligned(y, esize(dt))) return fail(AQ_ERR_ALIGNMENT, "y is not naturally aligned");
  }
  rq->x = x;
  rq->ldx = ldx;
  rq->y = y;
  rq->ldy = ldy;
  return AQ_OK;
}

// Path choice: fp32 -> generic fp32 kernel; bf16 with M <= 64 and a rank the
// streaming kernel holds -> decode kernel; otherwise the tiled MFMA kernel.
enum Path { P_F32, P_DECODE, P_PREFILL };

struct Plan {
  Path path;
  aq::DecodePlan dec;
  aq::PrefillPlan pf;
  size_t ws;
};

void make_plan(const aq::Recon &rq, Plan *pl) {
  pl->ws = 0;
  if (rq.dt == AQ_F32) {
    pl->path = P_F32;
    return;
  }
  if (aq::plan_decode(rq, &pl->dec)) {
    pl->path = P_DECODE;
    pl->ws = pl->dec.ws_bytes;
    return;
  }
  pl->path = P_PREFILL;
  aq::plan_prefill(rq, &pl->pf);
  pl->ws = pl->pf.ws_bytes;
}

// Zeroes n words (the hand-off counters of the library's own scratch before a
// launch that uses them): a kernel rather than a memset, so that a
// caller may capture it in a HIP graph.
__global__ void k_clear_words(unsigned *p, int n, int keep) {
  for (int i = threadIdx.x; i < n; i += blockDim.x)
    if (i != keep) p[i] = 0u;
}

// `clear_counters`: the workspace is the library's own scratch, whose counters
// are zeroed before each launch that waits on them (a prefill launch with the
// rank-r tiles inside); its flag word is kept for aq_workspace_check.
aq_status recon(aq_dtype dt, int64_t M, int64_t K, const void *x, int64_t ldx, const aq_proj *p,
                int nproj, void *y, int64_t ldy, void *ws, size_t ws_bytes, void *stream,
                bool clear_counters = false) {
  aq::Recon rq;
  aq_status s = build_recon(dt, M, K, x, ldx, p, nproj, y, ldy, true, &rq);
  if (s != AQ_OK || M == 0) return s;
  Plan pl;
  make_plan(rq, &pl);
  if (clear_counters && pl.ws > ws_bytes)
    return fail(AQ_ERR_UNSUPPORTED,
                "this call needs %zu bytes of scratch; the allocation-free entry point holds at most %zu "
                "(use aq_recon_* with a workspace)",
                pl.ws, ws_bytes);
  if (clear_counters && pl.path == P_PREFILL && pl.pf.fuse) {
    hipLaunchKernelGGL(k_clear_words, dim3(1), dim3(64), 0, (hipStream_t)stream, (unsigned *)ws, aq::kSyncWords,
                       aq::kSyncFlag);
    const hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return fail(AQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e0));
  }
  if (pl.ws > 0) {
    if (!ws) return fail(AQ_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", pl.ws);
    if (ws_bytes < pl.ws) return fail(AQ_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", pl.ws, ws_bytes);
    if (!aligned(ws, 256)) return fail(AQ_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  }
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  switch (pl.path) {
    case P_F32: e = aq::launch_recon_f32(rq, st); break;
    case P_DECODE: e = aq::launch_decode(rq, pl.dec, ws, st); break;
    case P_PREFILL: e = aq::launch_prefill(rq, pl.pf, ws, st); break;
  }
  if (e != hipSuccess) return fail(AQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return AQ_OK;
}

// ---- the library's own scratch (aq_recon_linear_noalloc) -------------------
// Each device's address of `scratch`, looked up once with that device current.
constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on its first use).
aq_status scratch_of_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(AQ_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(AQ_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(AQ_ERR_HIP, "looking up the scratch array on device %d failed: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return AQ_OK;
}

}  // namespace

int aq::debug_knob(aq_debug_knob k, int dflt) {
  const int v = (k >= 0 && k < AQ_DBG_COUNT) ? g_knobs.v[k] : kUnset;
  return v == kUnset ? dflt : v;
}

extern "C" {

aq_status aq_recon_linear(aq_dtype dt, int64_t M, int64_t K, const void *x, int64_t ldx,
                          const aq_proj *p, void *y, int64_t ldy, void *ws, size_t ws_bytes,
                          void *stream) {
  return recon(dt, M, K, x, ldx, p, 1, y, ldy, ws, ws_bytes, stream);
}

aq_status aq_recon_qkv_fused(aq_dtype dt, int64_t M, int64_t K, const void *x, int64_t ldx,
                             const aq_proj p[3], void *y, int64_t ldy, void *ws,
                             size_t ws_bytes, void *stream) {
  return recon(dt, M, K, x, ldx, p, 3, y, ldy, ws, ws_bytes, stream);
}

aq_status aq_recon_gateup_fused(aq_dtype dt, int64_t M, int64_t K, const void *x,
                                int64_t ldx, const aq_proj p[2], void *y, int64_t ldy,
                                void *ws, size_t ws_bytes, void *stream) {
  return recon(dt, M, K, x, ldx, p, 2, y, ldy, ws, ws_bytes, stream);
}

// Checks shared by the per-element rebuild and its workspace query.
aq_status check_rebuild(aq_dtype dt, int64_t M, const aq_proj *p, int nproj) {
  if (dt != AQ_BF16) return fail(AQ_ERR_UNSUPPORTED, "the per-element rebuild takes bf16 only");
  for (int b = 0; b < nproj; ++b)
    if (p[b].r > aq::kRebuildMaxRank)
      return fail(AQ_ERR_UNSUPPORTED, "projection %d: rank %lld exceeds the per-element rebuild's limit %d", b,
                  (long long)p[b].r, aq::kRebuildMaxRank);
  if (M > aq::kRebuildMaxM)
    return fail(AQ_ERR_UNSUPPORTED, "M = %lld: the per-element rebuild takes at most %d tokens", (long long)M,
                aq::kRebuildMaxM);
  return AQ_OK;
}

aq_status aq_rebuild_linear(aq_dtype dt, int64_t M, int64_t K, const void *x, int64_t ldx, const aq_proj *p,
                            int nproj, void *y, int64_t ldy, void *ws, size_t ws_bytes, void *stream) {
  if (nproj < 1 || nproj > aq::kMaxBlocks)
    return fail(AQ_ERR_INVALID_ARG, "nproj = %d must be 1, 2 or 3", nproj);
  aq::Recon rq;
  aq_status s = build_recon(dt, M, K, x, ldx, p, nproj, y, ldy, true, &rq);
  if (s != AQ_OK) return s;
  s = check_rebuild(dt, M, p, nproj);
  if (s != AQ_OK || M == 0) return s;
  aq::RebuildPlan pl;
  aq::plan_rebuild(rq, &pl);
  if (pl.ws_bytes > 0) {
    if (!ws) return fail(AQ_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", pl.ws_bytes);
    if (ws_bytes < pl.ws_bytes) return fail(AQ_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", pl.ws_bytes, ws_bytes);
    if (!aligned(ws, 256)) return fail(AQ_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  }
  const hipError_t e = aq::launch_rebuild(rq, pl, ws, (hipStream_t)stream);
  if (e != hipSuccess) return fail(AQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return AQ_OK;
}

aq_status aq_band_mean(aq_dtype dt, int L, const void *const *W, int64_t N, int64_t K, void *W0, void *stream) {
  if (dt != AQ_F32 && dt != AQ_BF16) return fail(AQ_ERR_INVALID_ARG, "dtype %d is not AQ_F32 or AQ_BF16", (int)dt);
  if (L < 1 || L > aq::kMaxBandLayers) return fail(AQ_ERR_UNSUPPORTED, "L = %d layers: 1 to %d per band", L, aq::kMaxBandLayers);
  if (!W || !W0) return fail(AQ_ERR_INVALID_ARG, "W or W0 is NULL");
  if (N < 1 || K < 1) return fail(AQ_ERR_SHAPE, "N = %lld and K = %lld must be >= 1", (long long)N, (long long)K);
  if (N > kMaxDim || K > kMaxDim || N * K > kMaxElems) return fail(AQ_ERR_UNSUPPORTED, "weight exceeds 2^31-1 elements");
  for (int l = 0; l < L; ++l) {
    if (!W[l]) return fail(AQ_ERR_INVALID_ARG, "layer %d: W is NULL", l);
    if (!aligned(W[l], esize(dt))) return fail(AQ_ERR_ALIGNMENT, "layer %d: W is not naturally aligned", l);
  }
  if (!aligned(W0, esize(dt))) return fail(AQ_ERR_ALIGNMENT, "W0 is not naturally aligned");
  const hipError_t e = aq::launch_band_mean(dt, L, W, N * K, W0, (hipStream_t)stream);
  if (e != hipSuccess) return fail(AQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return AQ_OK;
}

// Shape checks shared by aq_decompose and its workspace query.
static aq_status check_decompose(int64_t N, int64_t K, int64_t r, int64_t l, int q) {
  if (N < 1 || K < 1) return fail(AQ_ERR_SHAPE, "N = %lld and K = %lld must be >= 1", (long long)N, (long long)K);
  if (N > kMaxDim || K > kMaxDim || N * K > kMaxElems) return fail(AQ_ERR_UNSUPPORTED, "weight exceeds 2^31-1 elements");
  if (r < 0 || q < 0) return fail(AQ_ERR_INVALID_ARG, "rank %lld and subspace steps %d must be >= 0", (long long)r, q);
  if (r > AQ_MAX_RANK) return fail(AQ_ERR_UNSUPPORTED, "rank %lld exceeds the supported maximum %d", (long long)r, AQ_MAX_RANK);
  if (r > 0 && (l < r || l > (N < K ? N : K)))
    return fail(AQ_ERR_SHAPE, "probe width l = %lld must be in [r, min(N, K)] = [%lld, %lld]", (long long)l,
                (long long)r, (long long)(N < K ? N : K));
  if (l > aq::kDecompMaxL) return fail(AQ_ERR_UNSUPPORTED, "probe width l = %lld exceeds %d", (long long)l, aq::kDecompMaxL);
  if (q > 64) return fail(AQ_ERR_UNSUPPORTED, "q = %d subspace steps: at most 64", q);
  return AQ_OK;
}

aq_status aq_decompose(aq_dtype dt, int64_t N, int64_t K, int64_t r, int64_t l, int q, const void *W,
                       const void *W0, const double *omega, double *s, double *U, double *Vt, void *ws,
                       size_t ws_bytes, void *stream) {
  if (dt != AQ_F32 && dt != AQ_BF16) return fail(AQ_ERR_INVALID_ARG, "dtype %d is not AQ_F32 or AQ_BF16", (int)dt);
  aq_status st = check_decompose(N, K, r, l, q);
  if (st != AQ_OK) return st;
  if (!W || !W0 || !s) return fail(AQ_ERR_INVALID_ARG, "W, W0 or s is NULL");
  if (r > 0 && (!omega || !U || !Vt)) return fail(AQ_ERR_INVALID_ARG, "rank %lld but omega, U or Vt is NULL", (long long)r);
  if (!aligned(W, esize(dt)) || !aligned(W0, esize(dt))) return fail(AQ_ERR_ALIGNMENT, "W or W0 is not naturally aligned");
  if (!aligned(s, 8) || (r > 0 && (!aligned(omega, 8) || !aligned(U, 8) || !aligned(Vt, 8))))
    return fail(AQ_ERR_ALIGNMENT, "s, omega, U and Vt must be 8-byte aligned");
  aq::DecompPlan pl;
  const size_t need = r > 0 ? aq::decompose_ws_bytes(N, K, r, l, &pl) : 0;
  if (need > 0) {
    if (!ws) return fail(AQ_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
    if (ws_bytes < need) return fail(AQ_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws_bytes);
    if (!aligned(ws, 256)) return fail(AQ_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  } else {
    pl = aq::DecompPlan{};
    pl.lj = 32;
  }
  aq::DecompArgs d{dt, N, K, r, l, q, W, W0, omega, s, U, Vt};
  const hipError_t e = aq::launch_decompose(d, pl, ws, (hipStream_t)stream);
  if (e != hipSuccess) return fail(AQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return AQ_OK;
}

size_t aq_decompose_workspace_bytes(int64_t N, int64_t K, int64_t r, int64_t l) {
  if (r == 0 || check_decompose(N, K, r, l, 0) != AQ_OK) return 0;
  aq::DecompPlan pl;
  return aq::decompose_ws_bytes(N, K, r, l, &pl);
}

aq_status aq_recon_linear_noalloc(aq_dtype dt, int64_t M, int64_t K, const void *x, int64_t ldx,
                                  const aq_proj *p, int nproj, void *y, int64_t ldy, void *stream) {
  if (nproj < 1 || nproj > aq::kMaxBlocks)
    return fail(AQ_ERR_INVALID_ARG, "nproj = %d must be 1, 2 or 3", nproj);
  void *ws = nullptr;
  const aq_status s = scratch_of_current_device(&ws);
  if (s != AQ_OK) return s;
  return recon(dt, M, K, x, ldx, p, nproj, y, ldy, ws, kScratchBytes, stream, true);
}

// Argument checks of one materialisation (also each item of a batch).
static aq_status check_materialize(aq_dtype dt, int64_t K, const aq_proj *p, const void *w_eff, int64_t ldw) {
  if (dt != AQ_F32 && dt != AQ_BF16) return fail(AQ_ERR_INVALID_ARG, "dtype %d is not AQ_F32 or AQ_BF16", (int)dt);
  if (!p) return fail(AQ_ERR_INVALID_ARG, "projection descriptor pointer is NULL");
  if (K < 1) return fail(AQ_ERR_SHAPE, "K = %lld must be >= 1", (long long)K);
  if (K > kMaxDim) return fail(AQ_ERR_UNSUPPORTED, "K = %lld exceeds 2^24", (long long)K);
  const int64_t kdiv = dt == AQ_BF16 ? 8 : 4;
  if (K % kdiv) return fail(AQ_ERR_ALIGNMENT, "K = %lld must be a multiple of %lld for this dtype", (long long)K, (long long)kdiv);
  if (p->N < 1) return fail(AQ_ERR_SHAPE, "N = %lld must be >= 1", (long long)p->N);
  if (p->N > kMaxDim) return fail(AQ_ERR_UNSUPPORTED, "N = %lld exceeds 2^24", (long long)p->N);
  if (p->r < 0) return fail(AQ_ERR_SHAPE, "rank %lld is negative", (long long)p->r);
  if (p->r > AQ_MAX_RANK) return fail(AQ_ERR_UNSUPPORTED, "rank %lld exceeds the supported maximum %d", (long long)p->r, AQ_MAX_RANK);
  if (ldw < K) return fail(AQ_ERR_SHAPE, "ldw = %lld < K = %lld", (long long)ldw, (long long)K);
  if (ldw % kdiv) return fail(AQ_ERR_ALIGNMENT, "ldw = %lld must be a multiple of %lld", (long long)ldw, (long long)kdiv);
  if (p->N * ldw > kMaxElems) return fail(AQ_ERR_UNSUPPORTED, "W_eff exceeds 2^31-1 elements");
  if (!p->W0 || !p->s || !w_eff) return fail(AQ_ERR_INVALID_ARG, "W0, s or w_eff is NULL");
  if (p->r > 0 && (!p->U || !p->Vt)) return fail(AQ_ERR_INVALID_ARG, "rank %lld but U or Vt is NULL", (long long)p->r);
  if (!aligned(p->W0, 16) || !aligned(w_eff, 16)) return fail(AQ_ERR_ALIGNMENT, "W0 and w_eff must be 16-byte aligned");
  if (p->r > 0 && !aligned(p->Vt, 16)) return fail(AQ_ERR_ALIGNMENT, "Vt must be 16-byte aligned");
  if (!aligned(p->s, esize(dt)) || (p->r > 0 && !aligned(p->U, esize(dt)))) return fail(AQ_ERR_ALIGNMENT, "s or U is not naturally aligned");
  return AQ_OK;
}

// Prefixes the detail string of the failure just recorded with the item index.
static aq_status item_fail(aq_status st, int i) {
  char tmp[sizeof g_err];
  snprintf(tmp, sizeof tmp, "item %d: %s", i, g_err);
  memcpy(g_err, tmp, sizeof g_err);
  return st;
}

aq_status aq_materialize_weff(aq_dtype dt, int64_t K, const aq_proj *p, void *w_eff,
                              int64_t ldw, void *stream) {
  const aq_status cs = check_materialize(dt, K, p, w_eff, ldw);
  if (cs != AQ_OK) return cs;
  aq::Proj P{p->N, p->r, p->W0, p->s, p->U, p->Vt, 0};
  hipError_t e = aq::launch_materialize(dt, K, P, w_eff, ldw, (hipStream_t)stream);
  if (e != hipSuccess) return fail(AQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return AQ_OK;
}

static aq_status check_fp4_pack(int64_t N, int64_t K, const void *w_bf16, int64_t ldw, const uint8_t *packed,
                                const uint8_t *scales, const float *global_scale) {
  if (N < 1) return fail(AQ_ERR_SHAPE, "N = %lld must be >= 1", (long long)N);
  if (K < 16) return fail(AQ_ERR_SHAPE, "K = %lld must be >= 16", (long long)K);
  if (N > kMaxDim || K > kMaxDim) return fail(AQ_ERR_UNSUPPORTED, "N or K exceeds 2^24");
  if (K % 16) return fail(AQ_ERR_ALIGNMENT, "K = %lld must be a multiple of 16", (long long)K);
  if (ldw < K) return fail(AQ_ERR_SHAPE, "ldw = %lld < K = %lld", (long long)ldw, (long long)K);
  if (ldw % 8) return fail(AQ_ERR_ALIGNMENT, "ldw = %lld must be a multiple of 8", (long long)ldw);
  if (N * ldw > kMaxElems) return fail(AQ_ERR_UNSUPPORTED, "weight exceeds 2^31-1 elements");
  if (!w_bf16 || !packed || !scales || !global_scale) return fail(AQ_ERR_INVALID_ARG, "a data pointer is NULL");
  if (!aligned(w_bf16, 16)) return fail(AQ_ERR_ALIGNMENT, "w is not 16-byte aligned");
  if (!aligned(packed, 8)) return fail(AQ_ERR_ALIGNMENT, "packed is not 8-byte aligned");
  if (!aligned(global_scale, 4)) return fail(AQ_ERR_ALIGNMENT, "global_scale is not 4-byte aligned");
  return AQ_OK;
}

aq_status aq_quant_fp4_block16(int64_t N, int64_t K, const void *w_bf16, int64_t ldw,
                               uint8_t *packed, uint8_t *scales, float *global_scale,
                               void *ws, size_t ws_bytes, void *stream) {
  const aq_status cs = check_fp4_pack(N, K, w_bf16, ldw, packed, scales, global_scale);
  if (cs != AQ_OK) return cs;
  const size_t need = aq::kWsReserved + (size_t)aq::kFp4AmaxBlocks * 4;
  if (!ws) return fail(AQ_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
  if (ws_bytes < need) return fail(AQ_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws_bytes);
  if (!aligned(ws, 256)) return fail(AQ_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  hipError_t e = aq::launch_fp4(N, K, w_bf16, ldw, packed, scales, global_scale, ws, (hipStream_t)stream);
  if (e != hipSuccess) return fail(AQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return AQ_OK;
}

aq_status aq_materialize_batch(aq_dtype dt, int n, const aq_mat_item *items, uint32_t *amax, void *stream) {
  if (dt != AQ_BF16) return fail(AQ_ERR_UNSUPPORTED, "the batched materialisation is bf16 only (dtype %d)", (int)dt);
  if (n < 0 || n > kMaxBatchItems) return fail(AQ_ERR_INVALID_ARG, "n = %d outside [0, %d]", n, kMaxBatchItems);
  if (n == 0) return AQ_OK;
  if (!items) return fail(AQ_ERR_INVALID_ARG, "items is NULL");
  if (amax && !aligned(amax, 4)) return fail(AQ_ERR_ALIGNMENT, "amax is not 4-byte aligned");
  std::vector<aq::MatItem> v((size_t)n);
  for (int i = 0; i < n; ++i) {
    const aq_mat_item &it = items[i];
    const aq_status cs = check_materialize(dt, it.K, &it.p, it.w_eff, it.ldw);
    if (cs != AQ_OK) return item_fail(cs, i);
    if (it.p.r > aq::kMatBatchMaxRank)
      return item_fail(fail(AQ_ERR_UNSUPPORTED, "rank %lld above %d (use aq_materialize_weff)", (long long)it.p.r,
                            aq::kMatBatchMaxRank), i);
    v[(size_t)i] = aq::MatItem{it.p.N, it.K, it.p.r, it.ldw, it.p.W0, it.p.s, it.p.U, it.p.Vt, it.w_eff};
  }
  hipError_t e = aq::launch_materialize_batch(n, v.data(), amax, (hipStream_t)stream);
  if (e != hipSuccess) return fail(AQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return AQ_OK;
}

size_t aq_materialize_fp4_batch_workspace_bytes(int n) {
  if (n < 1 || n > kMaxBatchItems) return 0;
  return aq::kWsReserved + ((size_t)n * 4 + 255) / 256 * 256;
}

aq_status aq_materialize_fp4_batch(int n, const aq_mat_fp4_item *items, void *ws, size_t ws_bytes, void *stream) {
  if (n < 0 || n > kMaxBatchItems) return fail(AQ_ERR_INVALID_ARG, "n = %d outside [0, %d]", n, kMaxBatchItems);
  if (n == 0) return AQ_OK;
  if (!items) return fail(AQ_ERR_INVALID_ARG, "items is NULL");
  std::vector<aq::MatItem> v((size_t)n);
  for (int i = 0; i < n; ++i) {
    const aq_mat_fp4_item &it = items[i];
    // the materialisation's checks on the bundle (no W_eff: W0 stands in for
    // it) and the pack's on the outputs
    aq_status cs = check_materialize(AQ_BF16, it.K, &it.p, it.p.W0 ? it.p.W0 : (const void *)&it, it.K);
    if (cs == AQ_OK && it.p.r > aq::kMatBatchMaxRank)
      cs = fail(AQ_ERR_UNSUPPORTED, "rank %lld above %d", (long long)it.p.r, aq::kMatBatchMaxRank);
    if (cs == AQ_OK) cs = check_fp4_pack(it.p.N, it.K, it.p.W0, it.K, it.packed, it.scales, it.global_scale);
    if (cs != AQ_OK) return item_fail(cs, i);
    aq::MatItem &m = v[(size_t)i];
    m = aq::MatItem{it.p.N, it.K, it.p.r, it.K, it.p.W0, it.p.s, it.p.U, it.p.Vt, nullptr};
    m.packed = it.packed;
    m.scales = it.scales;
    m.gscale = it.global_scale;
  }
  const size_t need = aq_materialize_fp4_batch_workspace_bytes(n);
  if (!ws) return fail(AQ_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
  if (ws_bytes < need) return fail(AQ_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws_bytes);
  if (!aligned(ws, 256)) return fail(AQ_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  unsigned *amax = (unsigned *)((char *)ws + aq::kWsReserved);
  hipError_t e = aq::launch_materialize_batch(n, v.data(), amax, (hipStream_t)stream, 1);
  if (e == hipSuccess) e = aq::launch_materialize_batch(n, v.data(), amax, (hipStream_t)stream, 2);
  if (e != hipSuccess) return fail(AQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return AQ_OK;
}

size_t aq_quant_fp4_batch_workspace_bytes(int n, int have_amax) {
  if (n < 1 || n > kMaxBatchItems) return 0;
  return aq::fp4_batch_ws_bytes(n, have_amax != 0);
}

aq_status aq_quant_fp4_batch(int n, const aq_fp4_item *items, const uint32_t *amax, void *ws, size_t ws_bytes,
                             void *stream) {
  if (n < 0 || n > kMaxBatchItems) return fail(AQ_ERR_INVALID_ARG, "n = %d outside [0, %d]", n, kMaxBatchItems);
  if (n == 0) return AQ_OK;
  if (!items) return fail(AQ_ERR_INVALID_ARG, "items is NULL");
  if (amax && !aligned(amax, 4)) return fail(AQ_ERR_ALIGNMENT, "amax is not 4-byte aligned");
  std::vector<aq::Fp4Item> v((size_t)n);
  for (int i = 0; i < n; ++i) {
    const aq_fp4_item &it = items[i];
    const aq_status cs = check_fp4_pack(it.N, it.K, it.w, it.ldw, it.packed, it.scales, it.global_scale);
    if (cs != AQ_OK) return item_fail(cs, i);
    v[(size_t)i] = aq::Fp4Item{it.N, it.K, it.ldw, it.w, it.packed, it.scales, it.global_scale};
  }
  const size_t need = aq::fp4_batch_ws_bytes(n, amax != nullptr);
  if (need > 0) {
    if (!ws) return fail(AQ_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
    if (ws_bytes < need) return fail(AQ_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws_bytes);
    if (!aligned(ws, 256)) return fail(AQ_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  }
  hipError_t e = aq::launch_fp4_batch(n, v.data(), amax, ws, (hipStream_t)stream);
  if (e != hipSuccess) return fail(AQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return AQ_OK;
}

// Shape checks shared by the FP4 GEMV and its workspace query.
static aq_status check_fp4_linear(int64_t M, int64_t N, int64_t K) {
  if (M < 0) return fail(AQ_ERR_INVALID_ARG, "M = %lld is negative", (long long)M);
  if (M > 16) return fail(AQ_ERR_UNSUPPORTED, "M = %lld: the FP4 GEMV takes at most 16 tokens", (long long)M);
  if (N < 1) return fail(AQ_ERR_SHAPE, "N = %lld must be >= 1", (long long)N);
  if (K < 32) return fail(AQ_ERR_SHAPE, "K = %lld must be >= 32", (long long)K);
  if (N > kMaxDim || K > kMaxK) return fail(AQ_ERR_UNSUPPORTED, "N or K too large");
  if (K % 32) return fail(AQ_ERR_ALIGNMENT, "K = %lld must be a multiple of 32", (long long)K);
  if (N * (K / 2) > kMaxElems) return fail(AQ_ERR_UNSUPPORTED, "packed weight exceeds 2^31-1 bytes");
  return AQ_OK;
}

aq_status aq_fp4_linear(int64_t M, int64_t N, int64_t K, const void *x, int64_t ldx, const uint8_t *packed,
                        const uint8_t *scales, const float *global_scale, void *y, int64_t ldy, void *ws,
                        size_t ws_bytes, void *stream) {
  aq_status st = check_fp4_linear(M, N, K);
  if (st != AQ_OK) return st;
  if (ldx < K) return fail(AQ_ERR_SHAPE, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
  if (ldx % 8) return fail(AQ_ERR_ALIGNMENT, "ldx = %lld must be a multiple of 8", (long long)ldx);
  if (ldy < N) return fail(AQ_ERR_SHAPE, "ldy = %lld < N = %lld", (long long)ldy, (long long)N);
  if (M * ldx > kMaxElems || M * ldy > kMaxElems) return fail(AQ_ERR_UNSUPPORTED, "x or y exceeds 2^31-1 elements");
  if (M == 0) return AQ_OK;
  if (!x || !y || !packed || !scales || !global_scale) return fail(AQ_ERR_INVALID_ARG, "a data pointer is NULL");
  if (!aligned(x, 16) || !aligned(packed, 16)) return fail(AQ_ERR_ALIGNMENT, "x and packed must be 16-byte aligned");
  if (!aligned(scales, 2) || !aligned(y, 2) || !aligned(global_scale, 4))
    return fail(AQ_ERR_ALIGNMENT, "scales, y or global_scale is not naturally aligned");
  aq::Fp4LinPlan pl;
  aq::plan_fp4_linear(M, N, K, &pl);
  if (pl.ws_bytes > 0) {
    if (!ws) return fail(AQ_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", pl.ws_bytes);
    if (ws_bytes < pl.ws_bytes) return fail(AQ_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", pl.ws_bytes, ws_bytes);
    if (!aligned(ws, 256)) return fail(AQ_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  }
  hipError_t e = aq::launch_fp4_linear(M, N, K, x, ldx, packed, scales, global_scale, y, ldy, pl, ws,
                                       (hipStream_t)stream);
  if (e != hipSuccess) return fail(AQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return AQ_OK;
}

size_t aq_workspace_bytes(aq_op op, aq_dtype dt, int64_t M, int64_t K, const aq_proj *p,
                          int nproj) {
  if (op == AQ_OP_FP4) return aq::kWsReserved + (size_t)aq::kFp4AmaxBlocks * 4;
  if (op == AQ_OP_FP4_LINEAR) {
    if (!p || nproj != 1 || M == 0 || check_fp4_linear(M, p[0].N, K) != AQ_OK) return 0;
    aq::Fp4LinPlan pl;
    aq::plan_fp4_linear(M, p[0].N, K, &pl);
    return pl.ws_bytes;
  }
  if (op == AQ_OP_REBUILD) {
    if (!p || nproj < 1 || nproj > aq::kMaxBlocks || M == 0) return 0;
    int64_t ntot = 0;
    for (int b = 0; b < nproj; ++b) ntot += p[b].N > 0 ? p[b].N : 0;
    aq::Recon rq;
    if (build_recon(dt, M, K, nullptr, K, p, nproj, nullptr, ntot, false, &rq) != AQ_OK) return 0;
    if (check_rebuild(dt, M, p, nproj) != AQ_OK) return 0;
    aq::RebuildPlan pl;
    aq::plan_rebuild(rq, &pl);
    return pl.ws_bytes;
  }
  if (op != AQ_OP_RECON || nproj < 1 || nproj > aq::kMaxBlocks || !p) return 0;
  int64_t ntot = 0;
  for (int b = 0; b < nproj; ++b) ntot += p[b].N > 0 ? p[b].N : 0;
  aq::Recon rq;
  if (build_recon(dt, M, K, nullptr, K, p, nproj, nullptr, ntot, false, &rq) != AQ_OK) return 0;
  if (M == 0) return 0;
  rq.ldx = K;
  rq.ldy = rq.Ntot;
  Plan pl;
  make_plan(rq, &pl);
  return pl.ws;
}

const char *aq_status_string(aq_status s) {
  switch (s) {
    case AQ_OK: return "AQ_OK";
    case AQ_ERR_INVALID_ARG: return "AQ_ERR_INVALID_ARG";
    case AQ_ERR_SHAPE: return "AQ_ERR_SHAPE";
    case AQ_ERR_ALIGNMENT: return "AQ_ERR_ALIGNMENT";
    case AQ_ERR_UNSUPPORTED: return "AQ_ERR_UNSUPPORTED";
    case AQ_ERR_WORKSPACE: return "AQ_ERR_WORKSPACE";
    case AQ_ERR_HIP: return "AQ_ERR_HIP";
    case AQ_ERR_HANDOFF: return "AQ_ERR_HANDOFF";
  }
  return "AQ_ERR_UNKNOWN";
}

const char *aq_last_error(void) { return g_err; }

aq_status aq_workspace_check(void *ws, void *stream) {
  if (!ws) {
    const aq_status s = scratch_of_current_device(&ws);
    if (s != AQ_OK) return s;
  }
  if (!aligned(ws, 256)) return fail(AQ_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  unsigned w[aq::kSyncWords] = {};
  if (e == hipSuccess) e = hipMemcpy(w, ws, sizeof w, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(AQ_ERR_HIP, "reading the workspace failed: %s", hipGetErrorString(e));
  unsigned passed = 0, any = 0;
  for (int g = 0; g < aq::kHandoffGroups; ++g) passed += w[aq::kSyncGroup0 + aq::kSyncGroupStride * g];
  for (unsigned v : w) any |= v;
  if (!any) return AQ_OK;
  e = hipMemset(ws, 0, sizeof w);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return fail(AQ_ERR_HIP, "clearing the workspace failed: %s", hipGetErrorString(e));
  if (w[aq::kSyncFlag])
    return fail(AQ_ERR_HANDOFF,
                "a launch gave up waiting for the workgroups that compute t (arrivals %u, waiters passed %u): "
                "the outputs of the calls since the last check are not valid; the workspace has been cleared",
                w[aq::kSyncArrive], passed);
  return fail(AQ_ERR_WORKSPACE,
              "hand-off counters not zero (arrivals %u, groups %u, waiters passed %u): the workspace was not "
              "zero-filled or was used by concurrent calls; it has been cleared",
              w[aq::kSyncArrive], w[aq::kSyncGroups], passed);
}

aq_status aq_debug_force_plan(aq_debug_knob knob, int64_t value) {
  if (knob < 0 || knob >= AQ_DBG_COUNT) return fail(AQ_ERR_INVALID_ARG, "unknown plan knob %d", (int)knob);
  if (value < INT_MIN + 1 || value > INT_MAX) return fail(AQ_ERR_INVALID_ARG, "knob value out of range");
  g_knobs.v[knob] = (int)value;
  return AQ_OK;
}

void aq_debug_reset_plan(void) { g_knobs = Knobs(); }

int aq_version(void) { return 100; }

}  // extern "C"
