/*
 * aq.h -- C ABI of the MI355X (gfx950) theta-bundle reconstructed linear.
 *
 * A theta bundle replaces one projection's dense [out_dim, in_dim] weight by a
 * shared block W0, a per-output-row scale s and a rank-r pair U, V
 * ("How attnquant works", section "The theta bundle").  This library computes,
 * on one GPU and with hand-written HIP kernels:
 *
 *   y     = s * (x W0^T) + (x Vt^T) U^T           (the reconstruction identity)
 *   W_eff = diag(s) W0 + U Vt                     (the effective weight)
 *   FP4   = block-16 E2M1 codes + E4M3 scales + fp32 global scale of W_eff
 *   y     = x Wq^T                                (decode over the FP4-packed W_eff)
 *
 * Conventions shared by every call
 * --------------------------------
 * - Row vectors: x is [M, K] (M tokens, K = in_dim), y is [M, N] (N = out_dim).
 * - All matrices are row-major with unit column stride.  W0 is [N, K] with row
 *   stride K; s is [N]; U is [N, r] with row stride r; Vt = V^T is [r, K] with
 *   row stride K (the pages' V is [K, r]; it is passed transposed so that W0 and
 *   Vt are both K-contiguous).
 * - Every pointer to tensor data is a DEVICE pointer owned by the caller; the
 *   library never frees or retains it.  All tensors of one call share one dtype
 *   (aq_dtype).  Outputs must not alias inputs.
 * - Every call only enqueues work on `stream` (a hipStream_t; NULL = the null
 *   stream) and returns without synchronising.  Argument errors are detected on
 *   the host before anything is enqueued and return a status other than AQ_OK;
 *   in that case nothing was launched.  A launch failure returns AQ_ERR_HIP.
 *   Faults during execution surface at the caller's next synchronisation.
 * - aq_last_error() returns a thread-local, human-readable detail of the last
 *   failing call on this thread (which argument, which shape).
 * - No C++ exception crosses this boundary.
 */
#ifndef AQ_H
#define AQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum aq_status {
  AQ_OK = 0,
  AQ_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad enum             */
  AQ_ERR_SHAPE = 2,       /* sizes or strides that do not fit together         */
  AQ_ERR_ALIGNMENT = 3,   /* pointer / stride / K not aligned as required      */
  AQ_ERR_UNSUPPORTED = 4, /* valid request outside the library's limits        */
  AQ_ERR_WORKSPACE = 5,   /* workspace missing, too small or misaligned        */
  AQ_ERR_HIP = 6,         /* the HIP runtime refused a launch                  */
  AQ_ERR_HANDOFF = 7      /* a prefill launch's wait for t gave up (see
                             aq_workspace_check)                               */
} aq_status;

typedef enum aq_dtype { AQ_F32 = 0, AQ_BF16 = 1 } aq_dtype;

typedef enum aq_op { AQ_OP_RECON = 0, AQ_OP_FP4 = 1, AQ_OP_FP4_LINEAR = 2, AQ_OP_REBUILD = 3 } aq_op;

#define AQ_MAX_RANK 256

/* One projection's bundle ("How attnquant works", section "The theta bundle").
 * N = out_dim; r = rank (0 <= r <= AQ_MAX_RANK; for r == 0, U and Vt are
 * ignored and may be NULL, and the projection is a pure scaled shared block as
 * the end of "How the decomposition produces s, U, and V" describes).
 * W0 [N, K], s [N], U [N, r], Vt [r, K], all device pointers, one dtype. */
typedef struct aq_proj {
  int64_t N;
  int64_t r;
  const void *W0;
  const void *s;
  const void *U;
  const void *Vt;
} aq_proj;

/* y[M, ldy] (columns 0..N-1) = s * (x W0^T) + (x Vt^T) U^T.
 * "How attnquant works", section "The reconstruction identity"; row-batch form of
 * "Execution paths", section "The GEMM formulation".
 *   dt     AQ_BF16: bf16 storage, fp32 accumulation, one rounding of y to bf16.
 *          AQ_F32 : fp32 storage and arithmetic.
 *   M      tokens (0 is a no-op returning AQ_OK; x and y may then be NULL).
 *   K      in_dim >= 1; bf16 needs K % 8 == 0, f32 needs K % 4 == 0.
 *   x      [M, ldx], ldx >= K, same divisibility as K; 16-byte aligned.
 *   p      one projection; W0 and Vt 16-byte aligned; s, U naturally aligned.
 *   y      [M, ldy], ldy >= N; naturally aligned.
 *   ws     device workspace of at least aq_workspace_bytes(AQ_OP_RECON, ...)
 *          bytes, 256-byte aligned (NULL allowed when that size is 0).  Its
 *          first 64 KiB hold arrival counters (the hand-off of t from the
 *          rank-r pass to the main pass when both run in one prefill launch):
 *          they must be zero before the first use, and every call leaves them
 *          zero again; the rest is
 *          per-call scratch.  So one zeroed allocation can serve any number and
 *          kind of calls (recon and FP4) that are ordered on one stream.  Calls
 *          that share a workspace must not run concurrently.
 * Limits: 1 <= N <= 2^24; 1 <= K, ldx < 2^22; M <= 2^19; N * K and M * ldx, M * ldy
 * below 2^31 elements; r <= AQ_MAX_RANK (else
 * AQ_ERR_UNSUPPORTED, a refusal rather than a silent fallback, as the pages' own
 * custom op refuses ranks above its limit: "Execution paths", "The custom op"). */
aq_status aq_recon_linear(aq_dtype dt, int64_t M, int64_t K, const void *x, int64_t ldx,
                          const aq_proj *p, void *y, int64_t ldy, void *ws, size_t ws_bytes,
                          void *stream);

/* Fused Q/K/V: p[0..2] = (q, k, v) read the same x; y = [y_q | y_k | y_v]
 * concatenated along N (columns 0..Nq+Nk+Nv-1 of y), in one dispatch whose
 * down-contraction runs over [W0_q; W0_k; W0_v; Vt_q; Vt_k; Vt_v] and whose
 * up-projection is block-diagonal in U ("Execution paths", section "The GEMM
 * formulation", the Q/K/V batching paragraph; section "Precompute-outside" for
 * the concatenation along the output axis).  Arguments as aq_recon_linear;
 * ldy >= Nq + Nk + Nv.  Each block may have its own N and r. */
aq_status aq_recon_qkv_fused(aq_dtype dt, int64_t M, int64_t K, const void *x, int64_t ldx,
                             const aq_proj p[3], void *y, int64_t ldy, void *ws,
                             size_t ws_bytes, void *stream);

/* Fused gate/up: p[0..1] = (gate, up); y = [y_gate | y_up] along N.  Same
 * batching as Q/K/V ("Execution paths", section "The GEMM formulation": the MLP
 * fuses gate and up the same way).  No activation is applied (the pages name
 * none).  Arguments as aq_recon_linear; ldy >= Ngate + Nup. */
aq_status aq_recon_gateup_fused(aq_dtype dt, int64_t M, int64_t K, const void *x,
                                int64_t ldx, const aq_proj p[2], void *y, int64_t ldy,
                                void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * computation as aq_recon_linear (nproj = 1), aq_recon_gateup_fused (nproj =
 * 2, p = (gate, up)) or aq_recon_qkv_fused (nproj = 3, p = (q, k, v)), with the
 * same kernels and results, but with no workspace argument: the scratch comes
 * from an array of 16 MiB that the library holds on each GPU (allocated when
 * the library is loaded, kept until the process ends), the one of the device
 * that is current at the call (the stream must belong to it).  Nothing is
 * allocated or freed.  A call whose plan needs more scratch than 16 MiB
 * returns AQ_ERR_UNSUPPORTED (every decode and prefill dispatch of the
 * Gemma-3-1B-shaped and larger-decoder-shaped layers needs at most 7 MiB).
 * Every call on one GPU shares that GPU's array and overwrites what the
 * previous call left there; calls that overlap in time on one GPU (on
 * different streams, or from several threads) race and must not be issued.
 * Before a launch that hands t between its workgroups, the hand-off counters
 * are zeroed by a small kernel (graph-capturable); a wait that gave up is
 * reported by aq_workspace_check(NULL, stream).  Limits and errors as
 * aq_recon_linear; nproj outside 1..3 is AQ_ERR_INVALID_ARG. */
aq_status aq_recon_linear_noalloc(aq_dtype dt, int64_t M, int64_t K, const void *x, int64_t ldx,
                                  const aq_proj *p, int nproj, void *y, int64_t ldy, void *stream);

/* Per-element reconstruction: y = x W_eff^T with every weight of W_eff = diag(s)
 * W0 + U Vt rebuilt inside the kernel, rounded once to bf16, and the dense
 * [N, K] matrix never formed ("Execution paths", section "The custom op": the
 * weight rebuilt per element, one dispatch per projection).  p[0..nproj-1]
 * (nproj = 1, 2 or 3) read the same x; y = [y_0 | y_1 | ...] along N as for the
 * fused recon calls.  Limits as that section states for its custom op: r <= 64
 * per block (larger ranks are refused with AQ_ERR_UNSUPPORTED, a refusal rather
 * than a silent fallback; use aq_recon_* there), and it is a decode kernel:
 * M <= 16 tokens (else AQ_ERR_UNSUPPORTED; M == 0 is a no-op).  bf16 only
 * (AQ_F32 is AQ_ERR_UNSUPPORTED).  Arguments otherwise as aq_recon_linear;
 * ws: aq_workspace_bytes(AQ_OP_REBUILD, ...) bytes (0 unless long K is split
 * over workgroups: then fp32 partials after the reserved region), 256-byte
 * aligned.  Precision: the rank-r products and s W0 + U Vt in fp32, one bf16
 * rounding per rebuilt weight (relative <= 2^-8), exact products with x, fp32
 * sums, one rounding of y. */
aq_status aq_rebuild_linear(aq_dtype dt, int64_t M, int64_t K, const void *x, int64_t ldx,
                            const aq_proj *p, int nproj, void *y, int64_t ldy, void *ws,
                            size_t ws_bytes, void *stream);

/* W_eff[N, ldw] (columns 0..K-1) = diag(s) W0 + U Vt, accumulated in fp32 and
 * rounded once to dt.  "Execution paths", section "Precompute-outside" (the weight
 * rebuilt once at load) and "How attnquant works", section "The reconstruction
 * identity".  ldw >= K lets the caller write straight into a row range of a
 * stacked Q/K/V or gate/up buffer.  bf16: K % 8 == 0, ldw % 8 == 0, W0, Vt and
 * w_eff 16-byte aligned; f32: K % 4 == 0, ldw % 4 == 0.  No workspace.
 * For r == 0 (and for s = 1, U = Vt = 0) the result is bit-exact: one rounding
 * of the exact product s * W0. */
aq_status aq_materialize_weff(aq_dtype dt, int64_t K, const aq_proj *p, void *w_eff,
                              int64_t ldw, void *stream);

/* Block-16 FP4 pack of a bf16 weight w[N, ldw] (columns 0..K-1).
 * Container: "Internals and extension", section "Nvfp4Spec" -- two E2M1 codes per
 * byte, one FP8-E4M3 scale per 16 K-values in the linear [N, K/16] layout, one
 * fp32 global scale.  Recipe (the pages give only the container):
 *   g  = RN_f32(max|w| / 2688) (1 when max|w| == 0), written to *global_scale;
 *   scale[n, b] = E4M3FN round-to-nearest-even, saturating at 448, of
 *                 max|w[n, 16b..16b+15]| / (6 g);
 *   D  = RN_f32(g * scale); code = E2M1 round-to-nearest-even (ties to the even
 *        code, saturating at 6) of |w| / D, sign bit only on non-zero codes,
 *        all codes 0 when D == 0;
 *   packed[n, i] = code[n, 2i] | code[n, 2i+1] << 4.
 * Every decision is exact (no approximate division), so the output is one bit
 * pattern.  N >= 1, K % 16 == 0, ldw >= K, ldw % 8 == 0, w 16-byte aligned,
 * packed [N, K/2] 8-byte aligned (row stride K/2), scales [N, K/16] (row stride
 * K/16), global_scale: one device float.  ws: aq_workspace_bytes(AQ_OP_FP4, ...)
 * bytes, 256-byte aligned; its first 64 KiB (the recon counters) are not
 * touched, the scratch after them needs no zero-fill.  Input must be finite. */
aq_status aq_quant_fp4_block16(int64_t N, int64_t K, const void *w_bf16, int64_t ldw,
                               uint8_t *packed, uint8_t *scales, float *global_scale,
                               void *ws, size_t ws_bytes, void *stream);

/* Load-time materialisation of many projections in a few launches (bf16):
 * items[i] gets w_eff = diag(s) W0 + U Vt exactly as aq_materialize_weff
 * computes it (same bits), for the whole model at once ("Execution paths",
 * section "Precompute-outside": every layer's W_eff is rebuilt once at load;
 * "How attnquant works", section "The theta bundle": the layers of a band share
 * W0).  Consecutive items that name the same W0 (same pointer, N and K) form
 * a run -- the layers of one band for one projection family -- and each W0
 * tile is read once for the first two items of its run (a longer run is taken
 * two items at a time).  amax: NULL, or n device words; amax[i] receives the
 * largest magnitude of item i's W_eff as bf16 bits (bits 0..14 of the rounded
 * values, an exact maximum), which aq_quant_fp4_batch takes to skip its own
 * pass over the weights.  Per item as aq_materialize_weff (bf16), plus
 * r <= 64 (AQ_ERR_UNSUPPORTED above: use aq_materialize_weff); errors name
 * the item ("item 5: ...").  0 <= n <= 65536; no workspace; a few launches
 * (up to 24 runs each) on stream. */
typedef struct aq_mat_item {
  int64_t K;        /* in_dim */
  aq_proj p;        /* N, r, W0, s, U, Vt */
  void *w_eff;      /* bf16 [N, ldw], columns 0..K-1 written */
  int64_t ldw;
} aq_mat_item;
aq_status aq_materialize_batch(aq_dtype dt, int n, const aq_mat_item *items, uint32_t *amax, void *stream);

/* Block-16 FP4 pack of many bf16 weights, each exactly as
 * aq_quant_fp4_block16 packs it (same bytes and global scale), in a few
 * launches ("Execution paths", section "Precompute-outside": each W_eff is
 * quantised at load; "Internals and extension", section "Nvfp4Spec").  amax:
 * the weights' largest magnitudes as bf16 bits (from aq_materialize_batch),
 * then one pass reads each weight once; NULL: a first pass computes them into
 * the workspace.  ws: aq_quant_fp4_batch_workspace_bytes(n, amax != NULL)
 * bytes (0: may be NULL), 256-byte aligned, its first 64 KiB untouched.
 * Per item as aq_quant_fp4_block16; errors name the item. */
typedef struct aq_fp4_item {
  int64_t N, K, ldw;
  const void *w;          /* bf16 [N, ldw] */
  uint8_t *packed;        /* [N, K/2] */
  uint8_t *scales;        /* [N, K/16] */
  float *global_scale;    /* one device float */
} aq_fp4_item;
aq_status aq_quant_fp4_batch(int n, const aq_fp4_item *items, const uint32_t *amax, void *ws, size_t ws_bytes,
                             void *stream);
size_t aq_quant_fp4_batch_workspace_bytes(int n, int have_amax);

/* The FP4 weights of many projections without their bf16 W_eff: the same
 * bytes and global scales as aq_materialize_batch followed by
 * aq_quant_fp4_batch with its maxima ("Execution paths", section
 * "Precompute-outside": W_eff rebuilt at load and quantised there, where only
 * the quantised weight is kept; "Internals and extension", section
 * "Nvfp4Spec").  Two passes over the shared blocks and factors: the first
 * forms every W_eff tile and keeps only each weight's largest magnitude, the
 * second forms the same tiles again and encodes them; W_eff never reaches
 * memory.  bf16, r <= 64, K % 16 == 0; items as aq_mat_item with the packed
 * outputs of aq_fp4_item (dense [N, K/2] codes 8-byte aligned, [N, K/16]
 * scales, one device float); consecutive items on the same W0 (the layers of
 * a band) share its reads.  ws: aq_materialize_fp4_batch_workspace_bytes(n)
 * bytes, 256-byte aligned (the maxima, after the reserved region, which is
 * not touched).  Errors name the item.  Asynchronous on `stream`. */
typedef struct aq_mat_fp4_item {
  int64_t K;              /* in_dim */
  aq_proj p;              /* N, r, W0, s, U, Vt */
  uint8_t *packed;        /* [N, K/2] */
  uint8_t *scales;        /* [N, K/16] */
  float *global_scale;    /* one device float */
} aq_mat_fp4_item;
aq_status aq_materialize_fp4_batch(int n, const aq_mat_fp4_item *items, void *ws, size_t ws_bytes, void *stream);
size_t aq_materialize_fp4_batch_workspace_bytes(int n);

/* FP4 decode GEMV over a packed weight: y[m, n] = bf16(sum_k x[m, k] * Wq[n, k])
 * for m < M <= 16 tokens, where Wq[n, k] = E2M1(code) * RN_f32(g * E4M3(scale))
 * is the weight that aq_quant_fp4_block16's output stands for ("Execution
 * paths", section "Precompute-outside": the quantised W_eff replaces the dense
 * weight; "Internals and extension", section "Nvfp4Spec": the container).
 *   x       bf16 [M, ldx], ldx >= K, ldx % 8 == 0, 16-byte aligned.
 *   packed  [N, K/2] bytes (code 2i in the low nibble of byte i), 16-byte aligned;
 *   scales  [N, K/16] E4M3FN bytes; global_scale: one device float (g).
 *   y       bf16 [M, ldy], ldy >= N.
 *   ws      aq_workspace_bytes(AQ_OP_FP4_LINEAR, -, M, K, p = {N, ...}, 1)
 *           bytes (0 when K is not split; else fp32 partials after the
 *           reserved region), 256-byte aligned.
 * Each weight is rounded once to bf16 before the fp32-accumulated MFMA
 * product (relative error <= 2^-8 per weight), except for M <= 4 with K % 64
 * == 0, where the block step is applied per block after an exact product of the
 * E2M1 values.  K % 32 == 0, K >= 32; M > 16
 * is AQ_ERR_UNSUPPORTED; M == 0 is a no-op.  Asynchronous on `stream`. */
aq_status aq_fp4_linear(int64_t M, int64_t N, int64_t K, const void *x, int64_t ldx,
                        const uint8_t *packed, const uint8_t *scales, const float *global_scale,
                        void *y, int64_t ldy, void *ws, size_t ws_bytes, void *stream);

/* The decomposition that produces a bundle from trained weights, on the GPU
 * ("How attnquant works", section "How the decomposition produces s, U, and V",
 * and the band-mean sentence after it).  All results are float64.
 *
 * aq_band_mean: W0[N, K] = the mean of the L layer weights W[0..L-1] that share
 * it, summed in float64 (exact for bf16 and fp32 inputs), divided by L and
 * rounded once to dt; bit-exact against the exact mean rounded once.  W is a
 * HOST array of L device pointers (1 <= L <= 64), every weight [N, K]
 * row-major with unit stride, dt storage, naturally aligned.
 *
 * aq_decompose: for one weight W [N, K] and its shared block W0 [N, K] (dt
 * storage, row-major, unit stride):
 *   s[o]  = (W[o] . W0[o]) / (W0[o] . W0[o])   (1 where W0[o] is zero),
 *   R     = W - diag(s) W0,
 *   U, Vt = the rank-r truncated SVD of R with U absorbing the singular values,
 * the SVD by the randomized method (Halko, Martinsson and Tropp, 2009) with
 * the caller's Gaussian test matrix omega [l, K] (row j = probe j, l = r +
 * oversampling) and q steps of re-orthonormalised subspace iteration:
 * Y = R omega^T, Q = orth(Y); q times Q~ = orth(R^T Q), Q = orth(R Q~);
 * B = Q^T R = U_b S V^T; U = Q U_b[:, :r] S[:r]; Vt = V^T[:r].  The pages take
 * a full SVD when min(N, K) <= 256 or when the oversampled probe would cover
 * the matrix: pass l = min(N, K) there, and the same steps give the exact
 * truncated SVD.  Outputs: s [N], U [N, r] (row stride r), Vt [r, K] (row
 * stride K), float64, 8-byte aligned; r == 0 computes s only (omega, U, Vt may
 * be NULL).  Limits: r <= l <= min(N, K), l <= 256, q <= 64, N * K < 2^31.
 * ws: aq_decompose_workspace_bytes(N, K, r, l) bytes, 256-byte aligned (the
 * basis, the co-range, partial sums; no zero-fill needed); its first 64 KiB
 * (the recon calls' counter words) are not touched, so the same workspace
 * serves both kinds of call -- except the flag word that aq_workspace_check
 * reads: for l > 96 the eigensolver runs on many workgroups with bounded
 * grid barriers, and one that gives up sets that flag and makes U and Vt NaN
 * (never seen in practice; the call's stream must not run another call on the
 * same workspace at the same time).  Asynchronous on
 * stream; many launches, all on that stream.  Singular vectors are unique only
 * up to sign (and within repeated singular values): U Vt is the result. */
aq_status aq_band_mean(aq_dtype dt, int L, const void *const *W, int64_t N, int64_t K, void *W0,
                       void *stream);
aq_status aq_decompose(aq_dtype dt, int64_t N, int64_t K, int64_t r, int64_t l, int q, const void *W,
                       const void *W0, const double *omega, double *s, double *U, double *Vt, void *ws,
                       size_t ws_bytes, void *stream);
/* 0 for r == 0 or invalid arguments (the call itself then reports why). */
size_t aq_decompose_workspace_bytes(int64_t N, int64_t K, int64_t r, int64_t l);

/* Workspace size in bytes for one call.
 *   AQ_OP_RECON: (dt, M, K, p[0..nproj-1]) exactly as passed to the recon call
 *                (nproj = 1, 3 or 2).
 *   AQ_OP_FP4  : M and dt ignored; p[0].N and K are the weight's shape.
 *   AQ_OP_FP4_LINEAR: dt ignored; M tokens, p[0].N and K the packed weight's
 *                shape (nproj = 1).
 *   AQ_OP_REBUILD: (dt, M, K, p[0..nproj-1]) as passed to aq_rebuild_linear.
 * Returns 0 for invalid arguments (the call itself then reports why).
 * Host-only: touches no GPU state. */
size_t aq_workspace_bytes(aq_op op, aq_dtype dt, int64_t M, int64_t K, const aq_proj *p,
                          int nproj);

/* Health check of a workspace after the calls that used it: waits for `stream`
 * to drain (this call synchronises), then reads the reserved region.
 *
 * A prefill launch that also runs the rank-r pass in its first workgroups has
 * its main tiles wait, before they first read t, for every rank-r workgroup to
 * count itself in the workspace ("Execution paths", section "The GEMM
 * formulation": the down-contraction and the up-projection are two dependent
 * GEMMs; here they meet inside one launch).  That wait is bounded so that a
 * kernel can never hang: if it ever gives up, the main tiles go on with
 * whatever t holds and set a flag word in the reserved region.  This call
 * reports the flag as AQ_ERR_HANDOFF (the outputs of the prefill calls since
 * the last check are then not valid), and AQ_ERR_WORKSPACE if the counters are
 * not back at zero (a workspace that was not zero-filled, or shared by calls
 * that ran concurrently).  In both cases it clears the reserved region, so the
 * workspace can be used again.  AQ_OK otherwise.  ws must be the workspace
 * pointer passed to the calls (256-byte aligned); NULL checks the scratch of
 * aq_recon_linear_noalloc on the current device. */
aq_status aq_workspace_check(void *ws, void *stream);

const char *aq_status_string(aq_status s);
const char *aq_last_error(void);

/* Test-only plan overrides, for callers that must force one particular kernel
 * variant (the parity tests exercise every compiled tile shape, split and mode
 * this way): the kernel choice of a call otherwise depends only on its
 * arguments.  The overrides are thread-local, unset until set, and apply to
 * the calls made on the same thread; values that no compiled variant takes
 * are ignored by the planner, as if unset.  AQ_DBG_HANDOFF_SPIN bounds the
 * prefill wait for t, and each grid barrier of the decomposition's many-
 * workgroup eigensolver, to that many polls; AQ_DBG_HANDOFF_UNREACHABLE = 1
 * makes the awaited count one more than will arrive, so that a test can make
 * the wait give up from the host while every kernel still exits normally.
 * AQ_DBG_JACOBI picks the eigensolver (1: one workgroup with both matrices in
 * LDS, taken only where l <= 96; 2: the scalar many-workgroup one; 3: the
 * block one, the default above l = 96) and AQ_DBG_JACOBI_WGS the scalar
 * many-workgroup one's workgroups (1 to 64).
 * aq_debug_force_plan returns AQ_ERR_INVALID_ARG for an unknown knob. */
typedef enum aq_debug_knob {
  AQ_DBG_DECODE_SPLIT = 0, AQ_DBG_DECODE_NG, AQ_DBG_DECODE_ROWS, AQ_DBG_DECODE_S, AQ_DBG_DECODE_WAVES,
  AQ_DBG_PREFILL_BM, AQ_DBG_PREFILL_BN, AQ_DBG_PREFILL_BK, AQ_DBG_PREFILL_NST, AQ_DBG_PREFILL_W,
  AQ_DBG_PREFILL_S, AQ_DBG_PREFILL_SELF, AQ_DBG_PREFILL_FUSE, AQ_DBG_TPASS_S, AQ_DBG_TPASS_PARTS,
  AQ_DBG_FP4_NG, AQ_DBG_FP4_S, AQ_DBG_FP4_M4, AQ_DBG_HANDOFF_SPIN, AQ_DBG_HANDOFF_UNREACHABLE,
  AQ_DBG_REBUILD_NG, AQ_DBG_REBUILD_ROWS, AQ_DBG_REBUILD_S, AQ_DBG_MAT_STEPS, AQ_DBG_FP4_UNIT,
  AQ_DBG_JACOBI, AQ_DBG_JACOBI_WGS,
  AQ_DBG_COUNT
} aq_debug_knob;
aq_status aq_debug_force_plan(aq_debug_knob knob, int64_t value);
void aq_debug_reset_plan(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int aq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* AQ_H */
