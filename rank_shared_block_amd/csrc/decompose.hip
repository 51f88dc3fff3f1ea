// The decomposition that produces a theta bundle from trained weights, on the
// GPU ("How attnquant works", section "How the decomposition produces s, U, and
// V", and the band-mean sentence after it):
//
//   W0     = mean of the weights of the layers that share it         (aq_band_mean)
//   s[o]   = (W[o] . W0[o]) / (W0[o] . W0[o])     (s[o] = 1 where W0[o] = 0)
//   R      = W - diag(s) W0
//   U, Vt  = rank-r truncated SVD of R, U absorbing the singular values,
//            by the randomized method of Halko, Martinsson and Tropp (2009):
//            Y = R Omega^T, Q = orth(Y); q times Q~ = orth(R^T Q), Q = orth(R Q~);
//            B = Q^T R = U_b S V^T;  U = Q U_b[:, :r] S[:r],  Vt = V^T[:r]
//                                                                     (aq_decompose)
//
// Everything after the inputs is float64: a load-time step whose result every
// later forward pass reuses, so it is computed to the precision of the pages'
// numpy.  The residual R is never stored: every pass forms it from W, W0 (bf16
// or fp32) and s on the fly.  Tall matrices (the range basis Y, Q [N, l]; the
// co-range Z = R^T Q [K, l], which is B^T) are kept column-major, [l][len], so
// that each column is contiguous.
//
// Kernels (gfx950, fp64 on the vector ALU; every contraction has l <= 256 on
// one side, far below an MFMA tile's reuse, and the passes over W and W0 are
// bound by the fp64 FMA rate, not by HBM):
// * k_band_mean: sum in fp64 (exact for bf16 and fp32 inputs), one division,
//   one rounding to the storage type (via round-to-odd, so no double rounding);
// * k_lsq_scale: one wave per row, fp64 dot products, butterfly reduction;
// * k_contract<LJ, ...>: C[i][j] = sum_t A(t, i) B(t, j) over 64 x LJ output
//   tiles, t in slices of 32 staged in LDS, each thread a 4 x LJ/16 register
//   block -- R Omega^T, R^T Q (over N ranges, fp64 partials, then a fold),
//   Gram matrices M^T M, M R^{-1}, and the final U and Vt;
// * orth(M) is Cholesky QR applied twice (CholQR2): G = M^T M, G = L L^T,
//   M <- M L^{-T}; twice, so that the basis is orthonormal to working
//   precision.  A column whose remaining norm vanishes (rank deficiency) is
//   dropped (zeroed) instead of divided by zero;
// * k_chol_inv: Cholesky and the triangular inverse in one workgroup, both
//   triangles packed in LDS (k_chol_inv_global above l = 128);
// * k_jacobi_lds / k_jacobi_block / k_jacobi_grid: the symmetric
//   eigendecomposition of B B^T (l x l) by cyclic Jacobi, rotations of
//   disjoint pairs in parallel (round-robin ordering), sorted descending;
//   S = sqrt of the eigenvalues.  One workgroup with G and V in LDS up to
//   l = 96; above, the block version (64 x 64 subproblems in LDS, block
//   updates of G and V in global memory, two grid barriers per round of
//   block pairs); the scalar version over many workgroups (one grid barrier
//   per round of index pairs) on request.
// Where l = N (the full SVD of a matrix with at most as many rows as
// columns), Q = I and B = R; where l = K the subspace steps are skipped (the
// first basis already spans R's range).

#include <math.h>

#include <type_traits>

#include "aq_internal.h"
#include "device_common.h"

namespace aq {

namespace {

template <typename T>
__device__ __forceinline__ double load_el(const T *p, size_t i);
template <>
__device__ __forceinline__ double load_el<uint16_t>(const uint16_t *p, size_t i) {
  return (double)bf2f(p[i]);
}
template <>
__device__ __forceinline__ double load_el<float>(const float *p, size_t i) {
  return (double)p[i];
}

// float64 -> bf16 bits, round to nearest even in one step: round to odd onto
// the fp32 grid first (24 >= 8 + 2 bits, so the second rounding is exact).
__device__ __forceinline__ uint16_t d2bf(double x) {
  float f = (float)x;
  if (fabs((double)f) > fabs(x)) f = __int_as_float(__float_as_int(f) - 1);
  if ((double)f != x) f = __int_as_float(__float_as_int(f) | 1);
  return f2bf(f);
}

}  // namespace

// ---------------------------------------------------------------- band mean

struct BandArgs {
  const void *W[kMaxBandLayers];
  int L;
  long n;
  void *out;
};

template <typename T>
__global__ __launch_bounds__(256) void k_band_mean(const BandArgs a) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < a.n; i += (long)gridDim.x * 256) {
    double sum = 0.0;
    for (int l = 0; l < a.L; ++l) sum += load_el((const T *)a.W[l], (size_t)i);
    const double m = sum / a.L;
    if constexpr (std::is_same<T, uint16_t>::value)
      ((uint16_t *)a.out)[i] = d2bf(m);
    else
      ((float *)a.out)[i] = (float)m;
  }
}

// ---------------------------------------------------------------- least squares

template <typename T>
__global__ __launch_bounds__(256) void k_lsq_scale(const T *W, const T *W0, long N, int K, double *s) {
  const int lane = threadIdx.x & 63;
  const long n = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  double num = 0.0, den = 0.0;
  for (int k = lane; k < K; k += 64) {
    const double w = load_el(W, (size_t)n * K + k), w0 = load_el(W0, (size_t)n * K + k);
    num = fma(w, w0, num);
    den = fma(w0, w0, den);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    num += __shfl_xor(num, o);
    den += __shfl_xor(den, o);
  }
  if (lane == 0) s[n] = den == 0.0 ? 1.0 : num / den;
}

// ---------------------------------------------------------------- contractions

// C[i][j] = sum over t of A(t, i) B(t, j) for a 64 x LJ output tile (i0 ..,
// all j < LJ), t from tbeg to tend in slices of 32 staged in LDS.  fillA /
// fillB stage a slice ([32][64] / [32][LJ], zeros out of range) with the
// access order that is coalesced for their operand; store(i, j, v) writes one
// result.  256 threads: thread (ti, tj) = (tid % 16, tid / 16) owns i = ti +
// 16 a (a < 4) and j = tj + 16 b (b < LJ / 16).
template <int LJ, class FA, class FB, class FS>
__device__ __forceinline__ void contract(int i0, int tbeg, int tend, const FA &fillA, const FB &fillB,
                                         const FS &store) {
  constexpr int TT = 32, TI = 64, JB = LJ / 16;
  __shared__ double As[TT][TI + 1];
  __shared__ double Bs[TT][LJ + 1];
  const int tid = threadIdx.x, ti = tid & 15, tj = tid >> 4;
  double acc[4][JB];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < JB; ++b) acc[a][b] = 0.0;
  for (int t0 = tbeg; t0 < tend; t0 += TT) {
    __syncthreads();
    fillA(As, t0, i0, tend);
    fillB(Bs, t0, tend);
    __syncthreads();
#pragma unroll 4
    for (int tt = 0; tt < TT; ++tt) {
      double av[4], bv[JB];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = As[tt][ti + 16 * a];
#pragma unroll
      for (int b = 0; b < JB; ++b) bv[b] = Bs[tt][tj + 16 * b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < JB; ++b) acc[a][b] = fma(av[a], bv[b], acc[a][b]);
    }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < JB; ++b) store(i0 + ti + 16 * a, tj + 16 * b, acc[a][b]);
}

// Stage of R[n][k] = W[n][k] - s[n] W0[n][k] as As[t][i] with t = k (R x M).
template <typename T>
struct FillR_tk {
  const T *W, *W0;
  const double *s;
  long N;
  int K;
  __device__ void operator()(double (*As)[65], int t0, int i0, int tend) const {
    // 64 rows x 32 K values: thread -> row tid / 4, 8 consecutive K values
    const int row = threadIdx.x >> 2, kc = (threadIdx.x & 3) * 8;
    const long n = (long)i0 + row;
    const double sn = n < N ? s[n] : 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = t0 + kc + e;
      double v = 0.0;
      if (n < N && k < tend) v = fma(-sn, load_el(W0, (size_t)n * K + k), load_el(W, (size_t)n * K + k));
      As[kc + e][row] = v;
    }
  }
};

// Stage of R[n][k] as As[t][i] with t = n (R^T x M).
template <typename T>
struct FillR_nt {
  const T *W, *W0;
  const double *s;
  int K;
  __device__ void operator()(double (*As)[65], int t0, int i0, int tend) const {
    // 32 rows x 64 K values: thread -> row tid / 8, 8 consecutive K values
    const int row = threadIdx.x >> 3, kc = (threadIdx.x & 7) * 8;
    const long n = (long)t0 + row;
    const double sn = n < tend ? s[n] : 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = i0 + kc + e;
      double v = 0.0;
      if (n < tend && k < K) v = fma(-sn, load_el(W0, (size_t)n * K + k), load_el(W, (size_t)n * K + k));
      As[row][kc + e] = v;
    }
  }
};

// Stage of a column-major tall matrix Mt[j][t] (j < l) as [t][j] (B side) or,
// with the roles of the axes swapped, Mt[t][i] as [t][i] (A side).
template <int LJ>
struct FillColsB {            // Bs[t][j] = Mt[j][t0 + t]
  const double *Mt;
  long ld;
  int l;
  __device__ void operator()(double (*Bs)[LJ + 1], int t0, int tend) const {
    for (int idx = threadIdx.x; idx < LJ * 32; idx += 256) {
      const int j = idx >> 5, t = idx & 31;
      Bs[t][j] = (j < l && t0 + t < tend) ? Mt[(size_t)j * ld + t0 + t] : 0.0;
    }
  }
};
template <int LJ>
struct FillRowsB {            // Bs[t][j] = S[t0 + t][j] (small row-major matrix, row stride ld)
  const double *S;
  int ld, ncol;
  __device__ void operator()(double (*Bs)[LJ + 1], int t0, int tend) const {
    for (int idx = threadIdx.x; idx < LJ * 32; idx += 256) {
      const int t = idx / LJ, j = idx - t * LJ;
      Bs[t][j] = (j < ncol && t0 + t < tend) ? S[(size_t)(t0 + t) * ld + j] : 0.0;
    }
  }
};
struct FillRowsA {            // As[t][i] = Mt[t0 + t][i0 + i] (row-major [t][len])
  const double *Mt;
  long ld, len;
  __device__ void operator()(double (*As)[65], int t0, int i0, int tend) const {
    for (int idx = threadIdx.x; idx < 32 * 64; idx += 256) {
      const int t = idx >> 6, i = idx & 63;
      As[t][i] = (t0 + t < tend && i0 + i < len) ? Mt[(size_t)(t0 + t) * ld + i0 + i] : 0.0;
    }
  }
};
struct FillColsA {            // As[t][i] = Mt[i0 + i][t0 + t] (row-major [i][t]: the Gram's A side)
  const double *Mt;
  long ld;
  int ni;
  __device__ void operator()(double (*As)[65], int t0, int i0, int tend) const {
    for (int idx = threadIdx.x; idx < 32 * 64; idx += 256) {
      const int i = idx >> 5, t = idx & 31;
      As[t][i] = (i0 + i < ni && t0 + t < tend) ? Mt[(size_t)(i0 + i) * ld + t0 + t] : 0.0;
    }
  }
};

// partial p of Y^T[j][n] = sum_{k in range p} R[n][k] X^T[j][k]   (R X, X
// given as X^T [l][K]; one range: Y^T itself)
template <int LJ, typename T>
__global__ __launch_bounds__(256) void k_rmul(const T *W, const T *W0, const double *s, long N, int K,
                                              const double *Xt, int l, int kchunk, double *Yp) {
  const int i0 = blockIdx.x * 64, p = blockIdx.y;
  const int kb = p * kchunk, ke = kb + kchunk < K ? kb + kchunk : K;
  double *Y = Yp + (size_t)p * l * N;
  contract<LJ>(i0, kb, ke, FillR_tk<T>{W, W0, s, N, K}, FillColsB<LJ>{Xt, K, l},
               [&](int i, int j, double v) {
                 if (i < N && j < l) Y[(size_t)j * N + i] = v;
               });
}

// partial p of Z^T[j][k] = sum_{n in range p} R[n][k] Q^T[j][n]   (R^T Q)
template <int LJ, typename T>
__global__ __launch_bounds__(256) void k_rtmul(const T *W, const T *W0, const double *s, long N, int K,
                                               const double *Qt, int l, long nchunk, double *Zp) {
  const int i0 = blockIdx.x * 64, p = blockIdx.y;
  const long nb = (long)p * nchunk, ne = nb + nchunk < N ? nb + nchunk : N;
  double *Z = Zp + (size_t)p * l * K;
  contract<LJ>(i0, (int)nb, (int)ne, FillR_nt<T>{W, W0, s, K}, FillColsB<LJ>{Qt, N, l},
               [&](int i, int j, double v) {
                 if (i < K && j < l) Z[(size_t)j * K + i] = v;
               });
}

// partial p of G[a][b] = sum_{t in range p} M^T[a][t] M^T[b][t]   (M^T M)
template <int LJ>
__global__ __launch_bounds__(256) void k_gram(const double *Mt, long len, int l, long tchunk, double *Gp) {
  const int i0 = blockIdx.x * 64, p = blockIdx.y;
  const long tb = (long)p * tchunk, te = tb + tchunk < len ? tb + tchunk : len;
  double *G = Gp + (size_t)p * l * l;
  contract<LJ>(i0, (int)tb, (int)te, FillColsA{Mt, len, l}, FillColsB<LJ>{Mt, len, l},
               [&](int i, int j, double v) {
                 if (i < l && j < l) G[(size_t)i * l + j] = v;
               });
}

// Out^T[j][i] = sum_a M^T[a][i] S[a][j]  (M S for a tall M and a small S [l][ncol]);
// with transpose_out the result is written row-major, Out[i][j] (the final U).
template <int LJ>
__global__ __launch_bounds__(256) void k_small_right(const double *Mt, long len, int l, const double *S, int ncol,
                                                     double *out, int transpose_out) {
  const int i0 = blockIdx.x * 64;
  contract<LJ>(i0, 0, l, FillRowsA{Mt, len, len}, FillRowsB<LJ>{S, ncol, ncol},
               [&](int i, int j, double v) {
                 if (i < len && j < ncol) {
                   if (transpose_out)
                     out[(size_t)i * ncol + j] = v;
                   else
                     out[(size_t)j * len + i] = v;
                 }
               });
}

// out[i] = sum over p < S of part[p][i], in order
__global__ __launch_bounds__(256) void k_fold_parts(const double *part, int S, long n, double *out) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    double v = 0.0;
    for (int p = 0; p < S; ++p) v += part[(size_t)p * n + i];
    out[i] = v;
  }
}

// ---------------------------------------------------------------- small factorizations

// LDS of the one-workgroup Jacobi (doubles): G and V, n x n each, up to n = 96.
constexpr int kSmallLds = 18432;
__device__ __host__ __forceinline__ bool two_fit(int n) { return 2 * n * n <= kSmallLds; }
// Packed lower triangles in LDS (row i, column k <= i at i (i + 1) / 2 + k).
constexpr int kTriLmax = 128, kTriMax = kTriLmax * (kTriLmax + 1) / 2;
__device__ __forceinline__ int tri(int i) { return i * (i + 1) / 2; }
constexpr int kCholThreads = 1024, kCholTpr = kCholThreads / kTriLmax;   // threads per row
constexpr int kCholBatch = 4;   // updates of one thread with all their loads before any store

// G = L L^T (Cholesky, lower L), then Rinv = L^{-T} (upper): Q = M Rinv.  A
// pivot at or below 1e-24 of its column's original square norm (a column that
// adds no direction, or a zero column) gives a zero column of L and of Rinv.
//
// One workgroup, l <= 128: both triangles packed in LDS, right-looking.  Once
// column j of L is final, every entry below and to its right takes its update
// from it at once (kCholTpr threads per row, alternate columns).  Entry (i, k)
// still receives its updates in the order j = 0, 1, ..., k - 1, one fma each,
// as in the column-by-column form; the inverse likewise (row k of L^{-1} is
// final once its update from row k - 1 is in, then rows below take theirs).
// A thread's updates of one step touch other entries than the ones they read
// (column j, row k), so kCholBatch of them load before any stores.
__global__ __launch_bounds__(kCholThreads) void k_chol_inv(const double *G, int l, double *Rinv) {
  __shared__ double A[kTriMax];     // G's lower triangle, then L (diagonal in Ld)
  __shared__ double X[kTriMax];     // the identity, then L^{-1} (lower)
  __shared__ double g0[kTriLmax], Ld[kTriLmax];
  const int tid = threadIdx.x, row = tid / kCholTpr, h = tid % kCholTpr;
  const bool mine = row < l;
  const int trow = tri(row);
  if (mine) {
    for (int k = h; k <= row; k += kCholTpr) {
      A[trow + k] = G[(size_t)row * l + k];
      X[trow + k] = row == k ? 1.0 : 0.0;
    }
    if (h == 0) g0[row] = G[(size_t)row * l + row];
  }
  __syncthreads();
  for (int j = 0; j < l; ++j) {
    const double dj = A[tri(j) + j];
    const bool ok = dj > 1e-24 * g0[j] && dj > 0.0;
    const double rj = ok ? sqrt(dj) : 0.0;
    if (mine && h == 0 && row >= j) {
      if (row == j) Ld[j] = rj;
      else A[trow + j] = ok ? A[trow + j] / rj : 0.0;
    }
    __syncthreads();
    if (mine && row > j) {
      const double lij = A[trow + j];
      for (int k0 = j + 1 + h; k0 <= row; k0 += kCholBatch * kCholTpr) {
        double lk[kCholBatch], ak[kCholBatch];
#pragma unroll
        for (int u = 0; u < kCholBatch; ++u) {
          const int k = k0 + u * kCholTpr;
          lk[u] = k <= row ? A[tri(k) + j] : 0.0;
          ak[u] = k <= row ? A[trow + k] : 0.0;
        }
#pragma unroll
        for (int u = 0; u < kCholBatch; ++u) {
          const int k = k0 + u * kCholTpr;
          if (k <= row) A[trow + k] = fma(-lij, lk[u], ak[u]);
        }
      }
    }
    __syncthreads();
  }
  for (int k = 0; k < l; ++k) {
    const double lkk = Ld[k];
    const int tk = tri(k);
    for (int c = tid; c <= k; c += kCholThreads) X[tk + c] = lkk != 0.0 ? X[tk + c] / lkk : 0.0;
    __syncthreads();
    if (mine && row > k) {
      const double lik = A[trow + k];
      for (int c0 = h; c0 <= k; c0 += kCholBatch * kCholTpr) {
        double xk[kCholBatch], xr[kCholBatch];
#pragma unroll
        for (int u = 0; u < kCholBatch; ++u) {
          const int c = c0 + u * kCholTpr;
          xk[u] = c <= k ? X[tk + c] : 0.0;
          xr[u] = c <= k ? X[trow + c] : 0.0;
        }
#pragma unroll
        for (int u = 0; u < kCholBatch; ++u) {
          const int c = c0 + u * kCholTpr;
          if (c <= k) X[trow + c] = fma(-lik, xk[u], xr[u]);
        }
      }
    }
    __syncthreads();
  }
  for (int idx = tid; idx < l * l; idx += kCholThreads) {
    const int c = idx / l, i = idx - c * l;
    Rinv[idx] = i >= c ? X[tri(i) + c] : 0.0;
  }
}

// The same for l > 128, with L in `scratch` and the inverse built in Rinv
// (global memory, l x l doubles each): column-by-column Cholesky, then forward
// substitution, one column of the inverse per thread.
__global__ __launch_bounds__(256) void k_chol_inv_global(const double *G, int l, double *Rinv, double *L) {
  __shared__ double tmp[256];
  const int tid = threadIdx.x;
  for (int idx = tid; idx < l * l; idx += 256) L[idx] = 0.0;
  __syncthreads();
  for (int j = 0; j < l; ++j) {
    if (tid >= j && tid < l) {
      double t = G[(size_t)tid * l + j];
      for (int k = 0; k < j; ++k) t = fma(-L[tid * l + k], L[j * l + k], t);
      tmp[tid] = t;
    }
    __syncthreads();
    const double dj = tmp[j];
    const bool ok = dj > 1e-24 * G[(size_t)j * l + j] && dj > 0.0;
    const double rj = ok ? sqrt(dj) : 0.0;
    if (tid >= j && tid < l) L[tid * l + j] = ok ? (tid == j ? rj : tmp[tid] / rj) : 0.0;
    __syncthreads();
  }
  // Rinv[c][i] = L^{-1}[i][c], read back by the thread that wrote it
  if (tid < l) {
    const int c = tid;
    for (int i = 0; i < l; ++i) {
      double v = 0.0;
      if (i >= c) {
        const double lii = L[i * l + i];
        double t = i == c ? 1.0 : 0.0;
        for (int k = c; k < i; ++k) t = fma(-L[i * l + k], Rinv[(size_t)c * l + k], t);
        v = lii != 0.0 ? t / lii : 0.0;
      }
      Rinv[(size_t)c * l + i] = v;
    }
  }
}

// Symmetric eigendecomposition of G (l x l) by cyclic Jacobi.  A sweep is
// n - 1 rounds (n = l rounded up to even, with a zero row and column for a
// dummy index when l is odd); in a round the indices form n / 2 disjoint pairs
// (the round-robin schedule: one index fixed, the others moving one place per
// round, so that every pair meets once per sweep), each pair's rotation is
// taken from the round's G, and G <- J^T G J, V <- V J for all of them at
// once -- each 2 x 2 block of G (rows of pair i, columns of pair j) is rotated
// on both sides by one thread.  Sweeps repeat until no pair had an
// off-diagonal entry above 1e-15 of sqrt(|G_pp G_qq|), at most 40.  Then the
// eigenvalues are sorted descending (ties by position) and, for the r leading
// ones, sigma = sqrt(max(lambda, 0)) gives Wu[a][c] = V[a][c] sigma_c and
// Wv[a][c] = V[a][c] / sigma_c (0 where sigma_c <= 1e-15 sigma_0).

// The rotation that zeroes G_pq: tau = (G_qq - G_pp) / (2 G_pq),
// t = sign(tau) / (|tau| + sqrt(1 + tau^2)), c = 1 / sqrt(1 + t^2), s = t c;
// the identity where G_pq = 0.  `big`: G_pq is above the convergence bound.
__device__ __forceinline__ void jacobi_angle(double gpp, double gqq, double gpq, double &c, double &s, bool &big) {
  c = 1.0;
  s = 0.0;
  big = false;
  if (gpq != 0.0) {
    big = fabs(gpq) > 1e-15 * sqrt(fabs(gpp * gqq));
    const double tau = (gqq - gpp) / (2.0 * gpq);
    const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
    c = 1.0 / sqrt(1.0 + t * t);
    s = t * c;
  }
}

// One 2 x 2 block of J^T G J: rows (p_i, q_i) by (ci, si) -- new row p =
// c row p - s row q, new row q = s row p + c row q -- then columns (p_j, q_j)
// by (cj, sj) the same way.
__device__ __forceinline__ void rot_block(double &a00, double &a01, double &a10, double &a11, double ci, double si,
                                          double cj, double sj) {
  const double r00 = ci * a00 - si * a10, r01 = ci * a01 - si * a11;
  const double r10 = si * a00 + ci * a10, r11 = si * a01 + ci * a11;
  a00 = cj * r00 - sj * r01;
  a01 = sj * r00 + cj * r01;
  a10 = cj * r10 - sj * r11;
  a11 = sj * r10 + cj * r11;
}

// Eigenvalues lam[0..n) (the dummy at -inf), eigenvectors V(a, i) = vec(a, i):
// the sorted outputs.  One workgroup of NT threads; rank_of has room for n.
template <int NT, class VecAt>
__device__ __forceinline__ void jacobi_outputs(int l, int n, int r, double *lam, int *rank_of, VecAt vec,
                                               double *lam_out, double *Wu, double *Wv) {
  const int tid = threadIdx.x;
  for (int i = tid; i < n; i += NT) {
    int rk = 0;
    for (int j = 0; j < n; ++j) rk += (lam[j] > lam[i] || (lam[j] == lam[i] && j < i)) ? 1 : 0;
    rank_of[i] = rk;
    if (rk < l) lam_out[rk] = lam[i];
  }
  __syncthreads();
  double lmax = 0.0;
  for (int j = 0; j < n; ++j) lmax = lam[j] > lmax ? lam[j] : lmax;
  const double smax = sqrt(lmax);
  for (int idx = tid; idx < l * n; idx += NT) {
    const int a = idx / n, i = idx - a * n, c = rank_of[i];
    if (c >= r) continue;
    const double sg = sqrt(lam[i] > 0.0 ? lam[i] : 0.0);
    const double v = vec(a, i);
    Wu[(size_t)a * r + c] = v * sg;
    Wv[(size_t)a * r + c] = sg > 1e-15 * smax && sg > 0.0 ? v / sg : 0.0;
  }
}

// One workgroup of 1024 threads, G and V in LDS (n <= 96).  Each thread owns
// up to three blocks of G and five (pair, coordinate) entries of V for the
// whole run; pairs are looked up per round.
constexpr int kJacLdsMaxN = 96, kJacLdsB = 3, kJacLdsV = 5;
static_assert((kJacLdsMaxN / 2) * (kJacLdsMaxN / 2) <= kJacLdsB * 1024, "G blocks per thread");
static_assert((kJacLdsMaxN / 2) * kJacLdsMaxN <= kJacLdsV * 1024, "V entries per thread");
__global__ __launch_bounds__(1024) void k_jacobi_lds(const double *Gin, int l, int r, double *lam_out, double *Wu,
                                                    double *Wv) {
  __shared__ double S[kSmallLds];
  __shared__ double cs[kJacLdsMaxN / 2], sn[kJacLdsMaxN / 2];
  __shared__ int pp[kJacLdsMaxN / 2], qq[kJacLdsMaxN / 2];
  __shared__ int changed;
  __shared__ double lam[kJacLdsMaxN];
  __shared__ int rank_of[kJacLdsMaxN];
  const int n = l + (l & 1), np = n / 2, tid = threadIdx.x;
  double *G = S, *V = S + n * n;   // G[a][b]; V[a][i] = coordinate a of eigenvector i
  for (int idx = tid; idx < n * n; idx += 1024) {
    const int a = idx / n, b = idx - a * n;
    G[idx] = a < l && b < l ? Gin[(size_t)a * l + b] : 0.0;
    V[idx] = a == b ? 1.0 : 0.0;
  }
  int bi[kJacLdsB], bj[kJacLdsB], vi[kJacLdsV], va[kJacLdsV];
#pragma unroll
  for (int u = 0; u < kJacLdsB; ++u) {
    const int b = tid + u * 1024;
    bi[u] = b < np * np ? b / np : -1;
    bj[u] = b - (b / np) * np;
  }
#pragma unroll
  for (int u = 0; u < kJacLdsV; ++u) {
    const int e = tid + u * 1024;
    vi[u] = e < np * l ? e / l : -1;
    va[u] = e - (e / l) * l;
  }
  __syncthreads();
  for (int sweep = 0; sweep < 40; ++sweep) {
    if (tid == 0) changed = 0;
    __syncthreads();
    for (int round = 0; round < n - 1; ++round) {
      if (tid < np) {
        auto player = [&](int x) { return x == 0 ? 0 : ((x - 1 + round) % (n - 1)) + 1; };
        int p = player(tid), q = player(n - 1 - tid);
        if (p > q) {
          const int t = p;
          p = q;
          q = t;
        }
        double c, s;
        bool big;
        jacobi_angle(G[p * n + p], G[q * n + q], G[p * n + q], c, s, big);
        if (big) changed = 1;
        cs[tid] = c;
        sn[tid] = s;
        pp[tid] = p;
        qq[tid] = q;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kJacLdsB; ++u) {
        if (bi[u] < 0) continue;
        const int i = bi[u], j = bj[u];
        const int pi = pp[i], qi = qq[i], pj = pp[j], qj = qq[j];
        double a00 = G[pi * n + pj], a01 = G[pi * n + qj], a10 = G[qi * n + pj], a11 = G[qi * n + qj];
        rot_block(a00, a01, a10, a11, cs[i], sn[i], cs[j], sn[j]);
        G[pi * n + pj] = a00;
        G[pi * n + qj] = a01;
        G[qi * n + pj] = a10;
        G[qi * n + qj] = a11;
      }
#pragma unroll
      for (int u = 0; u < kJacLdsV; ++u) {
        if (vi[u] < 0) continue;
        const int i = vi[u], a = va[u], p = pp[i], q = qq[i];
        const double c = cs[i], s = sn[i], vp = V[a * n + p], vq = V[a * n + q];
        V[a * n + p] = c * vp - s * vq;
        V[a * n + q] = s * vp + c * vq;
      }
      __syncthreads();
    }
    if (!changed) break;
    __syncthreads();
  }
  for (int i = tid; i < n; i += 1024) lam[i] = i < l ? G[i * n + i] : -INFINITY;
  __syncthreads();
  jacobi_outputs<1024>(l, n, r, lam, rank_of, [&](int a, int i) { return V[a * n + i]; }, lam_out, Wu, Wv);
}

// Many workgroups, for n > 96: G and the eigenvectors in global memory, in
// the order of the round-robin slots (the pairs of a round are the slots
// (k, n - 1 - k), so the 2 x 2 blocks of a row of pairs are read as four
// contiguous runs), ping-pong buffers: each round reads one copy and writes
// the rotated matrix to the other at the slots its indices move to (slot 0
// stays, slot s moves to s + 1 within 1 .. n - 1).  Every workgroup computes
// all of a round's rotations from the same data (so they take the same
// convergence decision without exchanging it); one grid barrier per round.
struct JacobiGrid {
  const double *Gin;
  int l, r;
  double *g[2], *v[2];      // [n][n] each; v row = slot of the eigenvector, column = coordinate
  unsigned *ctr;            // barrier arrivals, zero at launch
  unsigned *flag;           // the workspace's give-up word
  int spin;                 // polls before a barrier wait gives up
  int extra;                // arrivals awaited beyond the grid's (a host-forced give-up)
  double *lam_out, *Wu, *Wv;
};
constexpr int kJacGridMaxWgs = 64;
constexpr unsigned kGridAbort = 1u << 31;   // set in the counter by a give-up (arrivals stay far below)

// Stores read by other workgroups after the barrier: device-coherent.
__device__ __forceinline__ void store_coherent(double *p, double v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long *>(p), (unsigned long long)__double_as_longlong(v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Barrier of the grid (at most kJacGridMaxWgs workgroups of 256 threads, all
// resident at once).  Every wave's stores complete, one release arrival per
// workgroup, a bounded poll, an acquire at agent scope.  A workgroup whose
// poll runs out sets bit kGridAbort (which releases every other waiter at
// once) and the flag word; false from then on, in every workgroup.
__device__ bool grid_barrier(unsigned *ctr, unsigned *flag, int spin, unsigned target, int *s_ok) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    unsigned v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int it = 0; v < target && it < spin; ++it) {
      __builtin_amdgcn_s_sleep(1);
      v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    bool ok = v >= target && v < kGridAbort;
    if (v < target) {
      __hip_atomic_fetch_or(ctr, kGridAbort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_or(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *s_ok = ok;
  }
  __syncthreads();
  return *s_ok != 0;
}
__device__ __forceinline__ bool grid_barrier(const JacobiGrid &a, unsigned target, int *s_ok) {
  return grid_barrier(a.ctr, a.flag, a.spin, target, s_ok);
}

__global__ __launch_bounds__(256) void k_jacobi_grid(const JacobiGrid a) {
  __shared__ double cs[kDecompMaxL / 2], sn[kDecompMaxL / 2];
  __shared__ int s_changed, s_ok;
  __shared__ double lam[kDecompMaxL];
  __shared__ int rank_of[kDecompMaxL];
  const int l = a.l, n = l + (l & 1), np = n / 2, nn = n * n;
  const int tid = threadIdx.x, nb = gridDim.x;
  const int gt = blockIdx.x * 256 + tid, gs = nb * 256;
  auto next = [&](int s) { return s == 0 ? 0 : (s == n - 1 ? 1 : s + 1); };
  for (int e = gt; e < nn; e += gs) {
    const int x = e / n, y = e - x * n;
    store_coherent(a.g[0] + e, x < l && y < l ? a.Gin[(size_t)x * l + y] : 0.0);
    store_coherent(a.v[0] + e, x == y ? 1.0 : 0.0);
  }
  // this thread's first block of G and first two entries of V (the default
  // grid has no others): loaded each round together with the angles' inputs,
  // so that a round costs one trip to memory
  const int nblk = np * np, nv = np * l;
  const bool hb = gt < nblk, hv0 = gt < nv, hv1 = gt + gs < nv;
  const int bi = hb ? gt / np : 0, bj = gt - bi * np;
  const int vi0 = hv0 ? gt / l : 0, vx0 = gt - vi0 * l;
  const int vi1 = hv1 ? (gt + gs) / l : 0, vx1 = gt + gs - vi1 * l;
  unsigned passed = 1;
  bool ok = grid_barrier(a, passed * nb + a.extra, &s_ok);
  int cur = 0, rounds = 0;
  for (int sweep = 0; ok && sweep < 40; ++sweep) {
    if (tid == 0) s_changed = 0;
    __syncthreads();
    for (int round = 0; ok && round < n - 1; ++round) {
      const double *gc = a.g[cur], *vc = a.v[cur];
      double *gn = a.g[cur ^ 1], *vn = a.v[cur ^ 1];
      double a00 = 0.0, a01 = 0.0, a10 = 0.0, a11 = 0.0, vp0 = 0.0, vq0 = 0.0, vp1 = 0.0, vq1 = 0.0;
      if (hb) {
        a00 = gc[bi * n + bj];
        a01 = gc[bi * n + n - 1 - bj];
        a10 = gc[(n - 1 - bi) * n + bj];
        a11 = gc[(n - 1 - bi) * n + n - 1 - bj];
      }
      if (hv0) {
        vp0 = vc[vi0 * n + vx0];
        vq0 = vc[(n - 1 - vi0) * n + vx0];
      }
      if (hv1) {
        vp1 = vc[vi1 * n + vx1];
        vq1 = vc[(n - 1 - vi1) * n + vx1];
      }
      if (tid < np) {
        const int p = tid, q = n - 1 - tid;
        double c, s;
        bool big;
        jacobi_angle(gc[p * n + p], gc[q * n + q], gc[p * n + q], c, s, big);
        if (big) s_changed = 1;
        cs[tid] = c;
        sn[tid] = s;
      }
      __syncthreads();
      auto put_block = [&](int i, int j, double b00, double b01, double b10, double b11) {
        rot_block(b00, b01, b10, b11, cs[i], sn[i], cs[j], sn[j]);
        const int npi = next(i), nqi = next(n - 1 - i), npj = next(j), nqj = next(n - 1 - j);
        store_coherent(gn + npi * n + npj, b00);
        store_coherent(gn + npi * n + nqj, b01);
        store_coherent(gn + nqi * n + npj, b10);
        store_coherent(gn + nqi * n + nqj, b11);
      };
      auto put_v = [&](int i, int x, double vp, double vq) {
        const double c = cs[i], s = sn[i];
        store_coherent(vn + next(i) * n + x, c * vp - s * vq);
        store_coherent(vn + next(n - 1 - i) * n + x, s * vp + c * vq);
      };
      if (hb) put_block(bi, bj, a00, a01, a10, a11);
      for (int b = gt + gs; b < nblk; b += gs) {   // grids smaller than the default
        const int i = b / np, j = b - i * np;
        put_block(i, j, gc[i * n + j], gc[i * n + n - 1 - j], gc[(n - 1 - i) * n + j],
                  gc[(n - 1 - i) * n + n - 1 - j]);
      }
      if (hv0) put_v(vi0, vx0, vp0, vq0);
      if (hv1) put_v(vi1, vx1, vp1, vq1);
      for (int e = gt + 2 * gs; e < nv; e += gs) {
        const int i = e / l, x = e - i * l;
        put_v(i, x, vc[i * n + x], vc[(n - 1 - i) * n + x]);
      }
      ++passed;
      ok = grid_barrier(a, passed * nb + a.extra, &s_ok);
      cur ^= 1;
      ++rounds;
    }
    if (!s_changed) break;
  }
  if (blockIdx.x != 0) return;
  if (!ok) {   // a barrier gave up: no valid result
    for (int idx = tid; idx < l * a.r; idx += 256) a.Wu[idx] = a.Wv[idx] = __builtin_nan("");
    for (int i = tid; i < l; i += 256) a.lam_out[i] = __builtin_nan("");
    return;
  }
  const double *gc = a.g[cur], *vc = a.v[cur];
  // index l (the dummy, odd l) started at slot n - 1 and moved one slot per round
  const int dummy = (l & 1) ? 1 + (n - 2 + rounds) % (n - 1) : -1;
  for (int i = tid; i < n; i += 256) lam[i] = i == dummy ? -INFINITY : gc[i * n + i];
  __syncthreads();
  jacobi_outputs<256>(l, n, a.r, lam, rank_of, [&](int x, int i) { return vc[i * n + x]; }, a.lam_out, a.Wu,
                      a.Wv);
}

// Block Jacobi, for 96 < l <= 256 (the default there): the index range, padded
// to n = 64 ceil(l / 64) with zero rows and columns (which no rotation ever
// touches: their off-diagonal entries stay exactly zero), is cut into blocks
// of 32; a round pairs the blocks round-robin (block 0 fixed, the others
// moving one place per round) into nsets = n / 64 sets of 64 indices.  Phase
// A: workgroup k runs one cyclic Jacobi sweep (the rotations of jacobi_angle,
// round-robin pairs, 63 rounds) on the 64 x 64 submatrix G[I_k, I_k] in LDS
// and accumulates its rotations into J_k (J <- J R, the update of V).
// Phase B: G[I_k, I_m] <- J_k^T G[I_k, I_m] J_m for every pair of sets and
// V[:, I_k] <- V[:, I_k] J_k, one 64 x 64 block per workgroup.  A sweep is the
// nb - 1 rounds in which every pair of blocks meets once; sweeps repeat until
// no rotation of a sweep met an off-diagonal entry above the bound (the
// scalar one, and an absolute floor below), at most 40.  Two grid barriers
// per round (instead of one per scalar round).
struct JacobiBlock {
  const double *Gin;
  int l, r, n;              // n: the padded size (a multiple of 64, at most 256)
  double *G, *V, *J;        // G, V: [n][n] (V[a][i]: coordinate a of eigenvector i); J: [nsets][64][64]
  unsigned *ctr;            // ctr[0]: barrier arrivals; ctr[1 + s % 3]: a rotation of sweep s was big
  unsigned *flag;
  int spin, extra;
  double *lam_out, *Wu, *Wv;
};

// LDS layouts: the phase-A submatrix with rows of 65 doubles (rows of a
// rotation pair fall in different banks) and J transposed (the columns p, q
// that a rotation updates are contiguous rows).  1024 threads: one 2 x 2 block
// of the submatrix and two entries of J per thread per scalar round, a 2 x 2
// output tile per thread in the block products.
constexpr int kJbA = 65;
__global__ __launch_bounds__(1024) void k_jacobi_block(const JacobiBlock a) {
  __shared__ __attribute__((aligned(16))) double A[64 * kJbA];
  __shared__ __attribute__((aligned(16))) double B1[64 * 64];
  __shared__ __attribute__((aligned(16))) double B2[64 * 64];
  __shared__ double cs[32], sn[32];
  __shared__ int pp[32], qq[32];
  __shared__ int s_big, s_ok;
  __shared__ double s_floor;
  __shared__ double lam[kDecompMaxL];
  __shared__ int rank_of[kDecompMaxL];
  const int l = a.l, n = a.n, nb = n / 32, nsets = nb / 2;
  const int tid = threadIdx.x, wg = blockIdx.x, nwg = gridDim.x;
  const int gt = wg * 1024 + tid, gs = nwg * 1024;
  for (int e = gt; e < n * n; e += gs) {
    const int x = e / n, y = e - x * n;
    store_coherent(a.G + e, x < l && y < l ? a.Gin[(size_t)x * l + y] : 0.0);
    store_coherent(a.V + e, x == y ? 1.0 : 0.0);
  }
  // The block updates recompute every entry as a 64-term sum, which leaves an
  // absolute error of order eps max|G| on each: an off-diagonal entry counts
  // as big only above 2^-43 (~1.1e-13) of the largest diagonal entry as well,
  // so that entries between two small eigenvalues, held at that noise level,
  // do not keep the sweeps going to their bound.
  if (tid < 64) {
    double m = 0.0;
    for (int i = tid; i < l; i += 64) m = fmax(m, fabs(a.Gin[(size_t)i * l + i]));
    for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o));
    if (tid == 0) s_floor = 0x1p-43 * m;
  }
  unsigned passed = 1;
  bool ok = grid_barrier(a.ctr, a.flag, a.spin, passed * nwg + a.extra, &s_ok);
  const double floor_big = s_floor;
  // this thread's 2 x 2 output tile of a 64 x 64 block product
  const int ti = tid >> 5, tj = tid & 31;
  for (int sweep = 0; ok && sweep < 40; ++sweep) {
    if (wg == 0 && tid == 0)   // last read at the end of sweep - 2
      __hip_atomic_store(a.ctr + 1 + (sweep + 1) % 3, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int round = 0; ok && round < nb - 1; ++round) {
      auto bplayer = [&](int x) { return x == 0 ? 0 : ((x - 1 + round) % (nb - 1)) + 1; };
      // global index of local index i (0..63) of set k
      auto gidx = [&](int k, int i) { return i < 32 ? 32 * bplayer(k) + i : 32 * bplayer(nb - 1 - k) + i - 32; };
      if (wg < nsets) {   // ---- phase A: one sweep on G[I_k, I_k]
        const int k = wg;
        for (int e = tid; e < 64 * 64; e += 1024) {
          const int i = e >> 6, j = e & 63;
          A[i * kJbA + j] = a.G[(size_t)gidx(k, i) * n + gidx(k, j)];
          B1[e] = i == j ? 1.0 : 0.0;   // J^T
        }
        if (tid == 0) s_big = 0;
        __syncthreads();
        // this thread's 2 x 2 block (pair rows bi, pair columns bj) and its
        // two entries of J (pair vi, row x)
        const int bi = tid >> 5, bj = tid & 31, vi = tid >> 5, vx = (tid & 31) * 2;
        for (int rr = 0; rr < 63; ++rr) {
          if (tid < 32) {
            auto player = [&](int x) { return x == 0 ? 0 : ((x - 1 + rr) % 63) + 1; };
            int p = player(tid), q = player(63 - tid);
            if (p > q) {
              const int t = p;
              p = q;
              q = t;
            }
            double c, s;
            bool big;
            const double gpq = A[p * kJbA + q];
            jacobi_angle(A[p * kJbA + p], A[q * kJbA + q], gpq, c, s, big);
            if (big && fabs(gpq) > floor_big) s_big = 1;
            cs[tid] = c;
            sn[tid] = s;
            pp[tid] = p;
            qq[tid] = q;
          }
          __syncthreads();
          {
            const int pi = pp[bi], qi = qq[bi], pj = pp[bj], qj = qq[bj];
            double a00 = A[pi * kJbA + pj], a01 = A[pi * kJbA + qj], a10 = A[qi * kJbA + pj],
                   a11 = A[qi * kJbA + qj];
            rot_block(a00, a01, a10, a11, cs[bi], sn[bi], cs[bj], sn[bj]);
            A[pi * kJbA + pj] = a00;
            A[pi * kJbA + qj] = a01;
            A[qi * kJbA + pj] = a10;
            A[qi * kJbA + qj] = a11;
          }
          {   // J <- J R: columns p, q of J, i.e. rows p, q of J^T
            const int p = pp[vi], q = qq[vi];
            const double c = cs[vi], s = sn[vi];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const double vp = B1[p * 64 + vx + u], vq = B1[q * 64 + vx + u];
              B1[p * 64 + vx + u] = c * vp - s * vq;
              B1[q * 64 + vx + u] = s * vp + c * vq;
            }
          }
          __syncthreads();
        }
        for (int e = tid; e < 64 * 64; e += 1024) {   // J[x][i] = J^T[i][x]
          const int i = e >> 6, x = e & 63;
          store_coherent(a.J + (size_t)k * 4096 + x * 64 + i, B1[e]);
        }
        if (tid == 0 && s_big)
          __hip_atomic_fetch_or(a.ctr + 1 + sweep % 3, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      ++passed;
      ok = grid_barrier(a.ctr, a.flag, a.spin, passed * nwg + a.extra, &s_ok);
      if (!ok) break;
      // ---- phase B: one 64 x 64 block per workgroup (row stride 64 in LDS)
      const bool gtask = wg < nsets * nsets, vtask = !gtask && wg < 2 * nsets * nsets;
      if (gtask || vtask) {
        const int t = gtask ? wg : wg - nsets * nsets, k = t / nsets, m = t - k * nsets;
        // G task (k, m): A = G[I_k, I_m]; V task (k, c = m): A = V[rows 64 c .., I_k]
        for (int e = tid; e < 64 * 64; e += 1024) {
          const int i = e >> 6, j = e & 63;
          A[e] = gtask ? a.G[(size_t)gidx(k, i) * n + gidx(m, j)] : a.V[(size_t)(64 * m + i) * n + gidx(k, j)];
          B1[e] = a.J[(size_t)k * 4096 + e];
          if (gtask) B2[e] = a.J[(size_t)m * 4096 + e];
        }
        __syncthreads();
        double acc[2][2];
        auto product = [&](const double *L, bool ltrans, const double *Rm) {
          // acc = op(L) Rm over this thread's tile, op(L) = L^T where ltrans
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int v = 0; v < 2; ++v) acc[u][v] = 0.0;
          for (int x = 0; x < 64; ++x) {
            double lv[2], rv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) lv[u] = ltrans ? L[x * 64 + 2 * ti + u] : L[(2 * ti + u) * 64 + x];
#pragma unroll
            for (int v = 0; v < 2; ++v) rv[v] = Rm[x * 64 + 2 * tj + v];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
              for (int v = 0; v < 2; ++v) acc[u][v] = __builtin_fma(lv[u], rv[v], acc[u][v]);
          }
        };
        if (gtask) {
          product(B1, true, A);               // T = J_k^T A
          __syncthreads();
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int v = 0; v < 2; ++v) A[(2 * ti + u) * 64 + 2 * tj + v] = acc[u][v];
          __syncthreads();
          product(A, false, B2);              // T J_m
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int v = 0; v < 2; ++v)
              store_coherent(a.G + (size_t)gidx(k, 2 * ti + u) * n + gidx(m, 2 * tj + v), acc[u][v]);
        } else {
          product(A, false, B1);              // V[rows, I_k] J_k
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int v = 0; v < 2; ++v)
              store_coherent(a.V + (size_t)(64 * m + 2 * ti + u) * n + gidx(k, 2 * tj + v), acc[u][v]);
        }
      }
      ++passed;
      ok = grid_barrier(a.ctr, a.flag, a.spin, passed * nwg + a.extra, &s_ok);
    }
    if (!ok) break;
    if (__hip_atomic_load(a.ctr + 1 + sweep % 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) break;
  }
  if (wg != 0) return;
  if (!ok) {   // a barrier gave up: no valid result
    for (int idx = tid; idx < l * a.r; idx += 1024) a.Wu[idx] = a.Wv[idx] = __builtin_nan("");
    for (int i = tid; i < l; i += 1024) a.lam_out[i] = __builtin_nan("");
    return;
  }
  for (int i = tid; i < n; i += 1024) lam[i] = i < l ? a.G[(size_t)i * n + i] : -INFINITY;
  __syncthreads();
  jacobi_outputs<1024>(l, n, a.r, lam, rank_of, [&](int x, int i) { return a.V[(size_t)x * n + i]; }, a.lam_out,
                       a.Wu, a.Wv);
}

// Q = I as [l = N][N]
__global__ __launch_bounds__(256) void k_eye(double *Y, long N) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < N * N; i += (long)gridDim.x * 256)
    Y[i] = i / N == i % N ? 1.0 : 0.0;
}

__global__ void k_zero_u32(unsigned *p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// ---------------------------------------------------------------- host side

size_t decompose_ws_bytes(int64_t N, int64_t K, int64_t r, int64_t l, DecompPlan *pl) {
  pl->lj = l <= 32 ? 32 : (l <= 64 ? 64 : (l <= 80 ? 80 : (l <= 128 ? 128 : 256)));
  // R X: N tiles of 64 x K ranges (of >= 64 columns, multiples of 32), about
  // 256 workgroups
  {
    const long nt = (N + 63) / 64;
    long sk = (256 + nt - 1) / nt;
    sk = sk < K / 64 ? sk : K / 64;
    sk = sk < 32 ? sk : 32;
    sk = sk > 1 ? sk : 1;
    pl->kchunk = (int)(((K + sk - 1) / sk + 31) / 32 * 32);
    pl->srm = (int)((K + pl->kchunk - 1) / pl->kchunk);
  }
  // R^T Q: K tiles of 64 x N ranges (ranges of >= 256 rows), about 256 workgroups
  const long kt = (K + 63) / 64;
  long sr = (256 + kt - 1) / kt;
  const long srmax = (N + 255) / 256;
  sr = sr < srmax ? sr : srmax;
  sr = sr < 64 ? sr : 64;
  pl->srt = (int)(sr > 1 ? sr : 1);
  pl->nchunk = (N + pl->srt - 1) / pl->srt;
  // Gram sums: ranges of >= 32 rows, about 256 workgroups with the l tiles
  const long len = N > K ? N : K;
  long sg = (256 + (l + 63) / 64 - 1) / ((l + 63) / 64);
  sg = sg < (len + 31) / 32 ? sg : (len + 31) / 32;
  sg = sg < 128 ? sg : 128;
  pl->sgram = (int)(sg > 1 ? sg : 1);
  // the eigendecomposition: one workgroup with G and V in LDS where they fit
  // (n <= 96), else the block Jacobi (2 nsets^2 workgroups); the scalar grid
  // version (kJacGridMaxWgs workgroups at most) on request
  const int n = (int)(l + (l & 1));
  const int jk = debug_knob(AQ_DBG_JACOBI, 0);
  const bool lds = jk == 1 ? two_fit(n) : (jk == 2 || jk == 3 ? false : two_fit(n));
  pl->jac_block = !lds && jk != 2;
  pl->jac_n = (int)((l + 63) / 64 * 64);
  // grid version: one 2 x 2 block of G per thread (and at most two entries of
  // V), at most kJacGridMaxWgs workgroups (n = 256)
  const int np = n / 2, wdef = (np * np + 255) / 256;
  const int wk = debug_knob(AQ_DBG_JACOBI_WGS, wdef);
  const int nsets = pl->jac_n / 64;
  pl->jac_wgs = lds ? 0 : (pl->jac_block ? 2 * nsets * nsets : (wk >= 1 && wk <= kJacGridMaxWgs ? wk : wdef));
  pl->jac_spin = debug_knob(AQ_DBG_HANDOFF_SPIN, kHandoffSpin);
  pl->jac_extra = debug_knob(AQ_DBG_HANDOFF_UNREACHABLE, 0) ? 1 : 0;
  // after the reserved region: its counter words belong to the recon calls
  // that share the workspace and must stay zero
  size_t off = kWsReserved;
  auto take = [&](size_t nd) {
    const size_t o = off;
    off += (nd * 8 + 255) / 256 * 256;
    return o;
  };
  pl->o_y1 = take((size_t)l * N);
  pl->o_y2 = take((size_t)l * N);
  pl->o_z1 = take((size_t)l * K);
  pl->o_z2 = take((size_t)l * K);
  pl->o_zp = take((size_t)pl->srt * l * K);
  pl->o_yp = take(pl->srm > 1 ? (size_t)pl->srm * l * N : 1);
  pl->o_gp = take((size_t)pl->sgram * l * l);
  pl->o_g = take((size_t)l * l);
  pl->o_rinv = take((size_t)l * l);
  pl->o_scr = take((size_t)l * l);
  // the grid Jacobi's two copies of G and of V, or the block Jacobi's G, V and J
  const size_t jn = (size_t)pl->jac_n;
  const size_t jgrid = 4 * (size_t)n * n, jblock = 2 * jn * jn + (size_t)nsets * 4096;
  pl->o_jac = take(jgrid > jblock ? jgrid : jblock);
  pl->o_ctr = take(32);              // barrier counter (and the block version's sweep flags)
  pl->o_lam = take((size_t)l);
  pl->o_wu = take((size_t)l * (r > 0 ? r : 1));
  pl->o_wv = take((size_t)l * (r > 0 ? r : 1));
  return off;
}

template <int LJ, typename T>
static void run_decompose_t(const DecompArgs &d, const DecompPlan &pl, char *ws, hipStream_t st) {
  const T *W = (const T *)d.W, *W0 = (const T *)d.W0;
  const long N = d.N;
  const int K = (int)d.K, l = (int)d.l, r = (int)d.r;
  double *s = d.s;
  double *Y1 = (double *)(ws + pl.o_y1), *Y2 = (double *)(ws + pl.o_y2);
  double *Z1 = (double *)(ws + pl.o_z1), *Z2 = (double *)(ws + pl.o_z2), *Zp = (double *)(ws + pl.o_zp);
  double *Gp = (double *)(ws + pl.o_gp), *G = (double *)(ws + pl.o_g), *Rinv = (double *)(ws + pl.o_rinv);
  double *scr = (double *)(ws + pl.o_scr), *lam = (double *)(ws + pl.o_lam);
  double *Wu = (double *)(ws + pl.o_wu), *Wv = (double *)(ws + pl.o_wv);

  hipLaunchKernelGGL((k_lsq_scale<T>), dim3((unsigned)((N + 3) / 4)), dim3(256), 0, st, W, W0, N, K, s);
  if (r == 0) return;

  auto gram = [&](const double *Mt, long len) {
    const long tch = ((len + pl.sgram - 1) / pl.sgram + 31) / 32 * 32;
    const int sg = (int)((len + tch - 1) / tch);
    hipLaunchKernelGGL((k_gram<LJ>), dim3((unsigned)((l + 63) / 64), sg), dim3(256), 0, st, Mt, len, l, tch, Gp);
    const long nn = (long)l * l;
    hipLaunchKernelGGL(k_fold_parts, dim3((unsigned)((nn + 255) / 256)), dim3(256), 0, st, (const double *)Gp, sg,
                       nn, G);
  };
  // orth(M): CholQR twice; the result ends where it started (a <-> b)
  auto orth = [&](double *a, double *b, long len) {
    for (int pass = 0; pass < 2; ++pass) {
      double *src = pass == 0 ? a : b, *dst = pass == 0 ? b : a;
      gram(src, len);
      if (l <= kTriLmax)
        hipLaunchKernelGGL(k_chol_inv, dim3(1), dim3(kCholThreads), 0, st, (const double *)G, l, Rinv);
      else
        hipLaunchKernelGGL(k_chol_inv_global, dim3(1), dim3(256), 0, st, (const double *)G, l, Rinv, scr);
      hipLaunchKernelGGL((k_small_right<LJ>), dim3((unsigned)((len + 63) / 64)), dim3(256), 0, st,
                         (const double *)src, len, l, (const double *)Rinv, l, dst, 0);
    }
  };
  auto rmul = [&](const double *Xt, double *Yt) {
    double *Yp = pl.srm > 1 ? (double *)(ws + pl.o_yp) : Yt;
    hipLaunchKernelGGL((k_rmul<LJ, T>), dim3((unsigned)((N + 63) / 64), pl.srm), dim3(256), 0, st, W, W0,
                       (const double *)s, N, K, Xt, l, pl.kchunk, Yp);
    if (pl.srm > 1) {
      const long nn = (long)l * N;
      hipLaunchKernelGGL(k_fold_parts, dim3((unsigned)((nn + 255) / 256 < 4096 ? (nn + 255) / 256 : 4096)),
                         dim3(256), 0, st, (const double *)Yp, pl.srm, nn, Yt);
    }
  };
  auto rtmul = [&](const double *Qt, double *Zt) {
    hipLaunchKernelGGL((k_rtmul<LJ, T>), dim3((unsigned)((K + 63) / 64), pl.srt), dim3(256), 0, st, W, W0,
                       (const double *)s, N, K, Qt, l, pl.nchunk, Zp);
    const long nn = (long)l * K;
    hipLaunchKernelGGL(k_fold_parts, dim3((unsigned)((nn + 255) / 256 < 4096 ? (nn + 255) / 256 : 4096)), dim3(256),
                       0, st, (const double *)Zp, pl.srt, nn, Zt);
  };

  if (l == N) {
    // The probe is as wide as the column space: any orthonormal basis of R^N
    // spans R's range exactly, so Q = I (B = R) and no subspace step can
    // change the result.
    hipLaunchKernelGGL(k_eye, dim3((unsigned)((N * N + 255) / 256 < 4096 ? (N * N + 255) / 256 : 4096)), dim3(256),
                       0, st, Y1, N);
  } else {
    rmul(d.omega, Y1);               // Y = R Omega^T
    orth(Y1, Y2, N);                 // Q
    // where l = K the first Q already spans R's range (omega is K x K):
    // the subspace steps would return the same space
    const int q = l == K ? 0 : d.q;
    for (int it = 0; it < q; ++it) {
      rtmul(Y1, Z1);                 // R^T Q
      orth(Z1, Z2, K);
      rmul(Z1, Y1);                  // R Q~
      orth(Y1, Y2, N);
    }
  }
  rtmul(Y1, Z1);                     // B^T = R^T Q, i.e. B = Q^T R as [l][K]
  gram(Z1, K);                       // B B^T
  if (pl.jac_wgs == 0) {
    hipLaunchKernelGGL(k_jacobi_lds, dim3(1), dim3(1024), 0, st, (const double *)G, l, r, lam, Wu, Wv);
  } else if (pl.jac_block) {
    const size_t jn = (size_t)pl.jac_n;
    double *jac = (double *)(ws + pl.o_jac);
    JacobiBlock jb{};
    jb.Gin = G;
    jb.l = l;
    jb.r = r;
    jb.n = pl.jac_n;
    jb.G = jac;
    jb.V = jac + jn * jn;
    jb.J = jac + 2 * jn * jn;
    jb.ctr = (unsigned *)(ws + pl.o_ctr);
    jb.flag = (unsigned *)ws + kSyncFlag;
    jb.spin = pl.jac_spin;
    jb.extra = pl.jac_extra;
    jb.lam_out = lam;
    jb.Wu = Wu;
    jb.Wv = Wv;
    hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(64), 0, st, jb.ctr, 4);
    hipLaunchKernelGGL(k_jacobi_block, dim3((unsigned)pl.jac_wgs), dim3(1024), 0, st, jb);
  } else {
    const size_t n2 = (size_t)(l + (l & 1)) * (l + (l & 1));
    double *jac = (double *)(ws + pl.o_jac);
    JacobiGrid ja{};
    ja.Gin = G;
    ja.l = l;
    ja.r = r;
    ja.g[0] = jac;
    ja.g[1] = jac + n2;
    ja.v[0] = jac + 2 * n2;
    ja.v[1] = jac + 3 * n2;
    ja.ctr = (unsigned *)(ws + pl.o_ctr);
    ja.flag = (unsigned *)ws + kSyncFlag;
    ja.spin = pl.jac_spin;
    ja.extra = pl.jac_extra;
    ja.lam_out = lam;
    ja.Wu = Wu;
    ja.Wv = Wv;
    hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(64), 0, st, ja.ctr, 1);
    hipLaunchKernelGGL(k_jacobi_grid, dim3((unsigned)pl.jac_wgs), dim3(256), 0, st, ja);
  }
  // U [N][r] = Q (V_r S_r);  Vt [r][K] = (V_r S_r^-1)^T B
  hipLaunchKernelGGL((k_small_right<LJ>), dim3((unsigned)((N + 63) / 64)), dim3(256), 0, st, (const double *)Y1, N, l,
                     (const double *)Wu, r, d.U, 1);
  hipLaunchKernelGGL((k_small_right<LJ>), dim3((unsigned)((K + 63) / 64)), dim3(256), 0, st, (const double *)Z1,
                     (long)K, l, (const double *)Wv, r, d.Vt, 0);
}

hipError_t launch_decompose(const DecompArgs &d, const DecompPlan &pl, void *ws, hipStream_t st) {
  char *w = (char *)ws;
  const bool bf = d.dt == AQ_BF16;
  switch (pl.lj) {
    case 32: bf ? run_decompose_t<32, uint16_t>(d, pl, w, st) : run_decompose_t<32, float>(d, pl, w, st); break;
    case 64: bf ? run_decompose_t<64, uint16_t>(d, pl, w, st) : run_decompose_t<64, float>(d, pl, w, st); break;
    case 80: bf ? run_decompose_t<80, uint16_t>(d, pl, w, st) : run_decompose_t<80, float>(d, pl, w, st); break;
    case 128: bf ? run_decompose_t<128, uint16_t>(d, pl, w, st) : run_decompose_t<128, float>(d, pl, w, st); break;
    default: bf ? run_decompose_t<256, uint16_t>(d, pl, w, st) : run_decompose_t<256, float>(d, pl, w, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_band_mean(aq_dtype dt, int L, const void *const *W, int64_t n, void *out, hipStream_t st) {
  BandArgs a = {};
  for (int l = 0; l < L; ++l) a.W[l] = W[l];
  a.L = L;
  a.n = n;
  a.out = out;
  const long blocks = (n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192;
  if (dt == AQ_BF16)
    hipLaunchKernelGGL(k_band_mean<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_band_mean<float>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace aq
