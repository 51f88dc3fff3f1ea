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
// * k_chol_inv: Cholesky and the triangular inverse in one workgroup;
// * k_jacobi: the symmetric eigendecomposition of B B^T (l x l) by cyclic
//   Jacobi in one workgroup of 1024 threads, rotations of disjoint pairs in parallel
//   (round-robin ordering), sorted descending; S = sqrt of the eigenvalues.

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

// Y^T[j][n] = sum_k R[n][k] X^T[j][k]   (R X, X given as X^T [l][K])
template <int LJ, typename T>
__global__ __launch_bounds__(256) void k_rmul(const T *W, const T *W0, const double *s, long N, int K,
                                              const double *Xt, int l, double *Yt) {
  const int i0 = blockIdx.x * 64;
  contract<LJ>(i0, 0, K, FillR_tk<T>{W, W0, s, N, K}, FillColsB<LJ>{Xt, K, l},
               [&](int i, int j, double v) {
                 if (i < N && j < l) Yt[(size_t)j * N + i] = v;
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

// G = L L^T (Cholesky, lower L), then Rinv = L^{-T} (upper): Q = M Rinv.  A
// pivot at or below 1e-24 of its column's original square norm (a column that
// adds no direction, or a zero column) gives a zero column of L and of Rinv.
// One workgroup; L in LDS for l <= 128, else in `scratch` (l x l doubles).
__global__ __launch_bounds__(256) void k_chol_inv(const double *G, int l, double *Rinv, double *scratch) {
  __shared__ double Ls[128 * 128];
  __shared__ double tmp[256];
  double *L = l <= 128 ? Ls : scratch;
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
  // X = L^{-1} by forward substitution, one column c per thread; written as
  // Rinv[c][i] = X[i][c] (so Rinv = X^T) and read back by the same thread.
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

// Symmetric eigendecomposition of G (l x l) by cyclic Jacobi: per round, the
// disjoint pairs of a round-robin schedule are rotated in parallel (rotation
// angles from the round's G, then all row rotations, then all column
// rotations and the eigenvector updates); sweeps until no pair has an
// off-diagonal entry above 1e-15 of sqrt(|G_pp G_qq|), at most 40.  Then the
// eigenvalues are sorted descending and, for the r leading ones, sigma =
// sqrt(max(lambda, 0)) gives Wu[a][c] = V[a][c] sigma_c and Wv[a][c] = V[a][c] /
// sigma_c (0 where sigma_c <= 1e-15 sigma_0).  One workgroup; G in LDS for
// l <= 128, else in `gscr`; V in `vscr` (both l x l doubles).
constexpr int kJacobiBatch = 8;
__global__ __launch_bounds__(1024) void k_jacobi(const double *Gin, int l, int r, double *gscr, double *vscr,
                                                double *lam_out, double *Wu, double *Wv) {
  __shared__ double Gs[128 * 128];
  __shared__ double cs[128], sn[128];
  __shared__ int pp[128], qq[128];
  __shared__ int changed;
  __shared__ double lam[256];
  __shared__ int rank_of[256];
  double *G = l <= 128 ? Gs : gscr;
  double *V = vscr;
  const int tid = threadIdx.x, NT = 1024;
  for (int idx = tid; idx < l * l; idx += NT) {
    G[idx] = Gin[idx];
    V[idx] = (idx / l == idx % l) ? 1.0 : 0.0;
  }
  const int n = l + (l & 1);   // even, with a dummy index l when l is odd
  const int np = n / 2;
  __syncthreads();
  for (int sweep = 0; sweep < 40; ++sweep) {
    if (tid == 0) changed = 0;
    __syncthreads();
    for (int round = 0; round < n - 1; ++round) {
      if (tid < np) {
        auto player = [&](int x) { return x == 0 ? 0 : ((x - 1 + round) % (n - 1)) + 1; };
        int p = player(tid), q = player(n - 1 - tid);
        if (p > q) { const int t = p; p = q; q = t; }
        double c = 1.0, s = 0.0;
        if (q < l) {
          const double gpq = G[p * l + q], gpp = G[p * l + p], gqq = G[q * l + q];
          if (gpq != 0.0) {
            if (fabs(gpq) > 1e-15 * sqrt(fabs(gpp * gqq))) changed = 1;
            const double tau = (gqq - gpp) / (2.0 * gpq);
            const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
            c = 1.0 / sqrt(1.0 + t * t);
            s = t * c;
          }
        }
        cs[tid] = c;
        sn[tid] = s;
        pp[tid] = p;
        qq[tid] = q < l ? q : -1;
      }
      __syncthreads();
      // rows p and q of every pair: G <- J^T G.  Eight updates per thread at a
      // time, all their loads before any store (the updates touch disjoint
      // elements), so that G in global memory costs one round trip per eight.
      for (int base = tid; base < np * l; base += NT * kJacobiBatch) {
        double gp[kJacobiBatch], gq[kJacobiBatch];
#pragma unroll
        for (int u = 0; u < kJacobiBatch; ++u) {
          const int idx = base + u * NT;
          const int m = idx / l, col = idx - m * l;
          const bool ok = idx < np * l && qq[m < np ? m : 0] >= 0;
          gp[u] = ok ? G[pp[m] * l + col] : 0.0;
          gq[u] = ok ? G[qq[m] * l + col] : 0.0;
        }
#pragma unroll
        for (int u = 0; u < kJacobiBatch; ++u) {
          const int idx = base + u * NT;
          const int m = idx / l, col = idx - m * l;
          if (idx >= np * l || qq[m] < 0) continue;
          const double c = cs[m], s = sn[m];
          G[pp[m] * l + col] = c * gp[u] - s * gq[u];
          G[qq[m] * l + col] = s * gp[u] + c * gq[u];
        }
      }
      __syncthreads();
      // columns p and q: G <- G J, V <- V J (batched the same way)
      for (int base = tid; base < np * l; base += NT * kJacobiBatch) {
        double gp[kJacobiBatch], gq[kJacobiBatch], vp[kJacobiBatch], vq[kJacobiBatch];
#pragma unroll
        for (int u = 0; u < kJacobiBatch; ++u) {
          const int idx = base + u * NT;
          const int m = idx / l, row = idx - m * l;
          const bool ok = idx < np * l && qq[m < np ? m : 0] >= 0;
          gp[u] = ok ? G[row * l + pp[m]] : 0.0;
          gq[u] = ok ? G[row * l + qq[m]] : 0.0;
          vp[u] = ok ? V[row * l + pp[m]] : 0.0;
          vq[u] = ok ? V[row * l + qq[m]] : 0.0;
        }
#pragma unroll
        for (int u = 0; u < kJacobiBatch; ++u) {
          const int idx = base + u * NT;
          const int m = idx / l, row = idx - m * l;
          if (idx >= np * l || qq[m] < 0) continue;
          const double c = cs[m], s = sn[m];
          G[row * l + pp[m]] = c * gp[u] - s * gq[u];
          G[row * l + qq[m]] = s * gp[u] + c * gq[u];
          V[row * l + pp[m]] = c * vp[u] - s * vq[u];
          V[row * l + qq[m]] = s * vp[u] + c * vq[u];
        }
      }
      __syncthreads();
    }
    if (!changed) break;
    __syncthreads();
  }
  // sort descending (rank = number of larger eigenvalues, ties by index)
  if (tid < l) lam[tid] = G[tid * l + tid];
  __syncthreads();
  if (tid < l) {
    int rk = 0;
    for (int j = 0; j < l; ++j) rk += (lam[j] > lam[tid] || (lam[j] == lam[tid] && j < tid)) ? 1 : 0;
    rank_of[tid] = rk;
    lam_out[rk] = lam[tid];
  }
  __syncthreads();
  double lmax = 0.0;
  for (int j = 0; j < l; ++j) lmax = lam[j] > lmax ? lam[j] : lmax;
  const double smax = sqrt(lmax);
  for (int idx = tid; idx < l * l; idx += NT) {
    const int a = idx / l, i = idx - a * l, c = rank_of[i];
    if (c >= r) continue;
    const double sg = sqrt(lam[i] > 0.0 ? lam[i] : 0.0);
    const double v = V[a * l + i];
    Wu[(size_t)a * r + c] = v * sg;
    Wv[(size_t)a * r + c] = sg > 1e-15 * smax && sg > 0.0 ? v / sg : 0.0;
  }
}

// ---------------------------------------------------------------- host side

size_t decompose_ws_bytes(int64_t N, int64_t K, int64_t r, int64_t l, DecompPlan *pl) {
  pl->lj = l <= 32 ? 32 : (l <= 64 ? 64 : (l <= 128 ? 128 : 256));
  // R^T Q: K tiles of 64 x N ranges (ranges of >= 256 rows), about 256 workgroups
  const long kt = (K + 63) / 64;
  long sr = (256 + kt - 1) / kt;
  const long srmax = (N + 255) / 256;
  sr = sr < srmax ? sr : srmax;
  sr = sr < 64 ? sr : 64;
  pl->srt = (int)(sr > 1 ? sr : 1);
  pl->nchunk = (N + pl->srt - 1) / pl->srt;
  const long len = N > K ? N : K;
  long sg = (len + 511) / 512;
  sg = sg < 128 ? sg : 128;
  pl->sgram = (int)(sg > 1 ? sg : 1);
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
  pl->o_gp = take((size_t)pl->sgram * l * l);
  pl->o_g = take((size_t)l * l);
  pl->o_rinv = take((size_t)l * l);
  pl->o_scr = take((size_t)l * l);
  pl->o_v = take((size_t)l * l);
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
  double *scr = (double *)(ws + pl.o_scr), *V = (double *)(ws + pl.o_v), *lam = (double *)(ws + pl.o_lam);
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
      hipLaunchKernelGGL(k_chol_inv, dim3(1), dim3(256), 0, st, (const double *)G, l, Rinv, scr);
      hipLaunchKernelGGL((k_small_right<LJ>), dim3((unsigned)((len + 63) / 64)), dim3(256), 0, st,
                         (const double *)src, len, l, (const double *)Rinv, l, dst, 0);
    }
  };
  auto rmul = [&](const double *Xt, double *Yt) {
    hipLaunchKernelGGL((k_rmul<LJ, T>), dim3((unsigned)((N + 63) / 64)), dim3(256), 0, st, W, W0, (const double *)s,
                       N, K, Xt, l, Yt);
  };
  auto rtmul = [&](const double *Qt, double *Zt) {
    hipLaunchKernelGGL((k_rtmul<LJ, T>), dim3((unsigned)((K + 63) / 64), pl.srt), dim3(256), 0, st, W, W0,
                       (const double *)s, N, K, Qt, l, pl.nchunk, Zp);
    const long nn = (long)l * K;
    hipLaunchKernelGGL(k_fold_parts, dim3((unsigned)((nn + 255) / 256 < 4096 ? (nn + 255) / 256 : 4096)), dim3(256),
                       0, st, (const double *)Zp, pl.srt, nn, Zt);
  };

  rmul(d.omega, Y1);                 // Y = R Omega^T
  orth(Y1, Y2, N);                   // Q
  for (int it = 0; it < d.q; ++it) {
    rtmul(Y1, Z1);                   // R^T Q
    orth(Z1, Z2, K);
    rmul(Z1, Y1);                    // R Q~
    orth(Y1, Y2, N);
  }
  rtmul(Y1, Z1);                     // B^T = R^T Q, i.e. B = Q^T R as [l][K]
  gram(Z1, K);                       // B B^T
  hipLaunchKernelGGL(k_jacobi, dim3(1), dim3(1024), 0, st, (const double *)G, l, r, scr, V, lam, Wu, Wv);
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
