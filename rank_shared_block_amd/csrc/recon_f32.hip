// fp32 reconstruction for any batch size: fp32 storage and fp32 arithmetic.
//
//     y[m, col_b + n] = s_b[n] * (x[m] . W0_b[n]) + sum_j U_b[n, j] * t[m, j],
//     t[m, j] = x[m] . Vt_b[j]
// ("How attnquant works", section "The reconstruction identity").
//
// The fp32 path is the precision reference of the library (small shapes, tight
// tolerance), not a throughput path: one workgroup owns 16 tokens x 16 output
// columns of one block, first computes t for its 16 tokens into LDS (every column
// of the tile reuses it), then each thread accumulates one output with fp32 FMAs
// in K order.

#include "aq_internal.h"
#include "device_common.h"

namespace aq {

struct F32Blk {
  const float *W0, *s, *U, *Vt;
  int N, r, col, tile0;
};

struct F32Args {
  const float *x;
  float *y;
  int ldx, ldy, M, K, nblk, ntiles;
  F32Blk b[kMaxBlocks];
};

__global__ __launch_bounds__(256) void k_recon_f32(const F32Args a) {
  __shared__ float ts[16 * AQ_MAX_RANK];
  const int tile = blockIdx.x;
  if (tile >= a.ntiles) return;
  int bi = 0;
  if (a.nblk > 1 && tile >= a.b[1].tile0) bi = 1;
  if (a.nblk > 2 && tile >= a.b[2].tile0) bi = 2;
  const F32Blk B = bi == 0 ? a.b[0] : (bi == 1 ? a.b[1] : a.b[2]);
  const int n0 = (tile - B.tile0) * 16, m0 = blockIdx.y * 16;
  const int tid = threadIdx.x, K = a.K, r = B.r;

  for (int e = tid; e < 16 * r; e += 256) {
    const int mi = e / r, j = e - mi * r, m = m0 + mi;
    float acc = 0.f;
    if (m < a.M) {
      const float *xr = a.x + (size_t)m * a.ldx;
      const float *vr = B.Vt + (size_t)j * K;
      for (int k = 0; k < K; ++k) acc = fmaf(xr[k], vr[k], acc);
    }
    ts[mi * AQ_MAX_RANK + j] = acc;
  }
  __syncthreads();

  const int mi = tid >> 4, ni = tid & 15;
  const int m = m0 + mi, n = n0 + ni;
  if (m >= a.M || n >= B.N) return;
  const float *xr = a.x + (size_t)m * a.ldx;
  const float *wr = B.W0 + (size_t)n * K;
  float z = 0.f;
  for (int k = 0; k < K; ++k) z = fmaf(xr[k], wr[k], z);
  float lr = 0.f;
  const float *ur = B.U + (size_t)n * r;
  for (int j = 0; j < r; ++j) lr = fmaf(ur[j], ts[mi * AQ_MAX_RANK + j], lr);
  a.y[(size_t)m * a.ldy + B.col + n] = fmaf(B.s[n], z, lr);
}

hipError_t launch_recon_f32(const Recon &rq, hipStream_t st) {
  F32Args a = {};
  a.x = (const float *)rq.x;
  a.y = (float *)rq.y;
  a.ldx = (int)rq.ldx;
  a.ldy = (int)rq.ldy;
  a.M = (int)rq.M;
  a.K = (int)rq.K;
  a.nblk = rq.nblk;
  int t0 = 0;
  for (int b = 0; b < rq.nblk; ++b) {
    const Proj &P = rq.blk[b];
    F32Blk &d = a.b[b];
    d.W0 = (const float *)P.W0;
    d.s = (const float *)P.s;
    d.U = (const float *)P.U;
    d.Vt = (const float *)P.Vt;
    d.N = (int)P.N;
    d.r = (int)P.r;
    d.col = (int)P.col;
    d.tile0 = t0;
    t0 += (int)((P.N + 15) / 16);
  }
  a.ntiles = t0;
  dim3 grid(t0, (unsigned)((rq.M + 15) / 16));
  hipLaunchKernelGGL(k_recon_f32, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace aq
