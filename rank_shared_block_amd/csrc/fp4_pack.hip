// Block-16 FP4 pack of a bf16 effective weight.
//
// Container: "Internals and extension", section "Nvfp4Spec" (two E2M1 codes per
// byte, one FP8-E4M3 scale per 16 K-values in the linear [N, K/16] layout, one
// fp32 global scale); "Execution paths", section "Precompute-outside" quantises
// each W_eff at load.  The recipe (the pages give only the container):
//   g     = RN_f32(A / 2688), A = max|w| (g = 1 when A == 0)
//   scale = E4M3FN(max|block| / (6 g)), round to nearest even, saturating at 448
//   D     = RN_f32(g * scale)
//   code  = E2M1 nearest to |w| / D, ties to the even code, saturating at 6;
//           sign bit only on non-zero codes; all zero when D == 0
//   byte  = code[2i] | code[2i+1] << 4
//
// Two passes over HBM:
//   1. amax: max |w| per workgroup as an integer max over the 15 magnitude bits
//      of the bf16 patterns (exact and order-independent); partials to ws.
//   2. pack: every wave folds the partials to A (1 KB from L2), derives g,
//      and packs one 16-value block per thread (2 x 16-byte loads, one 8-byte
//      store of codes, one scale byte).
//
// Exactness without a per-element division: the block-scale quotient is formed
// by a correctly rounded fp64 division (which cannot cross an E4M3 rounding
// boundary: the quotient of an 8-bit by a <= 26-bit significand is either exactly
// a midpoint or far from every midpoint relative to fp64's precision), and the
// element codes come from comparing |w| with the seven E2M1 midpoints times D,
// exactly: per block, each product is rounded to fp32 and its rounding error
// (an fma) decides whether the fp32 threshold is the product or the next float
// above it (products exact in fp64 where D is too small for that).  Equality
// with a midpoint selects the even code.

#include "aq_internal.h"
#include "device_common.h"
#include "fp4_block.h"

namespace aq {

__global__ __launch_bounds__(256) void k_fp4_amax(const uint16_t *w, int N, int K, int ldw,
                                                  unsigned *partial) {
  const int k8 = K >> 3;
  const long nchunks = (long)N * k8;
  unsigned m = 0;
  // Four 16-byte chunks per thread per step, all requested before any is used.
  const long stride = (long)gridDim.x * 256;
  for (long c0 = (long)blockIdx.x * 256 + threadIdx.x; c0 < nchunks; c0 += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long c = c0 + u * stride;
      const long n = c / k8;
      const int kk = (int)(c - n * k8) * 8;
      v[u] = c < nchunks ? ld16(w + n * ldw + kk) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t q[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m = max(m, q[i] & 0x7FFFu);
        m = max(m, (q[i] >> 16) & 0x7FFFu);
      }
    }
  }
  __shared__ unsigned red[256];
  red[threadIdx.x] = m;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void k_fp4_pack(const uint16_t *w, int N, int K, int ldw,
                                                  const unsigned *partial, int npartial,
                                                  uint8_t *packed, uint8_t *scales,
                                                  float *gscale) {
  // Every wave folds the (at most 256) partial maxima itself: four loads per
  // lane requested together, then a butterfly over the wave; no LDS and no
  // workgroup barrier before the packing starts.
  const int lane = threadIdx.x & 63;
  unsigned pm[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = lane + 64 * q;
    pm[q] = partial[i < npartial ? i : 0];
  }
  unsigned m = max(max(pm[0], pm[1]), max(pm[2], pm[3]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, o));
  const float A = bf2f((uint16_t)m);
  const float g = A == 0.f ? 1.0f : (float)((double)A / 2688.0);
  if (blockIdx.x == 0 && threadIdx.x == 0) *gscale = g;

  const int kb = K >> 4;
  const long nblocks = (long)N * kb;
  for (long blk = (long)blockIdx.x * 256 + threadIdx.x; blk < nblocks; blk += (long)gridDim.x * 256) {
    const long n = blk / kb;
    const int b = (int)(blk - n * kb);
    const uint16_t *src = w + n * ldw + b * 16;
    const uint4 v0 = ld16(src), v1 = ld16(src + 8);
    const uint32_t q[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t lo, hi, sf;
    pack_block16(q, g, lo, hi, sf);
    *reinterpret_cast<uint2 *>(packed + n * (K >> 1) + b * 8) = make_uint2(lo, hi);
    scales[n * kb + b] = (uint8_t)sf;
  }
}

hipError_t launch_fp4(int64_t N, int64_t K, const void *w, int64_t ldw, uint8_t *packed,
                      uint8_t *scales, float *gscale, void *ws_base, hipStream_t st) {
  void *ws = (char *)ws_base + kWsReserved;     // leave the counter region untouched
  const long nchunks = (long)N * (K / 8);
  int g1 = (int)((nchunks + 255) / 256);
  g1 = g1 < kNumCU ? g1 : kNumCU;               // <= 256 partials (the pack folds them per wave)
  hipLaunchKernelGGL(k_fp4_amax, dim3(g1), dim3(256), 0, st, (const uint16_t *)w, (int)N,
                     (int)K, (int)ldw, (unsigned *)ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long nblocks = (long)N * (K / 16);
  long g2 = (nblocks + 255) / 256;
  g2 = g2 < 8L * kNumCU * 4 ? g2 : 8L * kNumCU * 4;
  hipLaunchKernelGGL(k_fp4_pack, dim3((unsigned)g2), dim3(256), 0, st, (const uint16_t *)w,
                     (int)N, (int)K, (int)ldw, (const unsigned *)ws, g1, packed, scales, gscale);
  return hipGetLastError();
}

// ---- many weights per launch (load time) ----------------------------------------
//
// A work unit is 256 x BPT consecutive 16-value blocks of one weight (BPT per
// thread, all 2 BPT 16-byte loads requested before any is used).  The
// global scale of each weight comes from amax[] (its largest magnitude as bf16
// bits): from the batched materialisation, which folds it in while writing
// W_eff, or from k_fp4_amax_batch over the weights here.  The encoding is
// pack_block16, as for one weight, so the bytes are identical.
struct Fp4BItem {
  const uint16_t *w;
  uint8_t *packed, *scales;
  float *gscale;
  int N, K, ldw, unit0;
};
struct Fp4BatchArgs {
  int nitem, nunits, amax0, pad;
  unsigned *amax;
  Fp4BItem item[kFp4BatchItems];
};
static_assert(sizeof(Fp4BatchArgs) <= 3584, "kernel arguments stay well inside 4 KiB");

__device__ __forceinline__ int fp4b_item(const Fp4BatchArgs &a, int unit) {
  int i = 0;
  for (int j = 1; j < a.nitem; ++j)
    if (unit >= a.item[j].unit0) i = j;
  return i;
}

// Loads of the BPT blocks of this thread (zeros past the weight).
template <int BPT>
__device__ __forceinline__ void fp4b_load(const Fp4BItem &I, long b0, uint4 (&v)[2 * BPT], long (&blk)[BPT]) {
  const int kb = I.K >> 4;
  const long nblocks = (long)I.N * kb;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    blk[j] = b0 + 256 * j + threadIdx.x;
    if (blk[j] < nblocks) {
      const long n = blk[j] / kb;
      const uint16_t *src = I.w + n * I.ldw + (blk[j] - n * kb) * 16;
      v[2 * j] = ld16(src);
      v[2 * j + 1] = ld16(src + 8);
    } else {
      v[2 * j] = v[2 * j + 1] = make_uint4(0, 0, 0, 0);
      blk[j] = -1;
    }
  }
}

template <int BPT>
__global__ __launch_bounds__(256) void k_fp4_amax_batch(const Fp4BatchArgs a) {
  const int unit = (int)blockIdx.x;
  const int ii = fp4b_item(a, unit);
  const Fp4BItem &I = a.item[ii];
  uint4 v[2 * BPT];
  long blk[BPT];
  fp4b_load<BPT>(I, (long)(unit - I.unit0) * 256 * BPT, v, blk);
  unsigned m = 0;
#pragma unroll
  for (int j = 0; j < 2 * BPT; ++j) {
    const uint32_t q[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, max(q[i] & 0x7FFFu, (q[i] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, o));
  __shared__ unsigned red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(a.amax + a.amax0 + ii, max(max(red[0], red[1]), max(red[2], red[3])));
}

template <int BPT>
__global__ __launch_bounds__(256) void k_fp4_pack_batch(const Fp4BatchArgs a) {
  const int unit = (int)blockIdx.x;
  const int ii = fp4b_item(a, unit);
  const Fp4BItem &I = a.item[ii];
  uint4 v[2 * BPT];
  long blk[BPT];
  const long b0 = (long)(unit - I.unit0) * 256 * BPT;
  fp4b_load<BPT>(I, b0, v, blk);
  const float g = fp4_global_scale(a.amax[a.amax0 + ii]);
  if (b0 == 0 && threadIdx.x == 0) *I.gscale = g;
  const int kb = I.K >> 4;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    if (blk[j] < 0) continue;
    const uint32_t q[8] = {v[2 * j].x, v[2 * j].y, v[2 * j].z, v[2 * j].w,
                           v[2 * j + 1].x, v[2 * j + 1].y, v[2 * j + 1].z, v[2 * j + 1].w};
    uint32_t lo, hi, sf;
    pack_block16(q, g, lo, hi, sf);
    const long n = blk[j] / kb, b = blk[j] - n * kb;
    *reinterpret_cast<uint2 *>(I.packed + n * (I.K >> 1) + b * 8) = make_uint2(lo, hi);
    I.scales[n * kb + b] = (uint8_t)sf;
  }
}

__global__ __launch_bounds__(256) void k_fp4_fill_u32(unsigned *p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

size_t fp4_batch_ws_bytes(int n, bool have_amax) {
  return have_amax ? 0 : kWsReserved + ((size_t)n * 4 + 255) / 256 * 256;
}

hipError_t launch_fp4_batch(int n, const Fp4Item *it, const unsigned *amax_in, void *ws, hipStream_t st) {
  unsigned *amax = const_cast<unsigned *>(amax_in);
  const bool own = amax == nullptr;
  if (own) {
    amax = (unsigned *)((char *)ws + kWsReserved);
    hipLaunchKernelGGL(k_fp4_fill_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, amax, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int bpt = debug_knob(AQ_DBG_FP4_UNIT, 2);
  if (bpt != 1 && bpt != 2 && bpt != 4 && bpt != 8) bpt = 2;
  const int unit_blocks = 256 * bpt;
  for (int pass = own ? 0 : 1; pass < 2; ++pass) {
    for (int i0 = 0; i0 < n; i0 += kFp4BatchItems) {
      Fp4BatchArgs a = {};
      a.amax = amax;
      a.amax0 = i0;
      int units = 0;
      for (int i = i0; i < n && a.nitem < kFp4BatchItems; ++i) {
        Fp4BItem &I = a.item[a.nitem++];
        I.w = (const uint16_t *)it[i].w;
        I.packed = it[i].packed;
        I.scales = it[i].scales;
        I.gscale = it[i].gscale;
        I.N = (int)it[i].N;
        I.K = (int)it[i].K;
        I.ldw = (int)it[i].ldw;
        I.unit0 = units;
        const long nblocks = it[i].N * (it[i].K / 16);
        units += (int)((nblocks + unit_blocks - 1) / unit_blocks);
      }
      a.nunits = units;
      const dim3 grid((unsigned)units);
#define AQ_FP4B(B)                                                                     \
  if (bpt == B) {                                                                      \
    if (pass == 0)                                                                     \
      hipLaunchKernelGGL(k_fp4_amax_batch<B>, grid, dim3(256), 0, st, a);              \
    else                                                                               \
      hipLaunchKernelGGL(k_fp4_pack_batch<B>, grid, dim3(256), 0, st, a);              \
  }
      AQ_FP4B(1)
      AQ_FP4B(2)
      AQ_FP4B(4)
      AQ_FP4B(8)
#undef AQ_FP4B
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace aq
