// Stage 2: block summaries (mean of each block's valid tokens, in float64).
//
// [SPADE] "SPADE: An Input-Adaptive Sparse Attention Engine for Fast Video
// Diffusion Models Inference", abstract: dynamic masks are built from a
// Summarizer and an Estimator; the Summarizer here is the per-block mean.
//
// One workgroup per (b, h, block).  Lane groups stream whole 16-byte chunks of
// the block's contiguous rows (coalesced HBM reads), accumulate in float64,
// and a fixed-order LDS reduction combines the row groups.  Sums of bf16
// values are exact in float64 whenever the block's exponents span fewer than
// ~36 binades, so the result does not depend on the summation order.
#include "svsa_internal.h"

namespace svsa {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// kElt: 2 (bf16) or 4 (float32).  Each 16-byte chunk holds kPer elements.
template <int kElt>
__global__ void __launch_bounds__(kThreads)
pool_kernel(const uint4* __restrict__ x, double* __restrict__ out, int32_t head_dim, Geom g) {
  constexpr int kPer = 16 / kElt;
  extern __shared__ double red[];  // [groups][head_dim]
  const int32_t nb = g.nb;
  const int64_t bh = blockIdx.x / nb;
  const int32_t blk = blockIdx.x % nb;
  const int32_t n_valid = block_valid(g, blk);
  const int32_t chunks = head_dim / kPer;         // chunks per row
  const int32_t groups = kThreads / chunks;       // row groups
  const int32_t ch = threadIdx.x % chunks;
  const int32_t rg = threadIdx.x / chunks;
  const uint4* base = x + (bh * g.Npad + (int64_t)blk * g.Bk) * chunks;

  double acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.0;
  if (rg < groups) {
    for (int32_t r = rg; r < n_valid; r += groups) {
      const uint4 u = base[(int64_t)r * chunks + ch];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
      if (kElt == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += (double)bf16_lo(w[e]);
          acc[2 * e + 1] += (double)bf16_hi(w[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += (double)__uint_as_float(w[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) red[rg * head_dim + ch * kPer + e] = acc[e];
  }
  __syncthreads();
  const double inv_n = (double)n_valid;
  for (int32_t d = threadIdx.x; d < head_dim; d += kThreads) {
    double s = 0.0;
    for (int32_t r = 0; r < groups; ++r) s += red[r * head_dim + d];
    out[(bh * nb + blk) * head_dim + d] = s / inv_n;
  }
}

}  // namespace

hipError_t launch_pool(const void* x, bool is_bf16, double* out, int32_t bh, int32_t head_dim,
                       const Geom& g, hipStream_t stream) {
  const int elt = is_bf16 ? 2 : 4;
  const int32_t chunks = head_dim * elt / 16;
  if (chunks <= 0 || chunks > kThreads) return hipErrorInvalidValue;
  const int32_t groups = kThreads / chunks;
  const size_t lds = (size_t)groups * head_dim * sizeof(double);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)bh * g.nb;
  if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (is_bf16) {
    hipLaunchKernelGGL(pool_kernel<2>, dim3((uint32_t)blocks), dim3(kThreads), lds, stream,
                       (const uint4*)x, out, head_dim, g);
  } else {
    hipLaunchKernelGGL(pool_kernel<4>, dim3((uint32_t)blocks), dim3(kThreads), lds, stream,
                       (const uint4*)x, out, head_dim, g);
  }
  return hipGetLastError();
}

}  // namespace svsa
