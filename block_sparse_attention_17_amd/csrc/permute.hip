// Stage 1: tile reorder of (T,H,W) tokens (and its inverse).
//
// [PSA] "Parameterized Stripe Attention for Efficient Video Generation",
// Sec. 3.2: Q, K, V are reorganised from (T,H,W) into a block-centric layout
// so that each block's tokens are contiguous and loads coalesce.
//
// One workgroup moves one tile.  Tiles are walked row-major over the tile
// grid; inside a tile tokens are row-major in (t,h,w); edge tiles are partial.
// The tiled offset of tile (a,b,c) with extents (sa,sb,sc) is
//   a*tt*H*W + sa*(b*th)*W + sa*sb*(c*tw)
// because every tile before it in the walk is full along the axes that are
// already complete (packed layout), or tile_index * Bk (3D-padded layout,
// [PSA] App. C.2: every tile owns a whole block, padding after its tokens).
// Rows are copied 16 bytes per lane, so both the gather side and the scatter
// side move whole contiguous rows.
#include "svsa_internal.h"

namespace svsa {
namespace {

constexpr int kThreads = 256;

// floor(n / d) for n, d < 2^16 via a reciprocal m = ceil(2^32 / d): the
// quotient (n * m) >> 32 is exact because n * (m*d - 2^32) < n * d < 2^32.
// m needs 33 bits (d = 1 gives 2^32), so it is kept in 64 bits.
__device__ __forceinline__ uint32_t div_small(uint32_t n, uint64_t m) {
  return (uint32_t)(((uint64_t)n * m) >> 32);
}
__device__ __forceinline__ uint64_t recip_small(uint32_t d) {
  return (0x100000000ull + d - 1) / d;
}

// chunks_per_row = head_dim * element_bytes / 16 is a power of two (2^chunk_shift).
template <int kInverse>
__global__ void __launch_bounds__(kThreads)
tile_permute_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int32_t chunk_shift,
                    Geom g) {
  const int32_t chunks_per_row = 1 << chunk_shift;
  const int32_t ntiles = g.nT * g.nH * g.nW;
  const int32_t tile = blockIdx.x % ntiles;
  const int64_t bh = blockIdx.x / ntiles;
  const int32_t a = tile / (g.nH * g.nW);
  const int32_t b = (tile / g.nW) % g.nH;
  const int32_t c = tile % g.nW;
  const int32_t sa = min(g.tt, g.T - a * g.tt);
  const int32_t sb = min(g.th, g.H - b * g.th);
  const int32_t sc = min(g.tw, g.W - c * g.tw);
  const int32_t vol = sa * sb * sc;
  // packed layout: tiles back to back; 3D-padded layout: one Bk-slot block per tile
  const int64_t tiled0 = g.pad3d ? (int64_t)tile * g.Bk
                                 : (int64_t)a * g.tt * g.H * g.W + (int64_t)sa * (b * g.th) * g.W +
                                       (int64_t)sa * sb * (c * g.tw);
  const int64_t nat0 = ((int64_t)(a * g.tt) * g.H + b * g.th) * g.W + c * g.tw;
  const uint64_t m_sc = recip_small(sc), m_plane = recip_small(sb * sc);

  const int64_t nat_rows = (int64_t)g.N, tiled_rows = (int64_t)g.Npad;
  const uint4* sbase = src + bh * (kInverse ? tiled_rows : nat_rows) * chunks_per_row;
  uint4* dbase = dst + bh * (kInverse ? nat_rows : tiled_rows) * chunks_per_row;

  const int32_t total = vol * chunks_per_row;
  for (int32_t e = threadIdx.x; e < total; e += kThreads) {
    const uint32_t tok = (uint32_t)e >> chunk_shift;
    const int32_t ch = e & (chunks_per_row - 1);
    const uint32_t lt = div_small(tok, m_plane);
    const uint32_t rem = tok - lt * (uint32_t)(sb * sc);
    const uint32_t lh = div_small(rem, m_sc);
    const uint32_t lw = rem - lh * (uint32_t)sc;
    const int64_t nat = nat0 + ((int64_t)lt * g.H + lh) * g.W + lw;
    const int64_t til = tiled0 + tok;
    if (kInverse) {
      dbase[nat * chunks_per_row + ch] = sbase[til * chunks_per_row + ch];
    } else {
      dbase[til * chunks_per_row + ch] = sbase[nat * chunks_per_row + ch];
    }
  }
  // Padding slots are cleared (forward only): the rest of each partial tile's
  // block in the 3D-padded layout, the sequence tail (by the last tile's
  // workgroup) in the packed one.
  if (!kInverse && g.pad3d && vol < g.Bk) {
    const int32_t pad_chunks = (g.Bk - vol) * chunks_per_row;
    uint4* pad = dbase + (tiled0 + vol) * chunks_per_row;
    for (int32_t e = threadIdx.x; e < pad_chunks; e += kThreads) pad[e] = make_uint4(0, 0, 0, 0);
  }
  if (!kInverse && !g.pad3d && tile == ntiles - 1) {
    const int32_t pad_chunks = (g.Npad - g.N) * chunks_per_row;
    uint4* tail = dbase + (int64_t)g.N * chunks_per_row;
    for (int32_t e = threadIdx.x; e < pad_chunks; e += kThreads) tail[e] = make_uint4(0, 0, 0, 0);
  }
}

// Forward reorder fused with the block means (stages 1 and 2 in one pass).
// One workgroup per (b, h, block): the block's tiled slots are filled from
// their natural rows and the valid rows are summed in float64 on the way, so
// the tiled tensor is not read back for pooling.  Blocks are walked in the
// tiled order rather than by tile because in the packed layout a block can
// span several partial tiles.  The natural row of tiled slot p inverts the
// tile walk: the slab of tile rows along t (every earlier slab is full), then
// the row of tiles along h inside it (every earlier row is full), then the
// tile along w, then (t, h, w) inside the tile.  kElt: 2 (bf16) or 4 (f32).
constexpr int kMapRows = 1024;  // natural-row map entries held in LDS at once

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int kElt>
__global__ void __launch_bounds__(kThreads)
tile_permute_pool_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                         double* __restrict__ means, int32_t head_dim, Geom g) {
  constexpr int kPer = 16 / kElt;
  __shared__ int32_t nat_map[kMapRows];
  extern __shared__ double red[];  // [groups][head_dim]
  const int32_t nb = g.nb;
  const int64_t bh = blockIdx.x / nb;
  const int32_t blk = blockIdx.x % nb;
  const int32_t n_valid = block_valid(g, blk);
  const int32_t chunks = head_dim / kPer;
  const int32_t groups = kThreads / chunks;
  const int32_t ch = threadIdx.x % chunks;
  const int32_t rg = threadIdx.x / chunks;
  const uint4* sbase = src + bh * g.N * chunks;
  uint4* dbase = dst + (bh * g.Npad + (int64_t)blk * g.Bk) * chunks;

  double acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.0;
  for (int32_t r0 = 0; r0 < g.Bk; r0 += kMapRows) {
    const int32_t rows = min(kMapRows, g.Bk - r0);
    const int32_t valid = max(0, min(rows, n_valid - r0));
    if (r0 > 0) __syncthreads();  // the previous chunk's map is no longer read
    for (int32_t t = threadIdx.x; t < valid; t += kThreads) nat_map[t] = natural_row(g, blk, r0 + t);
    __syncthreads();
    for (int32_t r = rg; r < rows; r += groups) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (r < valid) {
        u = sbase[(int64_t)nat_map[r] * chunks + ch];
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
      dbase[(int64_t)(r0 + r) * chunks + ch] = u;
    }
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) red[rg * head_dim + ch * kPer + e] = acc[e];
  __syncthreads();
  const double n = (double)n_valid;
  for (int32_t d = threadIdx.x; d < head_dim; d += kThreads) {
    double s = 0.0;
    for (int32_t r = 0; r < groups; ++r) s += red[r * head_dim + d];
    means[(bh * nb + blk) * head_dim + d] = s / n;
  }
}

}  // namespace

hipError_t launch_tile_permute_pool(const void* src, void* dst, double* means, bool is_bf16,
                                    int32_t bh, int32_t head_dim, const Geom& g,
                                    hipStream_t stream) {
  const int elt = is_bf16 ? 2 : 4;
  const int32_t chunks = head_dim * elt / 16;
  if (chunks <= 0 || chunks > kThreads || kThreads % chunks != 0) return hipErrorInvalidValue;
  const size_t lds = (size_t)(kThreads / chunks) * head_dim * sizeof(double);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)bh * g.nb;
  if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (is_bf16) {
    hipLaunchKernelGGL(tile_permute_pool_kernel<2>, dim3((uint32_t)blocks), dim3(kThreads), lds,
                       stream, (const uint4*)src, (uint4*)dst, means, head_dim, g);
  } else {
    hipLaunchKernelGGL(tile_permute_pool_kernel<4>, dim3((uint32_t)blocks), dim3(kThreads), lds,
                       stream, (const uint4*)src, (uint4*)dst, means, head_dim, g);
  }
  return hipGetLastError();
}

hipError_t launch_tile_permute(const void* src, void* dst, int elt_bytes, int32_t bh,
                               int32_t head_dim, const Geom& g, bool inverse,
                               hipStream_t stream) {
  const int32_t chunks = head_dim * elt_bytes / 16;
  int32_t shift = 0;
  while ((1 << shift) < chunks) ++shift;
  if ((1 << shift) != chunks) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)bh * g.nT * g.nH * g.nW;
  if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (inverse) {
    hipLaunchKernelGGL(tile_permute_kernel<1>, dim3((uint32_t)blocks), dim3(kThreads), 0, stream,
                       (const uint4*)src, (uint4*)dst, shift, g);
  } else {
    hipLaunchKernelGGL(tile_permute_kernel<0>, dim3((uint32_t)blocks), dim3(kThreads), 0, stream,
                       (const uint4*)src, (uint4*)dst, shift, g);
  }
  return hipGetLastError();
}

}  // namespace svsa
