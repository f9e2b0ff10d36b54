// Stripe masks: [PSA] "Parameterized Stripe Attention for Efficient Video
// Generation", Sec. 3.2 "Unified Representation" and Alg. 1 "PSA Mask
// Definition".  Six integers M(Tw, To, Ts, Sw, So, Ss) give the width, offset
// and stride of an inter-frame band (over the frame distance dt = t_k - t_q)
// and an intra-frame band (over the in-frame distance ds = s_k - s_q); a pair
// attends when ((|dt - To|) mod Ts) <= Tw - 1 and ((|ds - So|) mod Ss) <= Sw - 1,
// an infinite stride meaning no modulo.  PSA applies the mask per PSABlock.
//
// Here the positions are tiles of the tile grid (nT, nH, nW): t = the tile's
// t index, s = h index * nW + w index; a stride <= 0 stands for infinity.  A
// query block keeps a key block when some tile of the first attends to some
// tile of the second (blocks of partial tiles hold several tiles), plus an
// optional diagonal band |i - j| <= band - 1.  The output is the same CSR as
// the top-p path, so the attention kernel runs on it unchanged.
//
// Kernels:
//   block_tiles_kernel   one thread per block: the tiles its valid tokens
//                        belong to (tokens of a tile are contiguous in tile
//                        order, so this walks tile by tile)
//   stripe_select_kernel one workgroup per (b, h, query block), one thread per
//                        key block: the tile-pair test, row bitmap and count
// then the shared scan / compaction kernels build the CSR.
#include "svsa_internal.h"

namespace svsa {
namespace {

struct StripeParams {
  int32_t v[kStripeMaxHeads][6];  // Tw, To, Ts, Sw, So, Ss per head
};

constexpr int kTilesThreads = 256;

// tiles[b * Bk + k] = (t', s') of the k-th tile of block b; ntiles[b] = count
__global__ void __launch_bounds__(kTilesThreads)
block_tiles_kernel(int2* __restrict__ tiles, int32_t* __restrict__ ntiles, Geom g) {
  const int32_t b = blockIdx.x * kTilesThreads + threadIdx.x;
  if (b >= g.nb) return;
  if (g.pad3d) {   // one block per tile
    tiles[(int64_t)b * g.Bk] = make_int2(b / (g.nH * g.nW), b % (g.nH * g.nW));
    ntiles[b] = 1;
    return;
  }
  const int64_t HW = (int64_t)g.H * g.W;
  int64_t p = (int64_t)b * g.Bk;
  const int64_t end = min((int64_t)(b + 1) * g.Bk, (int64_t)g.N);
  int32_t n = 0;
  while (p < end && n < g.Bk) {  // each tile adds >= 1 token, so n <= Bk
    // tile (a, c_h, c_w) holding tiled position p, and its first position
    const int32_t a = (int32_t)min(p / ((int64_t)g.tt * HW), (int64_t)g.nT - 1);
    const int32_t tta = min(g.tt, g.T - a * g.tt);
    const int64_t r = p - (int64_t)a * g.tt * HW;
    const int32_t ch = (int32_t)min(r / ((int64_t)tta * g.th * g.W), (int64_t)g.nH - 1);
    const int32_t thb = min(g.th, g.H - ch * g.th);
    const int64_t r2 = r - (int64_t)ch * tta * g.th * g.W;
    const int32_t cw = (int32_t)min(r2 / ((int64_t)tta * thb * g.tw), (int64_t)g.nW - 1);
    const int32_t twc = min(g.tw, g.W - cw * g.tw);
    const int64_t start = (int64_t)a * g.tt * HW + (int64_t)ch * tta * g.th * g.W +
                          (int64_t)cw * tta * thb * g.tw;
    tiles[(int64_t)b * g.Bk + n] = make_int2(a, ch * g.nW + cw);
    ++n;
    p = start + (int64_t)tta * thb * twc;  // first position of the next tile
  }
  ntiles[b] = n;
}

// ((|d - o|) mod s) <= w - 1, s <= 0 meaning no modulo
__device__ __forceinline__ bool in_band(int32_t d, int32_t w, int32_t o, int32_t s) {
  int32_t x = d - o;
  x = x < 0 ? -x : x;
  if (s > 0) x %= s;
  return x <= w - 1;
}

constexpr int kSelThreads = 256;

__global__ void __launch_bounds__(kSelThreads)
stripe_select_kernel(const int2* __restrict__ tiles, const int32_t* __restrict__ ntiles,
                     uint32_t* __restrict__ bits, int32_t* __restrict__ counts, int32_t nb,
                     int32_t Bk, int32_t heads, int32_t words, int32_t band, StripeParams prm) {
  extern __shared__ int2 qt[];          // tiles of the query block (<= Bk)
  __shared__ int32_t wcount[kSelThreads / 64];
  const int64_t row = blockIdx.x;
  const int32_t i = (int32_t)(row % nb);
  const int32_t h = (int32_t)((row / nb) % heads);
  const int32_t Tw = prm.v[h][0], To = prm.v[h][1], Ts = prm.v[h][2];
  const int32_t Sw = prm.v[h][3], So = prm.v[h][4], Ss = prm.v[h][5];
  const int32_t nq = ntiles[i];
  for (int32_t k = threadIdx.x; k < nq; k += kSelThreads) qt[k] = tiles[(int64_t)i * Bk + k];
  __syncthreads();
  uint32_t* brow = bits + row * words;
  int32_t cnt = 0;
  for (int32_t j0 = 0; j0 < nb; j0 += kSelThreads) {
    const int32_t j = j0 + threadIdx.x;
    bool keep = false;
    if (j < nb) {
      keep = (j - i <= band - 1) && (i - j <= band - 1);
      const int32_t nk = ntiles[j];
      const int2* kt = tiles + (int64_t)j * Bk;
      for (int32_t b = 0; b < nk && !keep; ++b) {
        const int2 kk = kt[b];
        for (int32_t a = 0; a < nq; ++a) {
          const int2 qq = qt[a];
          if (in_band(kk.x - qq.x, Tw, To, Ts) && in_band(kk.y - qq.y, Sw, So, Ss)) {
            keep = true;
            break;
          }
        }
      }
    }
    const uint64_t bal = __ballot(keep);
    const int lane = threadIdx.x & 63;
    // each wave owns two consecutive 32-bit words of the row bitmap
    const int32_t w0 = (j0 >> 5) + 2 * (threadIdx.x >> 6);
    if (lane == 0 && w0 < words) brow[w0] = (uint32_t)bal;
    if (lane == 0 && w0 + 1 < words) brow[w0 + 1] = (uint32_t)(bal >> 32);
    cnt += keep ? 1 : 0;
  }
  // row count
  int32_t c = cnt;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) c += __shfl_xor(c, s, 64);
  if ((threadIdx.x & 63) == 0) wcount[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t tot = 0;
    for (int k = 0; k < kSelThreads / 64; ++k) tot += wcount[k];
    counts[row] = tot;
  }
}

}  // namespace

StripeWs stripe_ws_layout(int64_t rows, const Geom& g) {
  StripeWs w{};
  w.words = (g.nb + 31) / 32;
  size_t off = 0;
  w.tiles_off = off;
  off = align_up(off + (size_t)g.nb * g.Bk * sizeof(int2), 256);
  w.ntiles_off = off;
  off = align_up(off + (size_t)g.nb * sizeof(int32_t), 256);
  w.bits_off = off;
  off = align_up(off + (size_t)rows * w.words * sizeof(uint32_t), 256);
  w.counts_off = off;
  off = align_up(off + (size_t)rows * sizeof(int32_t), 256);
  w.total = off;
  return w;
}

hipError_t launch_stripe_mask(const Geom& g, int32_t bh, int32_t heads, const int32_t* params,
                              int32_t band, int32_t* row_ptr, int32_t* col_idx, void* ws,
                              hipStream_t stream) {
  if (heads > kStripeMaxHeads) return hipErrorInvalidValue;
  const int64_t rows = (int64_t)bh * g.nb;
  if (rows > 0x7fffffff) return hipErrorInvalidValue;
  const StripeWs w = stripe_ws_layout(rows, g);
  char* base = static_cast<char*>(ws);
  int2* tiles = reinterpret_cast<int2*>(base + w.tiles_off);
  int32_t* ntiles = reinterpret_cast<int32_t*>(base + w.ntiles_off);
  uint32_t* bits = reinterpret_cast<uint32_t*>(base + w.bits_off);
  int32_t* counts = reinterpret_cast<int32_t*>(base + w.counts_off);
  StripeParams prm{};
  for (int32_t h = 0; h < heads; ++h)
    for (int k = 0; k < 6; ++k) prm.v[h][k] = params[h * 6 + k];
  hipLaunchKernelGGL(block_tiles_kernel, dim3((uint32_t)((g.nb + kTilesThreads - 1) / kTilesThreads)),
                     dim3(kTilesThreads), 0, stream, tiles, ntiles, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(stripe_select_kernel, dim3((uint32_t)rows), dim3(kSelThreads),
                     (size_t)g.Bk * sizeof(int2), stream, tiles, ntiles, bits, counts, g.nb, g.Bk,
                     heads, w.words, band, prm);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_csr_from_bits(bits, counts, row_ptr, col_idx, rows, w.words, stream);
}

}  // namespace svsa
