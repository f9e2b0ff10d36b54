// Variable-size blocks: query / key clustering and the cluster layout.
//
// [iCATS] "iCATS: Fast Video Generation via Interaction-Aware Sparse Attention
// and Timestep-Adaptive Sparsity", Sec. 3.1 and 4.1: clustering targets the
// error of the query-key interactions, written as a quadratic form in the
// feature space; query clusters start in plain feature space, later use the
// key clusters' metric, and guide the key clustering in turn.  [SVOO]
// "Attention Sparsity is Input-Stable: ... Online QK Co-Clustering":
// bidirectional co-clustering of queries and keys into blocks.
//
// Reading implemented here: replacing a token x by a centroid c changes its
// logits against the other side's tokens y by (x - c).y, whose summed square
// is (x - c)^T G (x - c) with G = sum_y y y^T, approximated from the other
// side's clusters as G = sum_j n_j c_j c_j^T.  Lloyd iterations under that
// fixed metric: assign every token to the centroid of least distance (ties:
// lowest index), then move every non-empty centroid to its members' mean.
//
// Kernels:
//   hist_kernel, offsets_kernel, place_kernel
//                  the layout: per-tile cluster counts, padded starts and tile
//                  offsets, then a stable counting sort inside each tile
//                  (members in ascending token order)
//   means_kernel   one wavefront per cluster: float64 sum of the members in
//                  that order, mean written only for non-empty clusters
//   metric_kernel  G = sum_c n_c c c^T, 16 x 16 tile of G per workgroup
//   prep_kernel    g_c = G c (float64) split into bf16 hi + lo, and c^T G c
//   assign_kernel  MFMA: 256 tokens per workgroup against all centroids in
//                  chunks of 32; d(x, c) - x^T G x = c^T G c - 2 x . g_c
//   permute_kernel rows gathered into the padded cluster layout (padding
//                  zero) or scattered back to token order
//   rows_to_bits_kernel, merge_kernel, relabel_kernel, pair_kernel,
//   move_kernel, popcount_kernel
//                  tail merging of the query clusters (see below)
#include "svsa_internal.h"

namespace svsa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// Layout in three passes over tiles of kLayTile tokens (many workgroups per
// head): tile histograms, then per (b, h) the padded cluster starts and each
// tile's first slot per cluster, then a stable placement inside every tile.
// Labels outside [0, C) are not placed (slot -1).
// ---------------------------------------------------------------------------
constexpr int kLayThreads = 256, kLayTile = 2048;

__global__ void __launch_bounds__(kLayThreads)
hist_kernel(const int32_t* __restrict__ labels, int32_t N, int32_t C, int32_t tiles,
            int32_t* __restrict__ tcount) {
  extern __shared__ int32_t cnt[];  // [C]
  const int64_t bh = blockIdx.y;
  const int32_t tile = blockIdx.x;
  for (int32_t c = threadIdx.x; c < C; c += kLayThreads) cnt[c] = 0;
  __syncthreads();
  const int32_t* lab = labels + bh * N;
  const int32_t t1 = min(N, (tile + 1) * kLayTile);
  for (int32_t t = tile * kLayTile + threadIdx.x; t < t1; t += kLayThreads) {
    const int32_t c = lab[t];
    if (c >= 0 && c < C) atomicAdd(&cnt[c], 1);
  }
  __syncthreads();
  int32_t* out = tcount + (bh * tiles + tile) * (int64_t)C;
  for (int32_t c = threadIdx.x; c < C; c += kLayThreads) out[c] = cnt[c];
}

// one workgroup per (b, h): sizes, padded starts, tile offsets (in place of
// the tile counts) and -1 in every slot of the padded length
__global__ void __launch_bounds__(kLayThreads)
offsets_kernel(int32_t C, int32_t align, int32_t tiles, int32_t* __restrict__ tcount,
               int32_t* __restrict__ start, int32_t* __restrict__ sizes,
               int32_t* __restrict__ token, int64_t lcap) {
  __shared__ int32_t part[kLayThreads];
  const int64_t bh = blockIdx.x;
  const int32_t tid = threadIdx.x;
  int32_t* tc = tcount + bh * tiles * (int64_t)C;
  const int32_t per = (C + kLayThreads - 1) / kLayThreads;
  const int32_t c0 = tid * per, c1 = min(C, c0 + per);
  int32_t local = 0;
  for (int32_t c = c0; c < c1; ++c) {
    int32_t n = 0;
    for (int32_t t = 0; t < tiles; ++t) n += tc[(int64_t)t * C + c];
    sizes[bh * C + c] = n;
    local += (n + align - 1) / align * align;
  }
  part[tid] = local;
  __syncthreads();
  for (int32_t off = 1; off < kLayThreads; off <<= 1) {
    const int32_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = part[tid] - local;
  int32_t* st = start + bh * (int64_t)(C + 1);
  for (int32_t c = c0; c < c1; ++c) {
    st[c] = run;
    int32_t cur = run;
    for (int32_t t = 0; t < tiles; ++t) {
      const int32_t n = tc[(int64_t)t * C + c];
      tc[(int64_t)t * C + c] = cur;
      cur += n;
    }
    run += (cur - run + align - 1) / align * align;
  }
  const int32_t total = part[kLayThreads - 1];
  if (tid == 0) st[C] = total;
  int32_t* tok = token + bh * lcap;
  for (int32_t s = tid; s < total; s += kLayThreads) tok[s] = -1;
}

// stable placement inside one tile: chunk by chunk in token order, a token's
// rank is the number of earlier tokens of its chunk with the same label
__global__ void __launch_bounds__(kLayThreads)
place_kernel(const int32_t* __restrict__ labels, int32_t N, int32_t C, int32_t tiles,
             const int32_t* __restrict__ toff, int32_t* __restrict__ slot,
             int32_t* __restrict__ token, int64_t lcap) {
  extern __shared__ int32_t cursor[];  // [C]
  __shared__ int32_t lab_s[kLayThreads];
  const int64_t bh = blockIdx.y;
  const int32_t tile = blockIdx.x, tid = threadIdx.x;
  const int32_t* to = toff + (bh * tiles + tile) * (int64_t)C;
  for (int32_t c = tid; c < C; c += kLayThreads) cursor[c] = to[c];
  const int32_t* lab = labels + bh * N;
  int32_t* tok = token + bh * lcap;
  int32_t* sl = slot ? slot + bh * N : nullptr;
  const int32_t t1 = min(N, (tile + 1) * kLayTile);
  __syncthreads();
  for (int32_t base = tile * kLayTile; base < t1; base += kLayThreads) {
    const int32_t t = base + tid;
    const int32_t c = t < t1 ? lab[t] : -1;
    lab_s[tid] = c;
    __syncthreads();
    const bool ok = c >= 0 && c < C;
    if (ok) {
      int32_t rank = 0;
      for (int32_t j = 0; j < tid; ++j) rank += lab_s[j] == c;
      const int32_t s = cursor[c] + rank;
      tok[s] = t;
      if (sl) sl[t] = s;
    } else if (t < t1 && sl) {
      sl[t] = -1;
    }
    __syncthreads();
    if (ok) atomicAdd(&cursor[c], 1);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// means_kernel: one wavefront per (b, h, c); members token[start .. start+n)
// (ascending token order, from the layout with align 1).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
means_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ start,
             const int32_t* __restrict__ sizes, const int32_t* __restrict__ token,
             double* __restrict__ cents, int32_t N, int32_t C, int32_t D, int64_t lcap,
             int64_t total) {
  const int64_t w = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  if (w >= total) return;
  const int32_t lane = threadIdx.x % 64;
  const int64_t bh = w / C;
  const int32_t c = (int32_t)(w % C);
  const int32_t n = sizes[bh * C + c];
  if (n == 0) return;  // empty: the centroid stays
  const int32_t s0 = start[bh * (int64_t)(C + 1) + c];
  const int32_t* tok = token + bh * lcap + s0;
  const uint16_t* xb = x + bh * (int64_t)N * D;
  double acc0 = 0.0, acc1 = 0.0;   // dims lane and lane + 64, summed in member order
  const int32_t d0 = lane < D ? lane : 0, d1 = lane + 64 < D ? lane + 64 : 0;
  int32_t m = 0;
  for (; m + 8 <= n; m += 8) {     // eight member rows in flight
    float a[8], b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint16_t* row = xb + (int64_t)tok[m + u] * D;
      a[u] = bf16_bits_to_float(row[d0]);
      b[u] = bf16_bits_to_float(row[d1]);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc0 += (double)a[u];
      acc1 += (double)b[u];
    }
  }
  for (; m < n; ++m) {
    const uint16_t* row = xb + (int64_t)tok[m] * D;
    acc0 += (double)bf16_bits_to_float(row[d0]);
    acc1 += (double)bf16_bits_to_float(row[d1]);
  }
  double* out = cents + (bh * C + c) * (int64_t)D;
  if (lane < D) out[lane] = acc0 / n;
  if (lane + 64 < D) out[lane + 64] = acc1 / n;
}

// ---------------------------------------------------------------------------
// metric_kernel: G[d][e] = sum_c n_c cent[c][d] cent[c][e] (float64).
// ---------------------------------------------------------------------------
constexpr int kMt = 16, kMc = 64;

__global__ void __launch_bounds__(256)
metric_kernel(const double* __restrict__ cents, const int32_t* __restrict__ sizes,
              double* __restrict__ G, int32_t C, int32_t D, int32_t tiles) {
  __shared__ double sd[kMc][kMt + 1];
  __shared__ double se[kMc][kMt + 1];
  __shared__ double sn[kMc];
  const int64_t bh = blockIdx.x / (tiles * tiles);
  const int32_t t2 = blockIdx.x % (tiles * tiles);
  const int32_t d0 = (t2 / tiles) * kMt, e0 = (t2 % tiles) * kMt;
  const int32_t dl = threadIdx.x / kMt, el = threadIdx.x % kMt;
  const double* cb = cents + bh * (int64_t)C * D;
  double acc = 0.0;
  for (int32_t cc = 0; cc < C; cc += kMc) {
    for (int32_t i = threadIdx.x; i < kMc * kMt; i += 256) {
      const int32_t r = i / kMt, k = i % kMt;
      const bool ok = cc + r < C;
      sd[r][k] = ok ? cb[(int64_t)(cc + r) * D + d0 + k] : 0.0;
      se[r][k] = ok ? cb[(int64_t)(cc + r) * D + e0 + k] : 0.0;
    }
    if (threadIdx.x < kMc) sn[threadIdx.x] = cc + (int)threadIdx.x < C
                                                  ? (double)sizes[bh * C + cc + threadIdx.x] : 0.0;
    __syncthreads();
    const int32_t lim = min(kMc, C - cc);
    for (int32_t r = 0; r < lim; ++r) acc = fma(sn[r] * sd[r][dl], se[r][el], acc);
    __syncthreads();
  }
  G[(bh * D + d0 + dl) * (int64_t)D + e0 + el] = acc;
}

// ---------------------------------------------------------------------------
// prep_kernel: per (b, h, c) g = G c (or c without a metric), q = c . g;
// g is stored as bf16 hi + lo (hi = bf16(g), lo = bf16(g - hi)) for the MFMA.
// kPrepC centroids per workgroup of 128 threads (thread d: component d); G is
// symmetric, so thread d reads column d (coalesced across the workgroup).
// ---------------------------------------------------------------------------
constexpr int kPrepC = 8;

__global__ void __launch_bounds__(128)
prep_kernel(const double* __restrict__ cents, const double* __restrict__ G,
            uint16_t* __restrict__ g_hi, uint16_t* __restrict__ g_lo, float* __restrict__ cq,
            int32_t C, int32_t D, int32_t cgroups) {
  __shared__ double cv[kPrepC][128];
  __shared__ double red[kPrepC][128];
  const int64_t bh = blockIdx.x / cgroups;
  const int32_t c0 = (int32_t)(blockIdx.x % cgroups) * kPrepC;
  const int32_t d = threadIdx.x;
  const int32_t nc = min(kPrepC, C - c0);
  const double* cb = cents + (bh * C + c0) * (int64_t)D;
  for (int32_t k = 0; k < kPrepC; ++k) cv[k][d] = (k < nc && d < D) ? cb[(int64_t)k * D + d] : 0.0;
  __syncthreads();
  double g[kPrepC];
#pragma unroll
  for (int32_t k = 0; k < kPrepC; ++k) g[k] = G ? 0.0 : cv[k][d];
  if (G && d < D) {
    const double* Gb = G + bh * (int64_t)D * D;
    for (int32_t e = 0; e < D; ++e) {
      const double ge = Gb[(int64_t)e * D + d];
#pragma unroll
      for (int32_t k = 0; k < kPrepC; ++k) g[k] = fma(ge, cv[k][e], g[k]);
    }
  }
#pragma unroll
  for (int32_t k = 0; k < kPrepC; ++k) {
    if (k < nc && d < D) {
      const int64_t w = (bh * C + c0 + k) * (int64_t)D + d;
      const float gf = (float)g[k];
      const uint32_t hi = float_to_bf16_bits(gf);
      g_hi[w] = (uint16_t)hi;
      g_lo[w] = (uint16_t)float_to_bf16_bits(gf - bf16_bits_to_float(hi));
    }
    red[k][d] = d < D ? cv[k][d] * g[k] : 0.0;
  }
  __syncthreads();
  for (int32_t sft = 64; sft > 0; sft >>= 1) {
    if (d < sft)
#pragma unroll
      for (int32_t k = 0; k < kPrepC; ++k) red[k][d] += red[k][d + sft];
    __syncthreads();
  }
  if (d < nc) cq[bh * C + c0 + d] = (float)red[d][0];
}

// ---------------------------------------------------------------------------
// assign_kernel: label[t] = argmin_c (c^T G c - 2 x_t . g_c), ties to the
// lowest c.  v_mfma_f32_32x32x16_bf16 with A = g (32 centroids x 16 dims,
// from LDS) and B = x^T (16 dims x 32 tokens, registers): each lane then holds
// one token column and 16 centroid rows of the 32 x 32 output.
// ---------------------------------------------------------------------------
constexpr int kAsWaves = 8, kAsTok = 32 * kAsWaves, kAsC = 32;

template <int D>
__global__ void __launch_bounds__(64 * kAsWaves)
assign_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ g_hi,
              const uint16_t* __restrict__ g_lo, const float* __restrict__ cq,
              int32_t* __restrict__ labels, int32_t N, int32_t C, int32_t tiles) {
  constexpr int kChunks = D / 8;              // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) uint4 ahi[2][kAsC * kChunks];
  __shared__ __attribute__((aligned(16))) uint4 alo[2][kAsC * kChunks];
  __shared__ float acq[2][kAsC];
  const int64_t bh = blockIdx.x / tiles;
  const int32_t t0 = (int32_t)(blockIdx.x % tiles) * kAsTok;
  const int32_t wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int32_t col = lane % 32, half = lane / 32;
  const int32_t tok = t0 + wave * 32 + col;

  // B operand: 8 consecutive dims of this lane's token per 16-dim step
  bf16x8 xb[D / 16];
  const uint4* xrow = reinterpret_cast<const uint4*>(x + (bh * N + (tok < N ? tok : 0)) * (int64_t)D);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    uint4 v = xrow[2 * ks + half];
    if (tok >= N) v = make_uint4(0, 0, 0, 0);
    xb[ks] = __builtin_bit_cast(bf16x8, v);
  }

  const uint4* ghi = reinterpret_cast<const uint4*>(g_hi + bh * (int64_t)C * D);
  const uint4* glo = reinterpret_cast<const uint4*>(g_lo + bh * (int64_t)C * D);
  const float* cqb = cq + bh * (int64_t)C;
  const int32_t nchunk = (C + kAsC - 1) / kAsC;
  // stage chunk k into buffer k & 1 (rows beyond C are zero, never selected);
  // row r's 16-byte piece q lands at q ^ (r & 15) so the operand reads of 32
  // rows at one column hit different banks
  auto stage = [&](int32_t k) {
    const int32_t buf = k & 1;
    for (int32_t i = threadIdx.x; i < kAsC * kChunks; i += 64 * kAsWaves) {
      const int32_t r = i / kChunks, q = i % kChunks;
      const int32_t c = k * kAsC + r;
      const int32_t dst = r * kChunks + (q ^ (r & (kChunks - 1) & 15));
      ahi[buf][dst] = c < C ? ghi[(int64_t)c * kChunks + q] : make_uint4(0, 0, 0, 0);
      alo[buf][dst] = c < C ? glo[(int64_t)c * kChunks + q] : make_uint4(0, 0, 0, 0);
    }
    if (threadIdx.x < kAsC) {
      const int32_t c = k * kAsC + threadIdx.x;
      acq[buf][threadIdx.x] = c < C ? cqb[c] : 0.0f;
    }
  };

  float best = __builtin_huge_valf();
  int32_t bidx = 0x7fffffff;
  stage(0);
  __syncthreads();
  for (int32_t k = 0; k < nchunk; ++k) {
    if (k + 1 < nchunk) stage(k + 1);
    const int32_t buf = k & 1;
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int32_t q = 2 * ks + half;
      const int32_t a_off = col * kChunks + (q ^ (col & (kChunks - 1) & 15));
      const bf16x8 ah = __builtin_bit_cast(bf16x8, ahi[buf][a_off]);
      const bf16x8 al = __builtin_bit_cast(bf16x8, alo[buf][a_off]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xb[ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xb[ks], acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int32_t row = (r / 4) * 8 + half * 4 + (r % 4);
      const int32_t c = k * kAsC + row;
      const float s = acq[buf][row] - 2.0f * acc[r];
      if (c < C && s < best) {   // rows ascend within a lane: strict < keeps the lowest
        best = s;
        bidx = c;
      }
    }
    __syncthreads();
  }
  // the two lanes of a token column hold interleaved row sets: combine
  const float ob = __shfl_xor(best, 32);
  const int32_t oi = __shfl_xor(bidx, 32);
  if (ob < best || (ob == best && oi < bidx)) {
    best = ob;
    bidx = oi;
  }
  if (half == 0 && tok < N) labels[bh * N + tok] = bidx;
}

// ---------------------------------------------------------------------------
// permute_kernel: forward dst[s] = src[token[s]] (zero for padding) over the
// slots s < start[C] of each (b, h); inverse dst[t] = src[slot[t]] (zero when
// the token was not placed).  16-byte chunks.
// ---------------------------------------------------------------------------
template <int kInverse>
__global__ void __launch_bounds__(256)
cluster_permute_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                       const int32_t* __restrict__ map, const int32_t* __restrict__ start,
                       int32_t N, int32_t C, int64_t lcap, int32_t chunk_shift,
                       int32_t rows_per_block) {
  const int32_t chunks = 1 << chunk_shift;
  const int64_t bh = blockIdx.y;
  const int64_t rows = kInverse ? N : start[bh * (int64_t)(C + 1) + C];
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  if (r0 >= rows) return;
  const int64_t r1 = min(rows, r0 + rows_per_block);
  const int64_t src_rows = kInverse ? lcap : N, dst_rows = kInverse ? N : lcap;
  const int32_t* m = map + bh * (kInverse ? (int64_t)N : lcap);
  for (int64_t e = r0 * chunks + threadIdx.x; e < r1 * chunks; e += 256) {
    const int64_t r = e >> chunk_shift;
    const int32_t ch = (int32_t)(e & (chunks - 1));
    const int32_t from = m[r];
    dst[(bh * dst_rows + r) * chunks + ch] =
        from >= 0 ? src[(bh * src_rows + from) * chunks + ch] : make_uint4(0, 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Tail merging ([iCATS] Sec. 4.3, App. E.1): query clusters with identical
// kept key-cluster sets merge into the lowest index; then, per round, every
// non-empty cluster with a tail (size mod block) finds its nearest other such
// cluster by Jaccard similarity of the kept sets (compared exactly as integer
// cross products; ties to the lowest index), and mutually nearest pairs whose
// tails fit one block move the smaller tail (equal: the higher index's) to
// the other cluster, which takes the union of both kept sets.  Kept sets are
// row bitmaps of `words` uint32.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(64)
rows_to_bits_kernel(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
                    uint32_t* __restrict__ bits, int32_t nk, int32_t words) {
  const int64_t r = blockIdx.x;
  uint32_t* b = bits + r * words;
  for (int32_t w = threadIdx.x; w < words; w += 64) b[w] = 0u;
  __syncthreads();
  for (int32_t e = row_ptr[r] + threadIdx.x; e < row_ptr[r + 1]; e += 64) {
    const int32_t j = col_idx[e];
    if (j >= 0 && j < nk) atomicOr(&b[j >> 5], 1u << (j & 31));
  }
}

__device__ __forceinline__ bool rows_equal(const uint32_t* a, const uint32_t* b, int32_t words) {
  for (int32_t w = 0; w < words; ++w)
    if (a[w] != b[w]) return false;
  return true;
}

// The bitmaps of one (b, h) are read many times by the two per-head kernels
// below: with kLds they are first copied into LDS (after the C counters).
constexpr int kTailThreads = 1024;   // per-head kernels: many waves to hide LDS latency

// The LDS copy uses an odd row stride (words | 1) so that the rows the lanes
// of a wavefront read at one word offset fall in different banks.
__host__ __device__ inline int32_t lds_stride(int32_t words) { return words | 1; }

template <bool kLds>
__device__ __forceinline__ const uint32_t* head_bits(const uint32_t* g, int32_t* sh, int32_t C,
                                                      int32_t words, int32_t* stride) {
  if (!kLds) {
    *stride = words;
    return g;
  }
  const int32_t ls = lds_stride(words);
  uint32_t* l = reinterpret_cast<uint32_t*>(sh + C);
  for (int32_t e = threadIdx.x; e < C * words; e += kTailThreads)
    l[(e / words) * ls + e % words] = g[e];
  __syncthreads();
  *stride = ls;
  return l;
}

// one workgroup per (b, h): rep[i] = lowest j <= i, both non-empty, with the
// same kept set
template <bool kLds>
__global__ void __launch_bounds__(kTailThreads)
merge_kernel(const int32_t* __restrict__ labels, int32_t N, int32_t C,
             const uint32_t* __restrict__ bits, int32_t words, int32_t* __restrict__ rep) {
  extern __shared__ int32_t cnt[];  // [C] (+ [C * words] bitmaps with kLds)
  const int64_t bh = blockIdx.x;
  for (int32_t c = threadIdx.x; c < C; c += kTailThreads) cnt[c] = 0;
  __syncthreads();
  const int32_t* lab = labels + bh * N;
  for (int32_t t = threadIdx.x; t < N; t += kTailThreads) {
    const int32_t c = lab[t];
    if (c >= 0 && c < C) atomicAdd(&cnt[c], 1);
  }
  __syncthreads();
  int32_t rs;
  const uint32_t* bb = head_bits<kLds>(bits + bh * (int64_t)C * words, cnt, C, words, &rs);
  for (int32_t i = threadIdx.x; i < C; i += kTailThreads) {
    int32_t r = i;
    if (cnt[i] > 0)
      for (int32_t j = 0; j < i; ++j)
        if (cnt[j] > 0 && rows_equal(bb + (int64_t)j * rs, bb + (int64_t)i * rs, words)) {
          r = j;
          break;
        }
    rep[bh * C + i] = r;
  }
}

__global__ void __launch_bounds__(256)
relabel_kernel(int32_t* __restrict__ labels, const int32_t* __restrict__ rep, int32_t N,
               int32_t C, int64_t total) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const int32_t c = labels[e];
  if (c >= 0 && c < C) labels[e] = rep[(e / N) * C + c];
}

// one workgroup per (b, h): the pairs of one round; move_to[d] = receiver of
// donor d (else -1), cut[d] = members of d that stay (its first ones)
template <bool kLds>
__global__ void __launch_bounds__(kTailThreads)
pair_kernel(const int32_t* __restrict__ sizes, int32_t C, uint32_t* __restrict__ bits,
            int32_t words, int32_t block, int32_t* __restrict__ move_to,
            int32_t* __restrict__ cut) {
  extern __shared__ int32_t near[];  // [C] (+ [C * words] bitmaps with kLds)
  const int64_t bh = blockIdx.x;
  const int32_t* sz = sizes + bh * C;
  uint32_t* bb = bits + bh * (int64_t)C * words;       // the unions go here
  int32_t rs;
  const uint32_t* rb = head_bits<kLds>(bb, near, C, words, &rs);
  for (int32_t i = threadIdx.x; i < C; i += kTailThreads) {
    int32_t best = -1;
    if (sz[i] > 0 && sz[i] % block > 0) {
      const uint32_t* bi = rb + (int64_t)i * rs;
      int64_t b_in = 0, b_un = 1;
      for (int32_t j = 0; j < C; ++j) {
        if (j == i || sz[j] == 0 || sz[j] % block == 0) continue;
        const uint32_t* bj = rb + (int64_t)j * rs;
        int64_t in = 0, un = 0;
        for (int32_t w = 0; w < words; ++w) {
          in += __popc(bi[w] & bj[w]);
          un += __popc(bi[w] | bj[w]);
        }
        if (un < 1) un = 1;
        if (best < 0 || in * b_un > b_in * un) {
          best = j;
          b_in = in;
          b_un = un;
        }
      }
    }
    near[i] = best;
    move_to[bh * C + i] = -1;
    cut[bh * C + i] = sz[i];
  }
  __syncthreads();
  for (int32_t i = threadIdx.x; i < C; i += kTailThreads) {
    const int32_t j = near[i];
    if (j > i && near[j] == i) {
      const int32_t ti = sz[i] % block, tj = sz[j] % block;
      if (ti + tj <= block) {
        const int32_t d = ti < tj ? i : j, r = ti < tj ? j : i;
        move_to[bh * C + d] = r;
        cut[bh * C + d] = sz[d] - (sz[d] % block);
        uint32_t* br = bb + (int64_t)r * words;
        const uint32_t* bd = rb + (int64_t)d * rs;
        const uint32_t* bo = rb + (int64_t)r * rs;
        for (int32_t w = 0; w < words; ++w) br[w] = bo[w] | bd[w];
      }
    }
  }
}

// tokens of a donor at rank >= cut (its last members in token order) move
__global__ void __launch_bounds__(256)
move_kernel(int32_t* __restrict__ labels, const int32_t* __restrict__ slot,
            const int32_t* __restrict__ start, const int32_t* __restrict__ move_to,
            const int32_t* __restrict__ cut, int32_t N, int32_t C, int64_t total) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const int64_t bh = e / N;
  const int32_t c = labels[e];
  if (c < 0 || c >= C) return;
  const int32_t to = move_to[bh * C + c];
  if (to >= 0 && slot[e] - start[bh * (C + 1) + c] >= cut[bh * C + c]) labels[e] = to;
}

__global__ void __launch_bounds__(256)
popcount_kernel(const uint32_t* __restrict__ bits, int32_t* __restrict__ counts, int32_t words,
                int64_t rows) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  int32_t n = 0;
  for (int32_t w = 0; w < words; ++w) n += __popc(bits[r * words + w]);
  counts[r] = n;
}

}  // namespace

TailWs tail_ws_layout(int32_t bh, int32_t N, int32_t C, int32_t nk) {
  TailWs w{};
  w.words = (nk + 31) / 32;
  size_t off = 0;
  w.bits_off = off; off = align_up(off + (size_t)bh * C * w.words * 4, 256);
  w.rep_off = off; off = align_up(off + (size_t)bh * C * 4, 256);
  w.move_off = off; off = align_up(off + (size_t)bh * C * 4, 256);
  w.cut_off = off; off = align_up(off + (size_t)bh * C * 4, 256);
  w.counts_off = off; off = align_up(off + (size_t)bh * C * 4, 256);
  w.start_off = off; off = align_up(off + (size_t)bh * (C + 1) * 4, 256);
  w.sizes_off = off; off = align_up(off + (size_t)bh * C * 4, 256);
  w.slot_off = off; off = align_up(off + (size_t)bh * N * 4, 256);
  w.token_off = off; off = align_up(off + (size_t)bh * N * 4, 256);
  w.layout_off = off; off += layout_ws_bytes(bh, N, C);
  w.total = off;
  return w;
}

hipError_t launch_tail_merge(int32_t* labels, int32_t bh, int32_t N, int32_t C, int32_t nk,
                             int32_t block, int32_t rounds, const int32_t* row_ptr,
                             const int32_t* col_idx, int32_t* row_ptr_out, int32_t* col_idx_out,
                             void* ws, hipStream_t stream) {
  const TailWs w = tail_ws_layout(bh, N, C, nk);
  char* base = static_cast<char*>(ws);
  uint32_t* bits = reinterpret_cast<uint32_t*>(base + w.bits_off);
  int32_t* rep = reinterpret_cast<int32_t*>(base + w.rep_off);
  int32_t* move_to = reinterpret_cast<int32_t*>(base + w.move_off);
  int32_t* cut = reinterpret_cast<int32_t*>(base + w.cut_off);
  int32_t* counts = reinterpret_cast<int32_t*>(base + w.counts_off);
  int32_t* start = reinterpret_cast<int32_t*>(base + w.start_off);
  int32_t* sizes = reinterpret_cast<int32_t*>(base + w.sizes_off);
  int32_t* slot = reinterpret_cast<int32_t*>(base + w.slot_off);
  int32_t* token = reinterpret_cast<int32_t*>(base + w.token_off);
  void* lay_ws = base + w.layout_off;
  const int64_t rows = (int64_t)bh * C, total = (int64_t)bh * N;
  const uint32_t tblocks = (uint32_t)((total + 255) / 256);
  hipLaunchKernelGGL(rows_to_bits_kernel, dim3((uint32_t)rows), dim3(64), 0, stream, row_ptr,
                     col_idx, bits, nk, w.words);
  // bitmaps in LDS when the counters and one head's bitmaps fit in 64 KB
  const size_t lds = (size_t)C * 4 * (1 + lds_stride(w.words));
  const bool in_lds = lds <= 65536;
  const size_t shmem = in_lds ? lds : (size_t)C * 4;
  if (in_lds)
    hipLaunchKernelGGL(merge_kernel<true>, dim3((uint32_t)bh), dim3(kTailThreads), shmem, stream,
                       (const int32_t*)labels, N, C, (const uint32_t*)bits, w.words, rep);
  else
    hipLaunchKernelGGL(merge_kernel<false>, dim3((uint32_t)bh), dim3(kTailThreads), shmem, stream,
                       (const int32_t*)labels, N, C, (const uint32_t*)bits, w.words, rep);
  hipLaunchKernelGGL(relabel_kernel, dim3(tblocks), dim3(256), 0, stream, labels,
                     (const int32_t*)rep, N, C, total);
  for (int32_t r = 0; r < rounds; ++r) {
    hipError_t e = launch_cluster_layout(labels, bh, N, C, 1, start, sizes, slot, token, lay_ws,
                                         stream);
    if (e != hipSuccess) return e;
    if (in_lds)
      hipLaunchKernelGGL(pair_kernel<true>, dim3((uint32_t)bh), dim3(kTailThreads), shmem,
                         stream,
                         (const int32_t*)sizes, C, bits, w.words, block, move_to, cut);
    else
      hipLaunchKernelGGL(pair_kernel<false>, dim3((uint32_t)bh), dim3(kTailThreads), shmem,
                         stream,
                         (const int32_t*)sizes, C, bits, w.words, block, move_to, cut);
    hipLaunchKernelGGL(move_kernel, dim3(tblocks), dim3(256), 0, stream, labels,
                       (const int32_t*)slot, (const int32_t*)start, (const int32_t*)move_to,
                       (const int32_t*)cut, N, C, total);
  }
  hipLaunchKernelGGL(popcount_kernel, dim3((uint32_t)((rows + 255) / 256)), dim3(256), 0, stream,
                     (const uint32_t*)bits, counts, w.words, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_csr_from_bits(bits, counts, row_ptr_out, col_idx_out, rows, w.words, stream);
}

int64_t cluster_lcap(int32_t N, int32_t C, int32_t align) {
  return ((int64_t)N + (int64_t)C * (align - 1) + align - 1) / align * align;
}

size_t layout_ws_bytes(int32_t bh, int32_t N, int32_t C) {
  const int64_t tiles = (N + kLayTile - 1) / kLayTile;
  return align_up((size_t)bh * tiles * C * sizeof(int32_t), 256);
}

hipError_t launch_cluster_layout(const int32_t* labels, int32_t bh, int32_t N, int32_t C,
                                 int32_t align, int32_t* start, int32_t* sizes, int32_t* slot,
                                 int32_t* token, void* ws, hipStream_t stream) {
  const int32_t tiles = (N + kLayTile - 1) / kLayTile;
  const int64_t lcap = cluster_lcap(N, C, align);
  int32_t* tcount = static_cast<int32_t*>(ws);
  const size_t shmem = (size_t)C * sizeof(int32_t);
  hipLaunchKernelGGL(hist_kernel, dim3((uint32_t)tiles, (uint32_t)bh), dim3(kLayThreads), shmem,
                     stream, labels, N, C, tiles, tcount);
  hipLaunchKernelGGL(offsets_kernel, dim3((uint32_t)bh), dim3(kLayThreads), 0, stream, C, align,
                     tiles, tcount, start, sizes, token, lcap);
  hipLaunchKernelGGL(place_kernel, dim3((uint32_t)tiles, (uint32_t)bh), dim3(kLayThreads), shmem,
                     stream, labels, N, C, tiles, (const int32_t*)tcount, slot, token, lcap);
  return hipGetLastError();
}

hipError_t launch_cluster_means(const void* x, const int32_t* start, const int32_t* sizes,
                                const int32_t* token, double* cents, int32_t bh, int32_t N,
                                int32_t C, int32_t D, int64_t lcap, hipStream_t stream) {
  const int64_t total = (int64_t)bh * C;
  hipLaunchKernelGGL(means_kernel, dim3((uint32_t)((total + 3) / 4)), dim3(256), 0, stream,
                     (const uint16_t*)x, start, sizes, token, cents, N, C, D, lcap, total);
  return hipGetLastError();
}

hipError_t launch_cluster_metric(const double* cents, const int32_t* sizes, double* G, int32_t bh,
                                 int32_t C, int32_t D, hipStream_t stream) {
  const int32_t tiles = D / kMt;
  hipLaunchKernelGGL(metric_kernel, dim3((uint32_t)(bh * tiles * tiles)), dim3(256), 0, stream,
                     cents, sizes, G, C, D, tiles);
  return hipGetLastError();
}

KmeansWs kmeans_ws_layout(int32_t bh, int32_t N, int32_t C, int32_t D) {
  KmeansWs w{};
  size_t off = 0;
  w.g_hi_off = off; off = align_up(off + (size_t)bh * C * D * 2, 256);
  w.g_lo_off = off; off = align_up(off + (size_t)bh * C * D * 2, 256);
  w.cq_off = off;   off = align_up(off + (size_t)bh * C * 4, 256);
  w.start_off = off; off = align_up(off + (size_t)bh * (C + 1) * 4, 256);
  w.token_off = off; off = align_up(off + (size_t)bh * N * 4, 256);
  w.layout_off = off; off += layout_ws_bytes(bh, N, C);
  w.total = off;
  return w;
}

hipError_t launch_kmeans(const void* x, int32_t bh, int32_t N, int32_t D, const double* G,
                         double* cents, int32_t C, int32_t iters, int32_t* labels,
                         int32_t* sizes, void* ws, hipStream_t stream) {
  const KmeansWs w = kmeans_ws_layout(bh, N, C, D);
  char* base = static_cast<char*>(ws);
  uint16_t* g_hi = reinterpret_cast<uint16_t*>(base + w.g_hi_off);
  uint16_t* g_lo = reinterpret_cast<uint16_t*>(base + w.g_lo_off);
  float* cq = reinterpret_cast<float*>(base + w.cq_off);
  int32_t* start = reinterpret_cast<int32_t*>(base + w.start_off);
  int32_t* token = reinterpret_cast<int32_t*>(base + w.token_off);
  void* lay_ws = base + w.layout_off;
  const int32_t tiles = (N + kAsTok - 1) / kAsTok;
  const int32_t cgroups = (C + kPrepC - 1) / kPrepC;
  for (int32_t it = 0; it < iters; ++it) {
    hipLaunchKernelGGL(prep_kernel, dim3((uint32_t)((int64_t)bh * cgroups)), dim3(128), 0, stream,
                       (const double*)cents, G, g_hi, g_lo, cq, C, D, cgroups);
    if (D == 128)
      hipLaunchKernelGGL(assign_kernel<128>, dim3((uint32_t)((int64_t)bh * tiles)),
                         dim3(64 * kAsWaves), 0, stream, (const uint16_t*)x, g_hi, g_lo, cq,
                         labels, N, C, tiles);
    else
      hipLaunchKernelGGL(assign_kernel<64>, dim3((uint32_t)((int64_t)bh * tiles)),
                         dim3(64 * kAsWaves), 0, stream, (const uint16_t*)x, g_hi, g_lo, cq,
                         labels, N, C, tiles);
    hipError_t e =
        launch_cluster_layout(labels, bh, N, C, 1, start, sizes, nullptr, token, lay_ws, stream);
    if (e != hipSuccess) return e;
    e = launch_cluster_means(x, start, sizes, token, cents, bh, N, C, D, N, stream);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t launch_cluster_permute(const void* src, void* dst, int elt_bytes, int32_t bh,
                                  int32_t N, int32_t D, int32_t C, int64_t lcap,
                                  const int32_t* map, const int32_t* start, bool inverse,
                                  hipStream_t stream) {
  const int32_t chunks = D * elt_bytes / 16;
  int32_t shift = 0;
  while ((1 << shift) < chunks) ++shift;
  if ((1 << shift) != chunks) return hipErrorInvalidValue;
  constexpr int32_t kRows = 64;
  const int64_t rows = inverse ? N : lcap;
  const dim3 grid((uint32_t)((rows + kRows - 1) / kRows), (uint32_t)bh);
  if (inverse)
    hipLaunchKernelGGL(cluster_permute_kernel<1>, grid, dim3(256), 0, stream,
                       (const uint4*)src, (uint4*)dst, map, start, N, C, lcap, shift, kRows);
  else
    hipLaunchKernelGGL(cluster_permute_kernel<0>, grid, dim3(256), 0, stream,
                       (const uint4*)src, (uint4*)dst, map, start, N, C, lcap, shift, kRows);
  return hipGetLastError();
}

}  // namespace svsa
