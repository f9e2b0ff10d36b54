// Stage 3: block scores and top-p / fixed-fraction selection -> CSR lists.
//
// [SPADE] "SPADE: An Input-Adaptive Sparse Attention Engine for Fast Video
// Diffusion Models Inference", abstract: an Estimator over block summaries and
// a low-overhead index search.  [iCATS] "iCATS: Fast Video Generation via
// Interaction-Aware Sparse Attention and Timestep-Adaptive Sparsity",
// abstract and Sec. 3.2: the fixed top-p rule keeps the most important key
// regions until their cumulative importance reaches p.  [PSA] "Parameterized
// Stripe Attention for Efficient Video Generation", Alg. 1: a distance d lies
// inside a band of width w when d <= w - 1.
//
// Kernels (all float64 arithmetic, all deterministic):
//   logits_kernel   L = scale * Qbar Kbar^T, 64x64 output tile per workgroup
//   select_kernel   one workgroup per row: softmax, bitonic sort of
//                   (score desc, index asc) in LDS, ordered prefix sum, kept
//                   bitmap, row count
//   scan_kernel     exclusive scan of row counts -> row_ptr
//   compact_kernel  one wavefront per row: bitmap -> ascending col_idx
#include "svsa_internal.h"

namespace svsa {
namespace {

constexpr int kMaxHeads = 256;
constexpr int kMaxNb = 4096;

struct HeadParams {
  float v[kMaxHeads];  // top_p[h] or keep_frac[h]
};

// ---------------------------------------------------------------------------
// L[bh][i][j] = scale * sum_d qbar[bh][i][d] * kbar[bh][j][d]
// ---------------------------------------------------------------------------
constexpr int kTile = 64, kDc = 32, kLThreads = 256;

__global__ void __launch_bounds__(kLThreads)
logits_kernel(const double* __restrict__ qbar, const double* __restrict__ kbar,
              double* __restrict__ L, int32_t nb, int32_t D, double scale, int32_t tiles) {
  __shared__ double As[kDc][kTile + 1];
  __shared__ double Bs[kDc][kTile + 1];
  const int64_t bh = blockIdx.x / (tiles * tiles);
  const int32_t t2 = blockIdx.x % (tiles * tiles);
  const int32_t i0 = (t2 / tiles) * kTile, j0 = (t2 % tiles) * kTile;
  const double* qb = qbar + bh * nb * D;
  const double* kb = kbar + bh * nb * D;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;

  for (int32_t dc = 0; dc < D; dc += kDc) {
    const int dl = threadIdx.x % kDc;
    for (int r = threadIdx.x / kDc; r < kTile; r += kLThreads / kDc) {
      const bool dok = dc + dl < D;
      As[dl][r] = (i0 + r < nb && dok) ? qb[(int64_t)(i0 + r) * D + dc + dl] : 0.0;
      Bs[dl][r] = (j0 + r < nb && dok) ? kb[(int64_t)(j0 + r) * D + dc + dl] : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int d = 0; d < kDc; ++d) {
      double av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = As[d][ty + 16 * a];
#pragma unroll
      for (int b = 0; b < 4; ++b) bv[b] = Bs[d][tx + 16 * b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fma(av[a], bv[b], acc[a][b]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int32_t i = i0 + ty + 16 * a;
    if (i >= nb) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int32_t j = j0 + tx + 16 * b;
      if (j < nb) L[(bh * nb + i) * nb + j] = acc[a][b] * scale;
    }
  }
}

// ---------------------------------------------------------------------------
// Per-row selection.
// ---------------------------------------------------------------------------
constexpr int kSThreads = 256;

__device__ __forceinline__ bool comes_before(uint64_t ka, uint32_t ia, uint64_t kb, uint32_t ib) {
  return ka > kb || (ka == kb && ia < ib);
}

template <typename T, typename Op>
__device__ T block_reduce(T v, T* scratch, Op op) {
  // fixed-order tree over the kSThreads partial values
  scratch[threadIdx.x] = v;
  __syncthreads();
  for (int s = kSThreads / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) scratch[threadIdx.x] = op(scratch[threadIdx.x], scratch[threadIdx.x + s]);
    __syncthreads();
  }
  const T r = scratch[0];
  __syncthreads();
  return r;
}

// mode: 0 = top-p, 1 = fixed fraction
__global__ void __launch_bounds__(kSThreads)
select_kernel(const double* __restrict__ L, uint32_t* __restrict__ bits,
              int32_t* __restrict__ counts, int32_t nb, int32_t heads, int32_t p2, int32_t words,
              int32_t band, int32_t mode, HeadParams hp) {
  extern __shared__ uint64_t smem[];
  uint64_t* key = smem;                                  // [p2]
  double* red = reinterpret_cast<double*>(key + p2);     // [kSThreads]
  uint32_t* flag = reinterpret_cast<uint32_t*>(red + kSThreads);  // [words]
  uint16_t* idx = reinterpret_cast<uint16_t*>(flag + words);      // [p2]

  const int64_t r = blockIdx.x;
  const int32_t i = (int32_t)(r % nb);
  const int32_t h = (int32_t)((r / nb) % heads);
  const double* Lr = L + r * nb;
  const int t = threadIdx.x;

  // 1. row max
  double mx = -INFINITY;
  for (int32_t j = t; j < nb; j += kSThreads) mx = fmax(mx, Lr[j]);
  mx = block_reduce(mx, red, [](double a, double b) { return fmax(a, b); });

  // 2. e_j = exp(L_j - max), thread-sequential partial sums, fixed tree
  double part = 0.0;
  for (int32_t j = t; j < nb; j += kSThreads) {
    const double e = exp(Lr[j] - mx);
    key[j] = __double_as_longlong(e);
    part += e;
  }
  const double Z = block_reduce(part, red, [](double a, double b) { return a + b; });

  // 3. scores and sort keys (scores are >= 0, so their bits order like them)
  for (int32_t j = t; j < p2; j += kSThreads) {
    if (j < nb) {
      const double s = __longlong_as_double(key[j]) / Z;
      key[j] = (uint64_t)__double_as_longlong(s);
    } else {
      key[j] = 0;
    }
    idx[j] = (uint16_t)j;
  }
  for (int32_t w = t; w < words; w += kSThreads) flag[w] = 0u;
  __syncthreads();

  // 4. bitonic sort: descending score, ascending index on ties
  for (int32_t k = 2; k <= p2; k <<= 1) {
    for (int32_t j = k >> 1; j > 0; j >>= 1) {
      for (int32_t q = t; q < (p2 >> 1); q += kSThreads) {
        const int32_t a = (q / j) * 2 * j + (q % j);
        const int32_t b = a + j;
        const uint64_t ka = key[a], kb = key[b];
        const uint32_t ia = idx[a], ib = idx[b];
        const bool up = (a & k) == 0;
        const bool swap = up ? comes_before(kb, ib, ka, ia) : comes_before(ka, ia, kb, ib);
        if (swap) {
          key[a] = kb; key[b] = ka;
          idx[a] = (uint16_t)ib; idx[b] = (uint16_t)ia;
        }
      }
      __syncthreads();
    }
  }

  // 5. ordered exclusive prefix sums: each thread owns a contiguous run of ranks
  const int32_t per = p2 / kSThreads > 0 ? p2 / kSThreads : 1;
  const int32_t lo = t * per;
  double run = 0.0;
  for (int32_t q = lo; q < lo + per && q < p2; ++q) run += __longlong_as_double(key[q]);
  red[t] = run;
  __syncthreads();
  if (t == 0) {  // sequential scan of the run totals (fixed order)
    double acc = 0.0;
    for (int s = 0; s < kSThreads; ++s) {
      const double v = red[s];
      red[s] = acc;
      acc += v;
    }
  }
  __syncthreads();
  const double pval = (double)hp.v[h];
  int32_t keep_k = nb;
  if (mode == 1) {
    keep_k = (int32_t)ceil(pval * (double)nb);
    keep_k = max(1, min(keep_k, nb));
  }
  double excl = red[t];
  for (int32_t q = lo; q < lo + per && q < p2; ++q) {
    const uint32_t j = idx[q];
    bool kept;
    if (mode == 1) kept = q < keep_k;
    else kept = (pval >= 1.0) || q == 0 || excl < pval;
    if (kept && (int32_t)j < nb) atomicOr(&flag[j >> 5], 1u << (j & 31));
    excl += __longlong_as_double(key[q]);
  }
  // 6. diagonal band |i - j| <= band - 1
  for (int32_t d = t - (band - 1); d <= band - 1; d += kSThreads) {
    const int32_t j = i + d;
    if (j >= 0 && j < nb) atomicOr(&flag[j >> 5], 1u << (j & 31));
  }
  __syncthreads();

  // 7. bitmap out + count
  int32_t c = 0;
  for (int32_t w = t; w < words; w += kSThreads) {
    const uint32_t f = flag[w];
    bits[r * words + w] = f;
    c += __popc(f);
  }
  __syncthreads();
  int32_t* ired = reinterpret_cast<int32_t*>(red);
  const int32_t total = block_reduce(c, ired, [](int32_t a, int32_t b) { return a + b; });
  if (t == 0) counts[r] = total;
}

// ---------------------------------------------------------------------------
// row_ptr = exclusive scan of counts (one workgroup; rows fit comfortably)
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 1024;

__global__ void __launch_bounds__(kScanThreads)
scan_kernel(const int32_t* __restrict__ counts, int32_t* __restrict__ row_ptr, int64_t rows) {
  __shared__ int32_t buf[kScanThreads];
  int32_t carry = 0;
  for (int64_t base = 0; base < rows; base += kScanThreads) {
    const int64_t r = base + threadIdx.x;
    const int32_t v = r < rows ? counts[r] : 0;
    buf[threadIdx.x] = v;
    __syncthreads();
    for (int s = 1; s < kScanThreads; s <<= 1) {
      const int32_t add = threadIdx.x >= s ? buf[threadIdx.x - s] : 0;
      __syncthreads();
      buf[threadIdx.x] += add;
      __syncthreads();
    }
    if (r < rows) row_ptr[r] = carry + buf[threadIdx.x] - v;
    const int32_t chunk_total = buf[kScanThreads - 1];
    __syncthreads();
    carry += chunk_total;
  }
  if (threadIdx.x == 0) row_ptr[rows] = carry;
}

// ---------------------------------------------------------------------------
// bitmap -> ascending column indices, one wavefront per row
// ---------------------------------------------------------------------------
constexpr int kCThreads = 256;

__global__ void __launch_bounds__(kCThreads)
compact_kernel(const uint32_t* __restrict__ bits, const int32_t* __restrict__ row_ptr,
               int32_t* __restrict__ col_idx, int64_t rows, int32_t words) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * (kCThreads / 64) + (threadIdx.x >> 6);
  if (r >= rows) return;
  int32_t out = row_ptr[r];
  const uint32_t* br = bits + r * words;
  for (int32_t w0 = 0; w0 < words; w0 += 64) {
    const int32_t w = w0 + lane;
    uint32_t f = w < words ? br[w] : 0u;
    const int32_t c = __popc(f);
    // inclusive wave scan of c
    int32_t inc = c;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const int32_t o = __shfl_up(inc, s, 64);
      if (lane >= s) inc += o;
    }
    int32_t pos = out + inc - c;
    while (f) {
      const int b = __ffs(f) - 1;
      col_idx[pos++] = w * 32 + b;
      f &= f - 1;
    }
    out += __shfl(inc, 63, 64);
  }
}

}  // namespace

MaskWs mask_ws_layout(int64_t rows, int32_t nb) {
  MaskWs m{};
  m.words = (nb + 31) / 32;
  size_t off = 0;
  m.logits_off = off;
  off = align_up(off + (size_t)rows * nb * sizeof(double), 256);
  m.bits_off = off;
  off = align_up(off + (size_t)rows * m.words * sizeof(uint32_t), 256);
  m.counts_off = off;
  off = align_up(off + (size_t)rows * sizeof(int32_t), 256);
  m.total = off;
  return m;
}

hipError_t launch_block_mask(const double* qbar, const double* kbar, int32_t bh, int32_t heads,
                             int32_t nb, int32_t head_dim, double scale, const float* top_p,
                             const float* keep_frac, int32_t band, int32_t* row_ptr,
                             int32_t* col_idx, void* ws, hipStream_t stream) {
  if (heads > kMaxHeads || nb > kMaxNb) return hipErrorInvalidValue;
  const int64_t rows = (int64_t)bh * nb;
  const MaskWs m = mask_ws_layout(rows, nb);
  char* w = static_cast<char*>(ws);
  double* L = reinterpret_cast<double*>(w + m.logits_off);
  uint32_t* bits = reinterpret_cast<uint32_t*>(w + m.bits_off);
  int32_t* counts = reinterpret_cast<int32_t*>(w + m.counts_off);

  const int32_t tiles = (nb + kTile - 1) / kTile;
  const int64_t lblocks = (int64_t)bh * tiles * tiles;
  if (lblocks > 0x7fffffff || rows > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(logits_kernel, dim3((uint32_t)lblocks), dim3(kLThreads), 0, stream, qbar,
                     kbar, L, nb, head_dim, scale, tiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  HeadParams hp{};
  const float* src = top_p ? top_p : keep_frac;
  for (int32_t h = 0; h < heads; ++h) hp.v[h] = src[h];
  int32_t p2 = 1;
  while (p2 < nb) p2 <<= 1;
  if (p2 < 2) p2 = 2;
  const size_t lds = (size_t)p2 * sizeof(uint64_t) + kSThreads * sizeof(double) +
                     (size_t)m.words * sizeof(uint32_t) + (size_t)p2 * sizeof(uint16_t);
  hipLaunchKernelGGL(select_kernel, dim3((uint32_t)rows), dim3(kSThreads), lds, stream, L, bits,
                     counts, nb, heads, p2, m.words, band, top_p ? 0 : 1, hp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, counts, row_ptr, rows);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t cblocks = (rows + kCThreads / 64 - 1) / (kCThreads / 64);
  hipLaunchKernelGGL(compact_kernel, dim3((uint32_t)cblocks), dim3(kCThreads), 0, stream, bits,
                     row_ptr, col_idx, rows, m.words);
  return hipGetLastError();
}

}  // namespace svsa
