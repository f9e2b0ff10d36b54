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
//   logits_kernel   L = scale * Qbar Kbar^T on the float64 MFMA, 64x64 output
//                   tile per workgroup
//   select_kernel   one workgroup per row: softmax, radix select of the
//                   boundary block over the score bits with fixed-point mass
//                   histograms, kept bitmap, row count
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
// L[bh][i][j] = scale * sum_d qbar[bh][i][d] * kbar[bh][j][d], a dense float64
// contraction on the float64 matrix cores (v_mfma_f64_16x16x4f64).  128 x 128
// output tile per workgroup of 8 waves; wave w owns rows 32 (w / 2) .. +31 and
// columns 64 (w % 2) .. +63 as 2 x 4 tiles of 16 x 16.  Operand layout of the
// instruction: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16], and
// holds D[4 r + l / 16][l % 16] in its r-th result.  Q-bar and K-bar chunks of
// kDc dims go through LDS with an odd row stride (no bank conflicts on the
// 16-row operand reads).
// ---------------------------------------------------------------------------
constexpr int kTile = 128, kDc = 16, kLThreads = 512, kLdsStride = kDc + 1;
typedef double f64x4 __attribute__((ext_vector_type(4)));

// With ksizes (cluster mode) every logit of key cluster j gets + ln n_j, and
// empty key clusters get -inf.
__global__ void __launch_bounds__(kLThreads)
logits_kernel(const double* __restrict__ qbar, const double* __restrict__ kbar,
              const int32_t* __restrict__ ksizes, double* __restrict__ L, int32_t nq,
              int32_t nk, int32_t D, double scale, int32_t tiles_q, int32_t tiles_k) {
  __shared__ double As[kTile * kLdsStride];
  __shared__ double Bs[kTile * kLdsStride];
  // Workgroups go to the chip's 8 XCDs in turn (workgroup w to XCD w % 8).
  // Numbering the tiles XCD-major hands each XCD a contiguous run of them, so
  // the tiles of one (b, h) share one L2 instead of every XCD fetching that
  // head's Qbar and Kbar.  XCD x takes q + (x < r) tiles, q = G / 8, r = G % 8.
  const uint32_t G = gridDim.x, q8 = G / 8, r8 = G % 8, x8 = blockIdx.x % 8;
  const uint32_t wg = x8 * q8 + min(x8, r8) + blockIdx.x / 8;
  const int64_t bh = wg / (tiles_q * tiles_k);
  const int32_t t2 = wg % (tiles_q * tiles_k);
  const int32_t i0 = (t2 / tiles_k) * kTile, j0 = (t2 % tiles_k) * kTile;
  const double* qb = qbar + bh * nq * D;
  const double* kb = kbar + bh * nk * D;
  const int32_t wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int32_t wr = 32 * (wave / 2), wc = 64 * (wave % 2);
  const int32_t lr = lane % 16, lk = lane / 16;
  f64x4 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};

  // Operand chunks (rows i0 .. i0 + kTile - 1 and j0 .. j0 + kTile - 1, kDc
  // dims) are loaded into registers one chunk ahead, so the global loads of
  // chunk c + 1 are in flight while the MFMAs of chunk c run.
  constexpr int kPerThread = kTile * kDc / kLThreads;
  static_assert(kTile * kDc % kLThreads == 0, "whole staging rounds");
  double pa[kPerThread], pb[kPerThread];
  auto load_chunk = [&](int32_t dc) {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int32_t e = threadIdx.x + u * kLThreads;
      const int32_t r = e / kDc, d = e % kDc;
      const bool dok = dc + d < D;
      pa[u] = (i0 + r < nq && dok) ? qb[(int64_t)(i0 + r) * D + dc + d] : 0.0;
      pb[u] = (j0 + r < nk && dok) ? kb[(int64_t)(j0 + r) * D + dc + d] : 0.0;
    }
  };
  load_chunk(0);
  for (int32_t dc = 0; dc < D; dc += kDc) {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int32_t e = threadIdx.x + u * kLThreads;
      const int32_t r = e / kDc, d = e % kDc;
      As[r * kLdsStride + d] = pa[u];
      Bs[r * kLdsStride + d] = pb[u];
    }
    __syncthreads();
    if (dc + kDc < D) load_chunk(dc + kDc);
#pragma unroll
    for (int ks = 0; ks < kDc / 4; ++ks) {
      const int32_t d = 4 * ks + lk;
      double av[2], bv[4];
#pragma unroll
      for (int a = 0; a < 2; ++a) av[a] = As[(wr + 16 * a + lr) * kLdsStride + d];
#pragma unroll
      for (int b = 0; b < 4; ++b) bv[b] = Bs[(wc + 16 * b + lr) * kLdsStride + d];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int32_t i = i0 + wr + 16 * a + 4 * r + lk;
      if (i >= nq) continue;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int32_t j = j0 + wc + 16 * b + lr;
        if (j >= nk) continue;
        double v = acc[a][b][r] * scale;
        if (ksizes) {
          const int32_t n = ksizes[bh * nk + j];
          v = n > 0 ? v + log((double)n) : -INFINITY;
        }
        L[(bh * nq + i) * nk + j] = v;
      }
    }
}

// ---------------------------------------------------------------------------
// Per-row selection by radix select (no sort).
//
// The kept set is a prefix of the (score desc, index asc) order, so it is
// fixed by its last element tau: every block scoring above tau is kept, and
// of the blocks scoring exactly tau the lowest-index ones up to the boundary.
// tau is found by an MSB-first radix select over the score bits (non-negative
// doubles order like their bit patterns), 8 bits per pass starting below the
// bits that all of the row's keys share, with a per-bin histogram of counts
// and of probability mass.  Mass is accumulated in 2^-63 fixed point with
// integer atomics, so the result is independent of the order of the atomics
// (bitwise deterministic); it differs from a float64 running sum by at most
// nb * 2^-63.  Most rows resolve in 2-3 passes (the boundary bin holds a
// single block).
// ---------------------------------------------------------------------------
constexpr int kSThreads = 256;

// Fixed-order reduction over the kSThreads (= 4 wavefronts) partial values: a
// butterfly inside each wavefront (every lane ends with the same value, as
// the operations are commutative), then the four wavefront results in index
// order.
static_assert(kSThreads == 256, "block_reduce combines four wavefronts");
template <typename T, typename Op>
__device__ T block_reduce(T v, T* scratch, Op op) {
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) v = op(v, __shfl_xor(v, s, 64));
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  const T r = op(op(scratch[0], scratch[1]), op(scratch[2], scratch[3]));
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint64_t to_fixed(double s) {
  return (uint64_t)(s * 9223372036854775808.0);  // floor(s * 2^63)
}

struct RadixStep {
  int32_t bin;          // crossing bin, -1 when the target is never reached
  uint32_t bin_cnt;     // elements in that bin
  uint32_t above_cnt;   // elements ranked before the bin
  uint64_t above_mass;  // their fixed-point mass
};

// mode: 0 = top-p, 1 = fixed fraction.  PER = elements per thread (nb <= 256 * PER).
// Rows r = (bh, i) with nq rows per head; nb columns (key blocks or clusters).
template <int PER>
__global__ void __launch_bounds__(kSThreads)
select_kernel(const double* __restrict__ L, uint32_t* __restrict__ bits,
              int32_t* __restrict__ counts, int32_t nq, int32_t nb, int32_t heads,
              int32_t words, int32_t band, int32_t mode, HeadParams hp) {
  __shared__ uint32_t hcnt[256];
  __shared__ unsigned long long hmass[256];
  __shared__ double red[4];   // one partial value per wavefront
  __shared__ uint32_t flag[kMaxNb / 32];
  __shared__ uint32_t tie[kMaxNb / 32];
  __shared__ RadixStep res;

  const int64_t r = blockIdx.x;
  const int32_t i = (int32_t)(r % nq);
  const int32_t h = (int32_t)((r / nq) % heads);
  const double* Lr = L + r * nb;
  const int t = threadIdx.x, lane = t & 63;

  // 1. softmax of the row, elements j = t + 256 k held in registers
  double x[PER];
  double mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int32_t j = t + k * kSThreads;
    x[k] = j < nb ? Lr[j] : -INFINITY;
    mx = fmax(mx, x[k]);
  }
  mx = block_reduce(mx, red, [](double a, double b) { return fmax(a, b); });
  double part = 0.0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int32_t j = t + k * kSThreads;
    x[k] = j < nb ? exp(x[k] - mx) : 0.0;
    part += x[k];
  }
  const double Z = block_reduce(part, red, [](double a, double b) { return a + b; });
  uint64_t key[PER], mass[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const double sc = x[k] / Z;
    key[k] = (uint64_t)__double_as_longlong(sc);
    mass[k] = to_fixed(sc);
  }

  // 2. targets
  const double pval = (double)hp.v[h];
  uint64_t P = 0;
  int32_t K = nb;
  bool keep_all;
  if (mode == 1) {
    K = max(1, min((int32_t)ceil(pval * (double)nb), nb));
    keep_all = K >= nb;
  } else {
    keep_all = pval >= 1.0;
    P = (uint64_t)ceil(pval * 9223372036854775808.0);
  }

  // 3. radix select of the boundary element.  The scores of a row share their
  // leading key bits (sign and high exponent bits), so the digits start below
  // the bits common to the row's smallest and largest key: 8-bit digits, the
  // last one narrower.  Keys of non-negative doubles have bit 63 clear, so at
  // least one bit is common.  A row of equal keys runs no pass and goes to the
  // tie rule with every element in the boundary bin.
  uint64_t kmin = ~0ull, kmax = 0ull;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int32_t j = t + k * kSThreads;
    if (j < nb) {
      kmin = key[k] < kmin ? key[k] : kmin;
      kmax = key[k] > kmax ? key[k] : kmax;
    }
  }
  unsigned long long* ured = reinterpret_cast<unsigned long long*>(red);
  kmin = block_reduce((unsigned long long)kmin, ured,
                      [](unsigned long long a, unsigned long long b) { return a < b ? a : b; });
  kmax = block_reduce((unsigned long long)kmax, ured,
                      [](unsigned long long a, unsigned long long b) { return a > b ? a : b; });
  int shift = kmin == kmax ? 0 : 64 - __clzll((long long)(kmin ^ kmax));
  uint64_t prefix = kmax >> shift, A = 0;
  uint32_t C = 0;
  bool resolved = false;
  uint32_t last_cnt = (uint32_t)nb;
  while (!keep_all && shift > 0) {
    const int w = shift < 8 ? shift : 8;   // digit width
    shift -= w;
    hcnt[t] = 0u;
    hmass[t] = 0ull;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int32_t j = t + k * kSThreads;
      if (j < nb && (key[k] >> (shift + w)) == prefix) {
        const uint32_t b = (uint32_t)(key[k] >> shift) & ((1u << w) - 1u);
        atomicAdd(&hcnt[b], 1u);
        atomicAdd(&hmass[b], (unsigned long long)mass[k]);
      }
    }
    __syncthreads();
    if (t < 64) {
      // lane holds positions 4 lane .. 4 lane + 3 of the descending bin order
      uint64_t ms[4], im[4];
      uint32_t cs[4], ic[4];
      uint64_t lm = 0;
      uint32_t lc = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int b = 255 - (4 * lane + q);
        ms[q] = hmass[b];
        cs[q] = hcnt[b];
        lm += ms[q];
        lc += cs[q];
        im[q] = lm;
        ic[q] = lc;
      }
      uint64_t pm = lm;
      uint32_t pc = lc;
#pragma unroll
      for (int s = 1; s < 64; s <<= 1) {
        const uint64_t om = __shfl_up(pm, s, 64);
        const uint32_t oc = __shfl_up(pc, s, 64);
        if (lane >= s) {
          pm += om;
          pc += oc;
        }
      }
      pm -= lm;  // exclusive over lanes
      pc -= lc;
      int first = -1;
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        const bool cross = mode == 1 ? (C + pc + ic[q] >= (uint32_t)K) : (A + pm + im[q] >= P);
        if (cross) first = q;
      }
      const unsigned long long bal = __ballot(first >= 0);
      if (bal == 0ull) {
        if (lane == 0) res.bin = -1;
      } else if (lane == __ffsll((long long)bal) - 1) {
        res.bin = 255 - (4 * lane + first);
        res.bin_cnt = cs[first];
        res.above_cnt = C + pc + ic[first] - cs[first];
        res.above_mass = A + pm + im[first] - ms[first];
      }
    }
    __syncthreads();
    const RadixStep st = res;
    if (st.bin < 0) {  // total mass below p (rounding): every block is kept
      keep_all = true;
      break;
    }
    prefix = (prefix << w) | (uint64_t)st.bin;
    A = st.above_mass;
    C = st.above_cnt;
    last_cnt = st.bin_cnt;
    if (st.bin_cnt == 1u) resolved = true;
    __syncthreads();
    if (resolved) break;
  }

  // 4. kept flags
  for (int32_t w = t; w < words; w += kSThreads) {
    flag[w] = 0u;
    tie[w] = 0u;
  }
  __syncthreads();
  uint32_t k_tie = 0;
  if (!keep_all && !resolved) {  // exact ties at tau: lowest indices first
    if (mode == 1) {
      k_tie = (uint32_t)K - C;
    } else {
      const uint64_t m_tau = to_fixed(__longlong_as_double((long long)prefix));
      const uint64_t need = P - A;
      k_tie = (uint32_t)((need + m_tau - 1) / m_tau);
    }
    k_tie = max(1u, min(k_tie, last_cnt));
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int32_t j = t + k * kSThreads;
    if (j >= nb) continue;
    bool kept;
    if (keep_all) {
      kept = true;
    } else {
      const uint64_t hi = key[k] >> shift;
      kept = hi > prefix || (hi == prefix && resolved);
      if (hi == prefix && !resolved) atomicOr(&tie[j >> 5], 1u << (j & 31));
    }
    if (kept) atomicOr(&flag[j >> 5], 1u << (j & 31));
  }
  // diagonal band |i - j| <= band - 1
  for (int32_t d = t - (band - 1); d <= band - 1; d += kSThreads) {
    const int32_t j = i + d;
    if (j >= 0 && j < nb) atomicOr(&flag[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  if (k_tie > 0 && t == 0) {
    uint32_t taken = 0;
    for (int32_t w = 0; w < words && taken < k_tie; ++w) {
      uint32_t f = tie[w];
      while (f && taken < k_tie) {
        const uint32_t lowbit = f & (~f + 1u);
        flag[w] |= lowbit;
        f ^= lowbit;
        ++taken;
      }
    }
  }
  __syncthreads();

  // 5. bitmap out + count
  int32_t c = 0;
  for (int32_t w = t; w < words; w += kSThreads) {
    const uint32_t f = flag[w];
    bits[r * words + w] = f;
    c += __popc(f);
  }
  int32_t* ired = reinterpret_cast<int32_t*>(red);
  const int32_t total = block_reduce(c, ired, [](int32_t a, int32_t b) { return a + b; });
  if (t == 0) counts[r] = total;
  (void)lane;
}

// ---------------------------------------------------------------------------
// row_ptr = exclusive scan of counts (one workgroup; rows fit comfortably)
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 1024;

__global__ void __launch_bounds__(kScanThreads)
scan_kernel(const int32_t* __restrict__ counts, int32_t* __restrict__ row_ptr, int64_t rows) {
  __shared__ int32_t wsum[kScanThreads / 64];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  constexpr int kPer = 4;
  constexpr int kChunk = kScanThreads * kPer;
  int32_t carry = 0;
  for (int64_t base = 0; base < rows; base += kChunk) {
    int32_t v[kPer];
    int32_t local = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int64_t r = base + (int64_t)t * kPer + q;
      v[q] = r < rows ? counts[r] : 0;
      local += v[q];
    }
    int32_t inc = local;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const int32_t o = __shfl_up(inc, s, 64);
      if (lane >= s) inc += o;
    }
    if (lane == 63) wsum[wv] = inc;
    __syncthreads();
    int32_t wbase = 0, total = 0;
    for (int k = 0; k < kScanThreads / 64; ++k) {
      const int32_t x = wsum[k];
      if (k < wv) wbase += x;
      total += x;
    }
    int32_t run = carry + wbase + inc - local;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int64_t r = base + (int64_t)t * kPer + q;
      if (r < rows) row_ptr[r] = run;
      run += v[q];
    }
    carry += total;
    __syncthreads();
  }
  if (t == 0) row_ptr[rows] = carry;
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

hipError_t launch_csr_from_bits(const uint32_t* bits, const int32_t* counts, int32_t* row_ptr,
                                int32_t* col_idx, int64_t rows, int32_t words,
                                hipStream_t stream) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, counts, row_ptr, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t cblocks = (rows + kCThreads / 64 - 1) / (kCThreads / 64);
  hipLaunchKernelGGL(compact_kernel, dim3((uint32_t)cblocks), dim3(kCThreads), 0, stream, bits,
                     row_ptr, col_idx, rows, words);
  return hipGetLastError();
}

MaskWs mask_ws_layout(int64_t rows, int32_t nb) {
  // rows x nb logits (nb = columns: key blocks or key clusters)
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
  return launch_cluster_mask(qbar, kbar, nullptr, bh, heads, nb, nb, head_dim, scale, top_p,
                             keep_frac, band, row_ptr, col_idx, ws, stream);
}

hipError_t launch_cluster_mask(const double* qbar, const double* kbar, const int32_t* ksizes,
                               int32_t bh, int32_t heads, int32_t nq, int32_t nb,
                               int32_t head_dim, double scale, const float* top_p,
                               const float* keep_frac, int32_t band, int32_t* row_ptr,
                               int32_t* col_idx, void* ws, hipStream_t stream) {
  if (heads > kMaxHeads || nb > kMaxNb) return hipErrorInvalidValue;
  const int64_t rows = (int64_t)bh * nq;
  const MaskWs m = mask_ws_layout(rows, nb);
  char* w = static_cast<char*>(ws);
  double* L = reinterpret_cast<double*>(w + m.logits_off);
  uint32_t* bits = reinterpret_cast<uint32_t*>(w + m.bits_off);
  int32_t* counts = reinterpret_cast<int32_t*>(w + m.counts_off);

  const int32_t tiles_q = (nq + kTile - 1) / kTile, tiles_k = (nb + kTile - 1) / kTile;
  const int64_t lblocks = (int64_t)bh * tiles_q * tiles_k;
  if (lblocks > 0x7fffffff || rows > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(logits_kernel, dim3((uint32_t)lblocks), dim3(kLThreads), 0, stream, qbar,
                     kbar, ksizes, L, nq, nb, head_dim, scale, tiles_q, tiles_k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  HeadParams hp{};
  const float* src = top_p ? top_p : keep_frac;
  for (int32_t h = 0; h < heads; ++h) hp.v[h] = src[h];
  const int mode = top_p ? 0 : 1;
  const dim3 grid((uint32_t)rows), blk(kSThreads);
  if (nb <= kSThreads)
    hipLaunchKernelGGL(select_kernel<1>, grid, blk, 0, stream, L, bits, counts, nq, nb, heads,
                       m.words, band, mode, hp);
  else if (nb <= 2 * kSThreads)
    hipLaunchKernelGGL(select_kernel<2>, grid, blk, 0, stream, L, bits, counts, nq, nb, heads,
                       m.words, band, mode, hp);
  else if (nb <= 4 * kSThreads)
    hipLaunchKernelGGL(select_kernel<4>, grid, blk, 0, stream, L, bits, counts, nq, nb, heads,
                       m.words, band, mode, hp);
  else if (nb <= 8 * kSThreads)
    hipLaunchKernelGGL(select_kernel<8>, grid, blk, 0, stream, L, bits, counts, nq, nb, heads,
                       m.words, band, mode, hp);
  else
    hipLaunchKernelGGL(select_kernel<16>, grid, blk, 0, stream, L, bits, counts, nq, nb, heads,
                       m.words, band, mode, hp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_csr_from_bits(bits, counts, row_ptr, col_idx, rows, m.words, stream);
}

}  // namespace svsa
