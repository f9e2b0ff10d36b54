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
//   logits_kernel   L = scale * Qbar Kbar^T on the float64 MFMA, 128x128 output
//                   tile per workgroup
//   select_kernel   one workgroup per row: softmax, radix select of the
//                   boundary block over the score bits with fixed-point mass
//                   histograms, kept bitmap, row count (rows of more than
//                   2048 columns)
//   select_wave_kernel  the same, one wavefront per row (up to 2048 columns)
//   scan_kernel     exclusive scan of row counts -> row_ptr
//   compact_kernel  one wavefront per row: bitmap -> ascending col_idx
#include <mutex>

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
// At most 128 VGPRs (4 waves per SIMD), so two workgroups share a CU and one's
// first loads and last stores overlap the other's MFMAs: 0.38 -> 0.33 ms at
// Wan2.1 720p.  The 16-dim chunk is walked one 4-dim step at a time (not
// unrolled) to stay within that budget without spills.
__global__ void __launch_bounds__(kLThreads, 4)
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
  const int32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
  const int32_t wr = 32 * (wave / 2), wc = 64 * (wave % 2);
  const int32_t lr = lane % 16, lk = lane / 16;
  // 16 x 16 result tiles of this wave that hold any row < nq and column < nk
  // (a prefix of a and of b): in the last tile row / column of a head the
  // others are skipped on the matrix cores.  The tiles that run keep the
  // accumulation order of a full tile, so every stored logit is unchanged.
  const int32_t na = min(2, max(0, (nq - i0 - wr + 15) / 16));
  const int32_t nbt = min(4, max(0, (nk - j0 - wc + 15) / 16));
  const bool full = na == 2 && nbt == 4;
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
    if (na > 0 && nbt > 0) {
#pragma unroll 1
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
            if (full || (a < na && b < nbt))  // wave-uniform
              acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
      }
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

// ---------------------------------------------------------------------------
// Wavefront-wide combines in registers, without LDS: DPP moves within rows of
// 16 lanes and gfx950's lane-swap permutes across rows and halves.
//
// xchg<S>: the value of a partner lane, step S of a butterfly: lane ^ 1 and
// lane ^ 2 (DPP quad permutes), the mirror lane within 8 and within 16 lanes
// (DPP row half-mirror and mirror: after the earlier steps every lane of a
// quad, then of 8 lanes, holds the same partial, so the mirror pairs whole
// groups as an xor would), lane ^ 16 and lane ^ 32 (permlane swaps).
// ---------------------------------------------------------------------------
template <int S>
__device__ __forceinline__ uint32_t xchg32(uint32_t x, int lane) {
  if constexpr (S == 0) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);  // quad [1,0,3,2]
  } else if constexpr (S == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);  // quad [2,3,0,1]
  } else if constexpr (S == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false);  // row_half_mirror
  } else if constexpr (S == 3) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, false);  // row_mirror
  } else if constexpr (S == 4) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return lane < 32 ? r[1] : r[0];
  }
}
template <int S, typename T>
__device__ __forceinline__ T xchg(T v, int lane) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, xchg32<S>(__builtin_bit_cast(uint32_t, v), lane));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = xchg32<S>((uint32_t)u, lane), hi = xchg32<S>((uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  }
}
// op over the 64 lanes, every lane ends with the result (op commutative and
// associative on the values combined; a float sum follows this fixed tree).
// The whole wavefront must be active.
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  const int lane = (int)(threadIdx.x & 63);
  v = op(v, xchg<0>(v, lane));
  v = op(v, xchg<1>(v, lane));
  v = op(v, xchg<2>(v, lane));
  v = op(v, xchg<3>(v, lane));
  v = op(v, xchg<4>(v, lane));
  v = op(v, xchg<5>(v, lane));
  return v;
}
// inclusive prefix sum over the 64 lanes (integers): shifts by 1, 2, 4, 8
// within each row of 16 (DPP row_shr; lanes without a source add 0), then
// row 0's total into row 1 and row 2's into row 3 (row_bcast:15), then the
// total of rows 0-1 into rows 2-3 (row_bcast:31).  The whole wavefront must
// be active.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, kRowMask, 0xF, false);
}
template <int kCtrl, int kRowMask, typename T>
__device__ __forceinline__ T dpp_or_zero_t(T v) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, dpp_or_zero<kCtrl, kRowMask>(__builtin_bit_cast(uint32_t, v)));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = dpp_or_zero<kCtrl, kRowMask>((uint32_t)u);
    const uint32_t hi = dpp_or_zero<kCtrl, kRowMask>((uint32_t)(u >> 32));
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  }
}
template <typename T>
__device__ __forceinline__ T wave_inclusive_sum(T v) {
  v += dpp_or_zero_t<0x111, 0xF>(v);  // row_shr:1
  v += dpp_or_zero_t<0x112, 0xF>(v);  // row_shr:2
  v += dpp_or_zero_t<0x114, 0xF>(v);  // row_shr:4
  v += dpp_or_zero_t<0x118, 0xF>(v);  // row_shr:8
  v += dpp_or_zero_t<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_or_zero_t<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}
// the value of lane src (wave-uniform), read into a scalar register
template <typename T>
__device__ __forceinline__ T lane_value(T v, int src) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, src);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), src);
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  }
}

// Fixed-order reduction over the kSThreads (= 4 wavefronts) partial values: a
// fixed tree inside each wavefront (wave_reduce; every lane ends with the same
// value), then the four wavefront results in index order.
static_assert(kSThreads == 256, "block_reduce combines four wavefronts");
template <typename T, typename Op>
__device__ T block_reduce(T v, T* scratch, Op op) {
  v = wave_reduce(v, op);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  const T r = op(op(scratch[0], scratch[1]), op(scratch[2], scratch[3]));
  __syncthreads();
  return r;
}

// e^t for t <= 0 (or -inf), to about one ulp.  Cody and Waite's argument
// reduction: t = n ln2 + r with n = rint(t / ln2), ln2 split into a high part
// of 32 significant bits (so n times it is exact for |n| < 2^21) and the
// remainder, leaving |r| <= ln2 / 2 (about).  e^r is the Taylor series to
// degree 13 (remainder below 6e-18, 0.05 ulp) by Horner's rule with fused
// multiply-adds, and e^t = 2^n e^r by ldexp, which rounds once when the result
// lands among the subnormals.  Arguments below -1100 are clamped there (e^-1100
// underflows to +0, as does e^-inf).  It needs none of the general exp's
// overflow and special-case code.  The constants live in scalar registers,
// set up once per thread (ExpConst), so each Horner step is one instruction.
struct ExpConst {
  double c[17];  // 1 / ln 2, ln 2 high part, ln 2 remainder, then 1 / k! for k = 13 .. 0
  __device__ __forceinline__ ExpConst() {
    constexpr double kInit[17] = {
        1.4426950408889634, 0.6931471806019545, -4.2009150726810846e-11,
        1.0 / 6227020800.0, 1.0 / 479001600.0, 1.0 / 39916800.0, 1.0 / 3628800.0,
        1.0 / 362880.0, 1.0 / 40320.0, 1.0 / 5040.0, 1.0 / 720.0, 1.0 / 120.0, 1.0 / 24.0,
        1.0 / 6.0, 0.5, 1.0, 1.0};
#pragma unroll
    for (int k = 0; k < 17; ++k) {
      c[k] = kInit[k];
      // opaque scalar: keeps the value in an SGPR pair as the fma's addend
      // instead of re-materialising it into VGPRs at every use
      asm volatile("" : "+s"(c[k]));
    }
  }
};

__device__ __forceinline__ double exp_nonpos(double t, const ExpConst& e) {
  t = fmax(t, -1100.0);
  const double n = rint(t * e.c[0]);
  double r = fma(-n, e.c[1], t);
  r = fma(-n, e.c[2], r);
  double p = e.c[3];
#pragma unroll
  for (int k = 4; k < 17; ++k) p = fma(p, r, e.c[k]);
  return ldexp(p, (int)n);
}

// x / z for 0 <= x <= z (z >= 1: the softmax denominator), with 1 / z shared
// by every element of a row: q0 = x r with r = 1 / z correctly rounded, then
// one correction by the remainder x - q0 z (exact in a fused multiply-add),
// q = q0 + (x - q0 z) r.  By Markstein's division theorem (r within half an
// ulp of 1 / z, q0 within one ulp of x / z) q is the correctly rounded
// quotient, i.e. the same double as x / z, whenever that is a normal number:
// three instructions per element instead of a dozen.  A nonzero x whose
// quotient falls below 2^-1000, where the remainder may not be exact, is
// flagged by div_needs_plain and its caller divides it plainly.
struct SharedDivisor {
  double z, r;
  __device__ __forceinline__ explicit SharedDivisor(double zz) : z(zz), r(1.0 / zz) {}
};
__device__ __forceinline__ double div_shared(double x, const SharedDivisor& d) {
  const double q0 = x * d.r;
  return fma(fma(-q0, d.z, x), d.r, q0);
}
__device__ __forceinline__ bool div_needs_plain(double x, double q) {
  return x > 0.0 && q < 0x1p-1000;
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
// L holds the logits of rows row0 .. row0 + gridDim.x - 1 (row r at L[(r - row0) * nb]);
// bits and counts are indexed by the global row r.
template <int PER>
__global__ void __launch_bounds__(kSThreads)
select_kernel(const double* __restrict__ L, uint32_t* __restrict__ bits,
              int32_t* __restrict__ counts, int32_t nq, int32_t nb, int32_t heads,
              int32_t words, int32_t band, int32_t mode, HeadParams hp, int64_t row0) {
  __shared__ uint32_t hcnt[256];
  __shared__ unsigned long long hmass[256];
  __shared__ double red[4];   // one partial value per wavefront
  __shared__ uint32_t flag[kMaxNb / 32];
  __shared__ uint32_t tie[kMaxNb / 32];
  __shared__ RadixStep res;

  const int64_t r = row0 + blockIdx.x;
  const int32_t i = (int32_t)(r % nq);
  const int32_t h = (int32_t)((r / nq) % heads);
  const double* Lr = L + (int64_t)blockIdx.x * nb;
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
  const ExpConst ec;
  double part = 0.0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int32_t j = t + k * kSThreads;
    x[k] = j < nb ? exp_nonpos(x[k] - mx, ec) : 0.0;
    part += x[k];
  }
  const double Z = block_reduce(part, red, [](double a, double b) { return a + b; });
  uint64_t key[PER], mass[PER];
  const SharedDivisor dz(Z);
  bool plain = false;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const double q = div_shared(x[k], dz);
    plain |= div_needs_plain(x[k], q);
    x[k] = q;
  }
  if (__builtin_amdgcn_ballot_w64(plain) != 0) {
    // rare (a quotient among the subnormals): those elements again, by plain division
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int32_t j = t + k * kSThreads;
      const double e = j < nb ? exp_nonpos(Lr[j] - mx, ec) : 0.0;
      if (div_needs_plain(e, x[k])) x[k] = e / Z;
    }
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const double sc = x[k];
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
      uint64_t pm = wave_inclusive_sum(lm);   // wavefront 0 only, whole
      uint32_t pc = wave_inclusive_sum(lc);
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
// The same selection with one wavefront per row (nb <= 64 * PER <= 2048):
// every reduction, the histograms and the search for the crossing bin stay
// inside the wavefront, so a row needs no workgroup barrier, and four rows
// share a workgroup.  Each lane holds the score keys of columns
// j = lane + 64 k; a key's fixed-point mass is recomputed from it when a pass
// needs it.  The softmax sums in another order than select_kernel's (lanes,
// then one wavefront's fixed tree, against four wavefronts' trees and their
// results in order), so Z, and with it a score's last bits, can differ from
// that kernel's; every step after Z is the same.
// ---------------------------------------------------------------------------
constexpr int kWRows = 4;          // rows (wavefronts) per workgroup
constexpr int kWMaxWords = 64;     // bitmap words of a row: nb <= 2048

// LDS accesses of one wavefront stay in program order; this keeps the
// compiler from moving them across the points where other lanes' results
// are read.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int PER>
__global__ void __launch_bounds__(64 * kWRows) __attribute__((amdgpu_waves_per_eu(PER <= 20 ? 3 : 1)))
select_wave_kernel(const double* __restrict__ L, uint32_t* __restrict__ bits,
                   int32_t* __restrict__ counts, int32_t nq, int32_t nb, int32_t heads,
                   int32_t words, int32_t band, int32_t mode, HeadParams hp, int64_t row0,
                   int64_t nrows) {
  __shared__ uint32_t hcnt_s[kWRows][256];
  __shared__ unsigned long long hmass_s[kWRows][256];
  __shared__ uint32_t flag_s[kWRows][kWMaxWords];
  __shared__ uint32_t tie_s[kWRows][kWMaxWords];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t rl = (int64_t)blockIdx.x * kWRows + wv;  // row of this launch
  if (rl >= nrows) return;                               // whole wavefront
  uint32_t* hcnt = hcnt_s[wv];
  unsigned long long* hmass = hmass_s[wv];
  uint32_t* flag = flag_s[wv];
  uint32_t* tie = tie_s[wv];
  const int64_t r = row0 + rl;
  const int32_t i = (int32_t)(r % nq);
  const int32_t h = (int32_t)((r / nq) % heads);
  const double* Lr = L + rl * nb;

  // 1. softmax of the row
  double x[PER];
  double mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int32_t j = lane + 64 * k;
    x[k] = j < nb ? Lr[j] : -INFINITY;
    mx = fmax(mx, x[k]);
  }
  mx = wave_reduce(mx, [](double a, double b) { return fmax(a, b); });
  const ExpConst ec;
  double part = 0.0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int32_t j = lane + 64 * k;
    x[k] = j < nb ? exp_nonpos(x[k] - mx, ec) : 0.0;
    part += x[k];
  }
  const double Z = wave_reduce(part, [](double a, double b) { return a + b; });
  uint64_t key[PER];
  const SharedDivisor dz(Z);
  bool plain = false;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const double q = div_shared(x[k], dz);
    plain |= div_needs_plain(x[k], q);
    x[k] = q;
  }
  if (__builtin_amdgcn_ballot_w64(plain) != 0) {
    // rare (a quotient among the subnormals): those elements again, by plain division
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int32_t j = lane + 64 * k;
      const double e = j < nb ? exp_nonpos(Lr[j] - mx, ec) : 0.0;
      if (div_needs_plain(e, x[k])) x[k] = e / Z;
    }
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) key[k] = (uint64_t)__double_as_longlong(x[k]);

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

  // 3. radix select of the boundary element (as in select_kernel)
  unsigned long long kmin = ~0ull, kmax = 0ull;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (lane + 64 * k < nb) {
      kmin = key[k] < kmin ? key[k] : kmin;
      kmax = key[k] > kmax ? key[k] : kmax;
    }
  }
  kmin = wave_reduce(kmin, [](unsigned long long a, unsigned long long b) { return a < b ? a : b; });
  kmax = wave_reduce(kmax, [](unsigned long long a, unsigned long long b) { return a > b ? a : b; });
  int shift = kmin == kmax ? 0 : 64 - __clzll((long long)(kmin ^ kmax));
  uint64_t prefix = kmax >> shift, A = 0;
  uint32_t C = 0;
  bool resolved = false;
  uint32_t last_cnt = (uint32_t)nb;
  while (!keep_all && shift > 0) {
    const int w = shift < 8 ? shift : 8;   // digit width
    shift -= w;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      hcnt[4 * lane + q] = 0u;
      hmass[4 * lane + q] = 0ull;
    }
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      if (lane + 64 * k < nb && (key[k] >> (shift + w)) == prefix) {
        const uint32_t b = (uint32_t)(key[k] >> shift) & ((1u << w) - 1u);
        atomicAdd(&hcnt[b], 1u);
        atomicAdd(&hmass[b], (unsigned long long)to_fixed(__longlong_as_double((long long)key[k])));
      }
    }
    wave_lds_sync();
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
    uint64_t pm = wave_inclusive_sum(lm);
    uint32_t pc = wave_inclusive_sum(lc);
    pm -= lm;  // exclusive over lanes
    pc -= lc;
    int first = -1;
#pragma unroll
    for (int q = 3; q >= 0; --q) {
      const bool cross = mode == 1 ? (C + pc + ic[q] >= (uint32_t)K) : (A + pm + im[q] >= P);
      if (cross) first = q;
    }
    const unsigned long long bal = __ballot(first >= 0);
    if (bal == 0ull) {  // total mass below p (rounding): every block is kept
      keep_all = true;
      break;
    }
    const int src = __ffsll((long long)bal) - 1;
    const int fq = first < 0 ? 0 : first;
    const int32_t my_bin = 255 - (4 * lane + fq);
    const uint32_t my_cnt = cs[fq];
    const uint32_t my_above_cnt = C + pc + ic[fq] - cs[fq];
    const uint64_t my_above_mass = A + pm + im[fq] - ms[fq];
    const int32_t bin = lane_value(my_bin, src);
    const uint32_t bin_cnt = lane_value(my_cnt, src);
    C = lane_value(my_above_cnt, src);
    A = lane_value(my_above_mass, src);
    prefix = (prefix << w) | (uint64_t)bin;
    last_cnt = bin_cnt;
    wave_lds_sync();   // the next pass clears the bins read above
    if (bin_cnt == 1u) {
      resolved = true;
      break;
    }
  }

  // 4. kept flags.  A ballot over step k holds columns 64 k .. 64 k + 63,
  // i.e. bitmap words 2 k (lanes 0-31) and 2 k + 1 (lanes 32-63), so the
  // words are written whole (2 PER <= kWMaxWords; words past the row's last
  // hold zeros), with no atomics on shared words.
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
    const bool valid = lane + 64 * k < nb;
    const uint64_t hi = key[k] >> shift;
    const bool kept = valid && (keep_all || hi > prefix || (hi == prefix && resolved));
    const bool at_tau = valid && !keep_all && hi == prefix && !resolved;
    const uint64_t kb = __ballot(kept), tb = __ballot(at_tau);
    if (lane == 0) {
      flag[2 * k] = (uint32_t)kb;
      flag[2 * k + 1] = (uint32_t)(kb >> 32);
      tie[2 * k] = (uint32_t)tb;
      tie[2 * k + 1] = (uint32_t)(tb >> 32);
    }
  }
  wave_lds_sync();
  // diagonal band |i - j| <= band - 1
  for (int32_t d = lane - (band - 1); d <= band - 1; d += 64) {
    const int32_t j = i + d;
    if (j >= 0 && j < nb) atomicOr(&flag[j >> 5], 1u << (j & 31));
  }
  wave_lds_sync();
  if (k_tie > 0 && lane == 0) {
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
  wave_lds_sync();

  // 5. bitmap out + count
  int32_t c = 0;
  if (lane < words) {
    const uint32_t f = flag[lane];
    bits[r * words + lane] = f;
    c = __popc(f);
  }
  c = wave_reduce(c, [](int32_t a, int32_t b) { return a + b; });
  if (lane == 0) counts[r] = c;
}

// ---------------------------------------------------------------------------
// row_ptr = exclusive scan of counts (one workgroup; rows fit comfortably)
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 1024;

__global__ void __launch_bounds__(kScanThreads)
scan_kernel(const int32_t* __restrict__ counts, int32_t* __restrict__ row_ptr, int64_t rows) {
  // 16 counts per thread per round: a round costs about one global load
  // latency and a few barriers, so fewer, larger rounds (3 at 47,280 rows).
  // Counts come in and offsets go out with consecutive threads on consecutive
  // rows (whole-line accesses), through an LDS buffer in which thread t's 16
  // consecutive rows are a contiguous run; runs are 17 words apart, so the
  // run reads and writes of a wavefront hit distinct banks.
  constexpr int kPer = 16;
  constexpr int kChunk = kScanThreads * kPer;
  __shared__ int32_t buf[kScanThreads * (kPer + 1)];
  __shared__ int32_t wsum[kScanThreads / 64];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  auto at = [](int e) { return (e / kPer) * (kPer + 1) + e % kPer; };   // row e of the chunk
  int32_t carry = 0;
  for (int64_t base = 0; base < rows; base += kChunk) {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = q * kScanThreads + t;
      buf[at(e)] = base + e < rows ? counts[base + e] : 0;
    }
    __syncthreads();
    int32_t v[kPer];
    int32_t local = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      v[q] = buf[t * (kPer + 1) + q];
      local += v[q];
    }
    const int32_t inc = wave_inclusive_sum(local);
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
      buf[t * (kPer + 1) + q] = run;
      run += v[q];
    }
    carry += total;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = q * kScanThreads + t;
      if (base + e < rows) row_ptr[base + e] = buf[at(e)];
    }
    __syncthreads();   // buf and wsum are rewritten by the next round
  }
  if (t == 0) row_ptr[rows] = carry;
}

// ---------------------------------------------------------------------------
// bitmap -> ascending column indices, one wavefront per row.  Per chunk of 64
// bitmap words (2048 columns) each lane writes the columns of its word into
// the wavefront's LDS buffer at their place in the row (a scan of the word
// counts gives it), then the wavefront copies the chunk's indices to col_idx
// with consecutive lanes on consecutive entries (whole-line stores).
// ---------------------------------------------------------------------------
constexpr int kCThreads = 256;
constexpr int kCChunk = 64 * 32;   // columns per chunk: 64 words of 32

__global__ void __launch_bounds__(kCThreads)
compact_kernel(const uint32_t* __restrict__ bits, const int32_t* __restrict__ row_ptr,
               int32_t* __restrict__ col_idx, int64_t rows, int32_t words) {
  __shared__ int32_t stage_s[kCThreads / 64][kCChunk];
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * (kCThreads / 64) + (threadIdx.x >> 6);
  if (r >= rows) return;   // whole wavefront
  int32_t* st = stage_s[threadIdx.x >> 6];
  int32_t out = row_ptr[r];
  const uint32_t* br = bits + r * words;
  for (int32_t w0 = 0; w0 < words; w0 += 64) {
    const int32_t w = w0 + lane;
    uint32_t f = w < words ? br[w] : 0u;
    const int32_t c = __popc(f);
    const int32_t inc = wave_inclusive_sum(c);
    int32_t pos = inc - c;
    while (f) {
      const int b = __ffs(f) - 1;
      st[pos++] = w * 32 + b;
      f &= f - 1;
    }
    const int32_t tot = lane_value(inc, 63);
    wave_lds_sync();
    for (int32_t k = lane; k < tot; k += 64) col_idx[out + k] = st[k];
    out += tot;
    wave_lds_sync();   // the next chunk rewrites the buffer
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

namespace {
// Logits and selection for the (b, h) pairs b0 .. b0 + cb - 1 (rows b0 * nq ..):
// the logits go to L (cb * nq * nb doubles), the kept bitmaps and counts to
// the global rows of bits / counts.
hipError_t mask_rows(const double* qbar, const double* kbar, const int32_t* ksizes, int64_t b0,
                     int64_t cb, int32_t heads, int32_t nq, int32_t nb, int32_t head_dim,
                     double scale, const HeadParams& hp, int mode, int32_t band, int32_t words,
                     double* L, uint32_t* bits, int32_t* counts, hipStream_t stream) {
  const int32_t tiles_q = (nq + kTile - 1) / kTile, tiles_k = (nb + kTile - 1) / kTile;
  const int64_t lblocks = cb * tiles_q * tiles_k;
  const int64_t rows = cb * nq;
  if (lblocks > 0x7fffffff || rows > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(logits_kernel, dim3((uint32_t)lblocks), dim3(kLThreads), 0, stream,
                     qbar + b0 * nq * head_dim, kbar + b0 * nb * head_dim,
                     ksizes ? ksizes + b0 * nb : nullptr, L, nq, nb, head_dim, scale, tiles_q,
                     tiles_k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t row0 = b0 * nq;
  if (nb <= 64 * 32) {
    const dim3 wgrid((uint32_t)((rows + kWRows - 1) / kWRows)), wblk(64 * kWRows);
    const int per = (nb + 63) / 64;
#define SVSA_SELECT_WAVE(PER_)                                                                  \
  hipLaunchKernelGGL(select_wave_kernel<PER_>, wgrid, wblk, 0, stream, L, bits, counts, nq, nb, \
                     heads, words, band, mode, hp, row0, rows)
    if (per <= 4) SVSA_SELECT_WAVE(4);
    else if (per <= 8) SVSA_SELECT_WAVE(8);
    else if (per <= 12) SVSA_SELECT_WAVE(12);
    else if (per <= 16) SVSA_SELECT_WAVE(16);
    else if (per <= 20) SVSA_SELECT_WAVE(20);
    else if (per <= 24) SVSA_SELECT_WAVE(24);
    else if (per <= 28) SVSA_SELECT_WAVE(28);
    else SVSA_SELECT_WAVE(32);
#undef SVSA_SELECT_WAVE
    return hipGetLastError();
  }
  const dim3 grid((uint32_t)rows), blk(kSThreads);
  if (nb <= kSThreads)
    hipLaunchKernelGGL(select_kernel<1>, grid, blk, 0, stream, L, bits, counts, nq, nb, heads,
                       words, band, mode, hp, row0);
  else if (nb <= 2 * kSThreads)
    hipLaunchKernelGGL(select_kernel<2>, grid, blk, 0, stream, L, bits, counts, nq, nb, heads,
                       words, band, mode, hp, row0);
  else if (nb <= 4 * kSThreads)
    hipLaunchKernelGGL(select_kernel<4>, grid, blk, 0, stream, L, bits, counts, nq, nb, heads,
                       words, band, mode, hp, row0);
  else if (nb <= 8 * kSThreads)
    hipLaunchKernelGGL(select_kernel<8>, grid, blk, 0, stream, L, bits, counts, nq, nb, heads,
                       words, band, mode, hp, row0);
  else
    hipLaunchKernelGGL(select_kernel<16>, grid, blk, 0, stream, L, bits, counts, nq, nb, heads,
                       words, band, mode, hp, row0);
  return hipGetLastError();
}

HeadParams head_params(int32_t heads, const float* top_p, const float* keep_frac) {
  HeadParams hp{};
  const float* src = top_p ? top_p : keep_frac;
  for (int32_t h = 0; h < heads; ++h) hp.v[h] = src[h];
  return hp;
}
}  // namespace

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
  const HeadParams hp = head_params(heads, top_p, keep_frac);
  hipError_t e = mask_rows(qbar, kbar, ksizes, 0, bh, heads, nq, nb, head_dim, scale, hp,
                           top_p ? 0 : 1, band, m.words, L, bits, counts, stream);
  if (e != hipSuccess) return e;
  return launch_csr_from_bits(bits, counts, row_ptr, col_idx, rows, m.words, stream);
}

// ---------------------------------------------------------------------------
// The block mask without a caller workspace: its scratch is a file-scope device
// array of kScratchBytes (held on each device the library runs on until the
// process ends).  The logits of a chunk of whole (b, h) pairs go to its first
// kScratchLogits bytes, one chunk after the other; the kept bitmaps and row
// counts of every row to the rest.  Each device's copy of the array has its
// own address, looked up once per device.
// ---------------------------------------------------------------------------
constexpr size_t kScratchLogits = (size_t)64 << 20;
constexpr size_t kScratchBits = (size_t)16 << 20;
constexpr size_t kScratchBytes = kScratchLogits + kScratchBits;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void* scratch_ptr[kMaxDevices];
hipError_t scratch_err[kMaxDevices];

// This device's address of `scratch` (nullptr and an error on failure).
hipError_t device_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(scratch_once[dev], [dev] {
    void* p = nullptr;
    scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    scratch_ptr[dev] = scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *out = scratch_ptr[dev];
  return scratch_err[dev];
}
}  // namespace

bool block_mask_fits_scratch(int64_t bh, int32_t nb) {
  const int64_t words = (nb + 31) / 32;
  const uint64_t per_head = (uint64_t)nb * nb * sizeof(double);
  const uint64_t rows = (uint64_t)bh * nb;
  return per_head <= kScratchLogits &&
         align_up(rows * words * sizeof(uint32_t), 256) + rows * sizeof(int32_t) <= kScratchBits;
}

hipError_t launch_block_mask_noalloc(const double* qbar, const double* kbar, int32_t bh,
                                     int32_t heads, int32_t nb, int32_t head_dim, double scale,
                                     const float* top_p, const float* keep_frac, int32_t band,
                                     int32_t* row_ptr, int32_t* col_idx, hipStream_t stream) {
  if (heads > kMaxHeads || nb > kMaxNb || !block_mask_fits_scratch(bh, nb))
    return hipErrorInvalidValue;
  void* base = nullptr;
  hipError_t e = device_scratch(&base);
  if (e != hipSuccess) return e;
  char* w = static_cast<char*>(base);
  double* L = reinterpret_cast<double*>(w);
  const int64_t rows = (int64_t)bh * nb;
  const int32_t words = (nb + 31) / 32;
  uint32_t* bits = reinterpret_cast<uint32_t*>(w + kScratchLogits);
  int32_t* counts = reinterpret_cast<int32_t*>(
      w + kScratchLogits + align_up((size_t)rows * words * sizeof(uint32_t), 256));
  const HeadParams hp = head_params(heads, top_p, keep_frac);
  const int64_t chunk = (int64_t)(kScratchLogits / ((size_t)nb * nb * sizeof(double)));
  for (int64_t b0 = 0; b0 < bh; b0 += chunk) {
    const int64_t cb = bh - b0 < chunk ? bh - b0 : chunk;
    e = mask_rows(qbar, kbar, nullptr, b0, cb, heads, nb, nb, head_dim, scale, hp,
                  top_p ? 0 : 1, band, words, L, bits, counts, stream);
    if (e != hipSuccess) return e;
  }
  return launch_csr_from_bits(bits, counts, row_ptr, col_idx, rows, words, stream);
}

}  // namespace svsa
