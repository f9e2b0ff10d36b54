// Stage 4: block-sparse flash attention over the kept blocks (gfx950).
//
// [PSA] "Parameterized Stripe Attention for Efficient Video Generation",
// App. B, Alg. 2: per query block, walk the list of needed KV blocks; for each,
// S = Q K^T, invalid (padded) positions set to -inf, safe softmax, P V
// accumulated into the block's output, which is written once at the end.
// [SPADE] "SPADE: An Input-Adaptive Sparse Attention Engine for Fast Video
// Diffusion Models Inference", abstract: flash block-sparse attention plus
// kernel grouping.
//
// Design for CDNA4 (not a port of the Hopper producer/consumer pipeline):
//  * A workgroup owns kGroup = 4 consecutive query blocks of one (b, h): 8
//    wavefronts, two per query block, 32 query rows per wavefront.  Adjacent
//    query blocks keep largely the same key blocks, so the workgroup streams
//    the UNION of their lists once through LDS and every wavefront whose block
//    keeps the current key block computes on it (4x LDS/L2 reuse of K and V).
//  * The schedule kernel merges the four CSR rows into that union list, with
//    a 4-bit "who keeps it" mask per entry, and orders work heaviest first.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane then owns one query column and the
//    row softmax (max / sum) is lane-local plus one exchange between the two
//    32-lane halves.  The float32 probabilities convert in registers into the
//    bf16 B operand of O^T += V^T P^T (the key order inside an MFMA K-step is
//    permuted consistently between P^T and the LDS image of V^T).
//  * K is staged row-major with a 16-byte XOR swizzle; V is transposed while
//    it is staged (4x4 register transposes) so the V^T operand is one 16-byte
//    LDS read per lane.  Two LDS buffers: the next key block's global loads
//    are in flight while the current one is computed.
//  * Online softmax in base 2 (scale * log2 e folded into one FMA), float32
//    state, final 1/l applied before the bf16 store.
#include "svsa_internal.h"

namespace svsa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kBk = 64;                 // tokens per block (4x4x4 tiles)
constexpr int kGroup = kQBlocksPerGroup;
constexpr int kWaves = 2 * kGroup;
constexpr int kThreads = 64 * kWaves;

// ---------------------------------------------------------------------------
// Schedule: per item (b, h, group of kGroup query blocks) the ascending union
// of the group's kept key blocks; entry = j | (mask << 24).
// ---------------------------------------------------------------------------
constexpr int kSchedThreads = 256;

__global__ void __launch_bounds__(kSchedThreads)
union_kernel(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
             int32_t* __restrict__ list, int32_t* __restrict__ count, int32_t nb, int32_t groups) {
  extern __shared__ uint32_t mask[];  // [nb]
  __shared__ int32_t wave_tot[kSchedThreads / 64];
  const int64_t item = blockIdx.x;
  const int64_t bh = item / groups;
  const int32_t g = (int32_t)(item % groups);
  const int t = threadIdx.x;
  for (int32_t j = t; j < nb; j += kSchedThreads) mask[j] = 0u;
  __syncthreads();
  for (int m = 0; m < kGroup; ++m) {
    const int32_t i = g * kGroup + m;
    if (i >= nb) break;
    const int64_t row = bh * nb + i;
    const int32_t e0 = row_ptr[row], e1 = row_ptr[row + 1];
    for (int32_t e = e0 + t; e < e1; e += kSchedThreads) {
      const int32_t j = col_idx[e];
      if (j >= 0 && j < nb) atomicOr(&mask[j], 1u << m);
    }
  }
  __syncthreads();
  int32_t* out = list + item * nb;
  int32_t off = 0;
  const int lane = t & 63, wv = t >> 6;
  for (int32_t base = 0; base < nb; base += kSchedThreads) {
    const int32_t j = base + t;
    const uint32_t m = j < nb ? mask[j] : 0u;
    const unsigned long long bal = __ballot(m != 0u);
    const int32_t before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wv] = __popcll(bal);
    __syncthreads();
    int32_t wbase = 0, tot = 0;
    for (int k = 0; k < kSchedThreads / 64; ++k) {
      if (k < wv) wbase += wave_tot[k];
      tot += wave_tot[k];
    }
    if (m != 0u) out[off + wbase + before] = j | (int32_t)(m << 24);
    off += tot;
    __syncthreads();
  }
  if (t == 0) count[item] = off;
}

// order[] = items sorted by union length, longest first (counting sort).
constexpr int kOrderThreads = 1024;

__global__ void __launch_bounds__(kOrderThreads)
order_kernel(const int32_t* __restrict__ count, int32_t* __restrict__ order, int64_t items,
             int32_t nb) {
  extern __shared__ int32_t hist[];  // [nb + 1]
  __shared__ int32_t buf[kOrderThreads];
  const int t = threadIdx.x;
  for (int32_t c = t; c <= nb; c += kOrderThreads) hist[c] = 0;
  __syncthreads();
  for (int64_t it = t; it < items; it += kOrderThreads) atomicAdd(&hist[min(count[it], nb)], 1);
  __syncthreads();
  // exclusive scan over bins in descending count order: start[c] = sum_{c' > c} hist[c']
  int32_t carry = 0;
  for (int32_t base = 0; base <= nb; base += kOrderThreads) {
    const int32_t c = nb - (base + t);  // descending bins
    const int32_t v = c >= 0 ? hist[c] : 0;
    buf[t] = v;
    __syncthreads();
    for (int s = 1; s < kOrderThreads; s <<= 1) {
      const int32_t add = t >= s ? buf[t - s] : 0;
      __syncthreads();
      buf[t] += add;
      __syncthreads();
    }
    const int32_t excl = carry + buf[t] - v;
    const int32_t chunk = buf[kOrderThreads - 1];
    __syncthreads();
    if (c >= 0) hist[c] = excl;
    carry += chunk;
    __syncthreads();
  }
  for (int64_t it = t; it < items; it += kOrderThreads) {
    const int32_t pos = atomicAdd(&hist[min(count[it], nb)], 1);
    order[pos] = (int32_t)it;
  }
}

// ---------------------------------------------------------------------------
// Attention kernel.
// ---------------------------------------------------------------------------
template <int D>
struct Lds {
  // K tile: [64 rows][D] bf16, 16-byte chunks XOR-swizzled per row.
  // V^T tile: [D rows][64 keys] bf16, keys permuted inside each 16-key step
  // and 16-byte chunks XOR-swizzled per row.
  static constexpr int kKBytes = kBk * D * 2;
  static constexpr int kVBytes = D * kBk * 2;
  static constexpr int kBufBytes = kKBytes + kVBytes;
  static constexpr int kBytes = 2 * kBufBytes;
};

template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
__device__ __forceinline__ int v_swz(int d) { return (d >> 1) & 7; }

template <int D>
struct TileRegs {
  static constexpr int kKChunks = kBk * D / 8;             // 16-byte chunks of K
  static constexpr int kKPer = (kKChunks + kThreads - 1) / kThreads;
  static constexpr int kVUnits = kBk * D / 16;             // 4 keys x 4 dims units of V
  uint4 k[kKPer];
  uint2 v[4];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const __bf16* kh, const __bf16* vh,
                                          int32_t j, int tid) {
  const uint4* kt = reinterpret_cast<const uint4*>(kh + (int64_t)j * kBk * D);
#pragma unroll
  for (int u = 0; u < TileRegs<D>::kKPer; ++u) {
    const int c = tid + u * kThreads;
    if (c < TileRegs<D>::kKChunks) r.k[u] = kt[c];
  }
  if (tid < TileRegs<D>::kVUnits) {
    const int dgrp = tid % (D / 4), kvq = tid / (D / 4);
    const __bf16* vt = vh + ((int64_t)j * kBk + 4 * kvq) * D + 4 * dgrp;
#pragma unroll
    for (int q = 0; q < 4; ++q) r.v[q] = *reinterpret_cast<const uint2*>(vt + q * D);
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& r, char* buf, int tid) {
  char* ks = buf;
  char* vs = buf + Lds<D>::kKBytes;
  constexpr int kChunksPerRow = D / 8;
#pragma unroll
  for (int u = 0; u < TileRegs<D>::kKPer; ++u) {
    const int c = tid + u * kThreads;
    if (c < TileRegs<D>::kKChunks) {
      const int row = c / kChunksPerRow, cc = c % kChunksPerRow;
      *reinterpret_cast<uint4*>(ks + row * (2 * D) + ((cc ^ k_swz<D>(row)) << 4)) = r.k[u];
    }
  }
  if (tid < TileRegs<D>::kVUnits) {
    const int dgrp = tid % (D / 4), kvq = tid / (D / 4);
    const int kv0 = 4 * kvq;
    // key kv = 16 s + 8 a + 4 h + e is stored at position 16 s + 8 h + 4 a + e
    const int s = kv0 >> 4, a = (kv0 >> 3) & 1, hh = (kv0 >> 2) & 1;
    const int chunk = 2 * s + hh, byte_in = 8 * a;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d = 4 * dgrp + e;
      const int sh = (e & 1) * 16;
      uint32_t x0 = ((e < 2 ? r.v[0].x : r.v[0].y) >> sh) & 0xffffu;
      uint32_t x1 = ((e < 2 ? r.v[1].x : r.v[1].y) >> sh) & 0xffffu;
      uint32_t x2 = ((e < 2 ? r.v[2].x : r.v[2].y) >> sh) & 0xffffu;
      uint32_t x3 = ((e < 2 ? r.v[3].x : r.v[3].y) >> sh) & 0xffffu;
      uint2 w;
      w.x = x0 | (x1 << 16);
      w.y = x2 | (x3 << 16);
      *reinterpret_cast<uint2*>(vs + d * (2 * kBk) + ((chunk ^ v_swz(d)) << 4) + byte_in) = w;
    }
  }
}

template <int D>
__global__ void __launch_bounds__(kThreads)
attn_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
            const __bf16* __restrict__ v, __bf16* __restrict__ out,
            const int32_t* __restrict__ list, const int32_t* __restrict__ count,
            const int32_t* __restrict__ order, int32_t groups, int32_t nb, int32_t Npad,
            int32_t last_valid, float c_log2) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int kS = D / 16;    // MFMA K-steps over the head dimension
  constexpr int kDT = D / 32;   // 32-row tiles of O^T

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int qb = wave >> 1, half = wave & 1;
  const int l32 = lane & 31, hh = lane >> 5;

  const int64_t item = order[blockIdx.x];
  const int64_t bh = item / groups;
  const int32_t g = (int32_t)(item % groups);
  const int32_t iq = g * kGroup + qb;
  const bool wave_has_rows = iq < nb;
  const int32_t n_u = count[item];
  const int32_t* lst = list + item * nb;

  const __bf16* qh = q + bh * (int64_t)Npad * D;
  const __bf16* kh = k + bh * (int64_t)Npad * D;
  const __bf16* vh = v + bh * (int64_t)Npad * D;
  __bf16* oh = out + bh * (int64_t)Npad * D;

  const int32_t qrow = (wave_has_rows ? iq : nb - 1) * kBk + half * 32 + l32;
  bf16x8 qreg[kS];
#pragma unroll
  for (int s = 0; s < kS; ++s)
    qreg[s] = *reinterpret_cast<const bf16x8*>(qh + (int64_t)qrow * D + 16 * s + 8 * hh);

  f32x16 oacc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  TileRegs<D> regs;
  if (n_u > 0) {
    load_tile<D>(regs, kh, vh, lst[0] & 0xffffff, tid);
    store_tile<D>(regs, lds, tid);
  }
  __syncthreads();

  for (int32_t e = 0; e < n_u; ++e) {
    const int32_t ent = lst[e];
    const int32_t j = ent & 0xffffff;
    const uint32_t who = (uint32_t)ent >> 24;
    const bool more = e + 1 < n_u;
    if (more) load_tile<D>(regs, kh, vh, lst[e + 1] & 0xffffff, tid);

    const char* buf = lds + (e & 1) * Lds<D>::kBufBytes;
    if (wave_has_rows && ((who >> qb) & 1u)) {
      const char* ks = buf;
      const char* vs = buf + Lds<D>::kKBytes;
      // S^T[kv][q] = sum_d K[kv][d] Q[q][d]
      f32x16 sacc[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[c][r] = 0.f;
        const int row = 32 * c + l32;
#pragma unroll
        for (int s = 0; s < kS; ++s) {
          const int cc = 2 * s + hh;
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(ks + row * (2 * D) + ((cc ^ k_swz<D>(row)) << 4));
          sacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], sacc[c], 0, 0, 0);
        }
      }
      // padded keys of the tail block -> -inf
      if (j == nb - 1 && last_valid < kBk) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kv = 32 * c + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (kv >= last_valid) sacc[c][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[c][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx * c_log2);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float rs = 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[c][r], c_log2, -m_new));
          sacc[c][r] = p;
          rs += p;
        }
      l_run = l_run * alpha + rs;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      bf16x8 pk[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int x = 0; x < 8; ++x) pk[s][x] = (__bf16)sacc[s >> 1][8 * (s & 1) + x];
      // O^T[d][q] += sum_kv V^T[d][kv] P^T[kv][q]
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        const int d = 32 * dt + l32;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int chunk = 2 * s + hh;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vs + d * (2 * kBk) +
                                                            ((chunk ^ v_swz(d)) << 4));
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[s], oacc[dt], 0, 0, 0);
        }
      }
    }
    if (more) store_tile<D>(regs, lds + ((e + 1) & 1) * Lds<D>::kBufBytes, tid);
    __syncthreads();
  }

  if (!wave_has_rows) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  __bf16* orow = oh + (int64_t)qrow * D;
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = 32 * dt + 8 * rq + 4 * hh;
      typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
      bf16x4 o;
#pragma unroll
      for (int x = 0; x < 4; ++x) o[x] = (__bf16)(oacc[dt][4 * rq + x] * inv);
      *reinterpret_cast<bf16x4*>(orow + d0) = o;
    }
}

}  // namespace

AttnWs attn_ws_layout(int32_t bh, int32_t nb) {
  AttnWs w{};
  w.groups = (nb + kGroup - 1) / kGroup;
  w.items = (int64_t)bh * w.groups;
  size_t off = 0;
  w.list_off = off;
  off = align_up(off + (size_t)w.items * nb * sizeof(int32_t), 256);
  w.count_off = off;
  off = align_up(off + (size_t)w.items * sizeof(int32_t), 256);
  w.order_off = off;
  off = align_up(off + (size_t)w.items * sizeof(int32_t), 256);
  w.total = off;
  return w;
}

hipError_t launch_block_sparse_attn(const void* q, const void* k, const void* v, void* out,
                                    int32_t bh, int32_t head_dim, const Geom& g, float scale,
                                    const int32_t* row_ptr, const int32_t* col_idx, void* ws,
                                    hipStream_t stream) {
  if (g.Bk != kBk) return hipErrorInvalidValue;
  const AttnWs w = attn_ws_layout(bh, g.nb);
  if (w.items > 0x7fffffff) return hipErrorInvalidValue;
  char* base = static_cast<char*>(ws);
  int32_t* list = reinterpret_cast<int32_t*>(base + w.list_off);
  int32_t* count = reinterpret_cast<int32_t*>(base + w.count_off);
  int32_t* order = reinterpret_cast<int32_t*>(base + w.order_off);

  hipLaunchKernelGGL(union_kernel, dim3((uint32_t)w.items), dim3(kSchedThreads),
                     (size_t)g.nb * sizeof(uint32_t), stream, row_ptr, col_idx, list, count, g.nb,
                     w.groups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(order_kernel, dim3(1), dim3(kOrderThreads),
                     (size_t)(g.nb + 1) * sizeof(int32_t), stream, count, order, w.items, g.nb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const float c_log2 = scale * 1.4426950408889634f;
  const int32_t last_valid = g.N - (g.nb - 1) * kBk;
  if (head_dim == 128) {
    hipLaunchKernelGGL(attn_kernel<128>, dim3((uint32_t)w.items), dim3(kThreads),
                       Lds<128>::kBytes, stream, (const __bf16*)q, (const __bf16*)k,
                       (const __bf16*)v, (__bf16*)out, list, count, order, w.groups, g.nb, g.Npad,
                       last_valid, c_log2);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL(attn_kernel<64>, dim3((uint32_t)w.items), dim3(kThreads),
                       Lds<64>::kBytes, stream, (const __bf16*)q, (const __bf16*)k,
                       (const __bf16*)v, (__bf16*)out, list, count, order, w.groups, g.nb, g.Npad,
                       last_valid, c_log2);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace svsa
