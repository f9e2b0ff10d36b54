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
//  * A workgroup is 8 wavefronts (32 query rows each) and owns 256 consecutive
//    query rows of one (b, h): 4 blocks of 64 tokens, or 8 blocks of 32.
//    Neighbouring query blocks keep largely the same key blocks, so the
//    workgroup streams the UNION of their lists through LDS once and every
//    wavefront whose block keeps the current key block computes on it (up to
//    8x LDS / L2 reuse of K and V).
//  * The schedule kernel merges the group's CSR rows into that union list,
//    with a "who keeps it" bit mask per entry, and orders the work items
//    longest first.
//  * K and V tiles are double-buffered in LDS: the next key block's global
//    loads are issued into registers before the current block is computed and
//    written to the other buffer after it.  Both tiles are row-major with a
//    16-byte XOR swizzle chosen for their read pattern.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane then owns one query column, so the
//    row max / row sum are lane-local plus one exchange between the two
//    32-lane halves.  The float32 probabilities convert in registers into the
//    bf16 B operand of O^T += V^T P^T; the V^T A operand comes straight from
//    the row-major V tile through ds_read_b64_tr_b16 (LDS transpose reads).
//    The key order inside each 16-key MFMA step is permuted identically on
//    both operands.
//  * Online softmax in base 2 with lazy rescaling: the running max only moves
//    (and O, l are only rescaled) when a tile raises it by more than 2^8, so
//    probabilities stay <= 256 and the O rescale is skipped on most tiles.
#include "svsa_internal.h"

namespace svsa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerItem = 32 * kWaves;  // query rows owned by one workgroup
constexpr float kLazy = 8.0f;              // log2 of the largest unnormalised probability

// ---------------------------------------------------------------------------
// Schedule: per item (b, h, group of query blocks) the ascending union of the
// group's kept key blocks; entry = j | (mask << 24), bit m of mask set when the
// m-th query block of the group keeps j.
// ---------------------------------------------------------------------------
constexpr int kSchedThreads = 256;

__global__ void __launch_bounds__(kSchedThreads)
union_kernel(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
             int32_t* __restrict__ list, int32_t* __restrict__ count, int32_t nb, int32_t groups,
             int32_t group_size) {
  extern __shared__ uint32_t mask[];  // [nb]
  __shared__ int32_t wave_tot[kSchedThreads / 64];
  const int64_t item = blockIdx.x;
  const int64_t bh = item / groups;
  const int32_t g = (int32_t)(item % groups);
  const int t = threadIdx.x;
  for (int32_t j = t; j < nb; j += kSchedThreads) mask[j] = 0u;
  __syncthreads();
  for (int m = 0; m < group_size; ++m) {
    const int32_t i = g * group_size + m;
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

// order[] = items sorted by union length, longest first (counting sort; the
// order among equal lengths is arbitrary and does not affect any result).
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
  // start[c] = number of items longer than c (bins scanned in descending order)
  int32_t carry = 0;
  for (int32_t base = 0; base <= nb; base += kOrderThreads) {
    const int32_t c = nb - (base + t);
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
template <int D, int BK>
struct Cfg {
  static constexpr int kTileBytes = BK * D * 2;          // one K (or V) tile
  static constexpr int kStageBytes = 2 * kTileBytes;     // K + V
  static constexpr int kLdsBytes = 2 * kStageBytes;      // double buffer
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kSTiles = BK / 32;   // 32-key tiles of S^T
  static constexpr int kPSteps = BK / 16;   // 16-key MFMA steps of P V
  static constexpr int kWavesPerBlock = BK / 32;
  static constexpr int kGroup = kWaves / kWavesPerBlock;  // query blocks per item
};

// K tile: read as the A operand of S^T (32 consecutive rows, one 16-byte
// chunk each): the chunk index is XORed with the row so 16 rows hit 16
// different bank groups.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
// V tile: read by ds_read_b64_tr_b16; a half-wavefront touches 4 rows x 4
// chunks, spread over all banks by XORing bits 2..3 of the chunk index.
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

// Staging of one key block (K tile then V tile) through registers: every
// thread loads kPer 16-byte chunks (coalesced along rows) early in an
// iteration and writes them, swizzled, into the other LDS buffer at its end.
template <int D, int BK>
struct Stage {
  static constexpr int kChunksPerTile = BK * D / 8;
  static constexpr int kPer = 2 * kChunksPerTile / kThreads;
  static_assert((2 * kChunksPerTile) % kThreads == 0, "tile chunks must split over the threads");
  u32x4 r[kPer];

  __device__ __forceinline__ void load(const __bf16* kh, const __bf16* vh, int32_t j, int tid) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c = tid + u * kThreads;
      const bool is_v = c >= kChunksPerTile;
      const int cc = is_v ? c - kChunksPerTile : c;
      const int row = cc / (D / 8), lc = cc % (D / 8);
      r[u] = *reinterpret_cast<const u32x4*>((is_v ? vh : kh) + ((int64_t)j * BK + row) * D +
                                             lc * 8);
    }
  }
  __device__ __forceinline__ void store(char* stage, int tid) const {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c = tid + u * kThreads;
      const bool is_v = c >= kChunksPerTile;
      const int cc = is_v ? c - kChunksPerTile : c;
      const int row = cc / (D / 8), lc = cc % (D / 8);
      const int pc = lc ^ (is_v ? v_swz<D>(row) : k_swz<D>(row));
      *reinterpret_cast<u32x4*>(stage + (is_v ? Cfg<D, BK>::kTileBytes : 0) +
                                row * Cfg<D, BK>::kRowBytes + (pc << 4)) = r[u];
    }
  }
};

template <int D, int BK>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
            const __bf16* __restrict__ v, __bf16* __restrict__ out,
            const int32_t* __restrict__ list, const int32_t* __restrict__ count,
            const int32_t* __restrict__ order, int32_t groups, int32_t nb, int32_t Npad,
            int32_t last_valid, float c_log2) {
  using C = Cfg<D, BK>;
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  constexpr int kS = D / 16;    // MFMA K-steps over the head dimension
  constexpr int kDT = D / 32;   // 32-row tiles of O^T

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int qb = wave / C::kWavesPerBlock;                 // query block inside the group
  const int sub = wave % C::kWavesPerBlock;                // 32-row slice inside the block
  const int l32 = lane & 31, hh = lane >> 5;

  const int64_t item = order[blockIdx.x];
  const int64_t bh = item / groups;
  const int32_t g = (int32_t)(item % groups);
  const int32_t iq = g * C::kGroup + qb;
  const bool wave_has_rows = iq < nb;
  const int32_t n_u = count[item];
  const int32_t* lst = list + item * nb;

  const __bf16* qh = q + bh * (int64_t)Npad * D;
  const __bf16* kh = k + bh * (int64_t)Npad * D;
  const __bf16* vh = v + bh * (int64_t)Npad * D;
  __bf16* oh = out + bh * (int64_t)Npad * D;

  Stage<D, BK> stg;
  if (n_u > 0) stg.load(kh, vh, lst[0] & 0xffffff, tid);

  const int32_t qrow = (wave_has_rows ? iq : nb - 1) * BK + sub * 32 + l32;
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

  if (n_u > 0) stg.store(lds, tid);
  __syncthreads();

  for (int32_t e = 0; e < n_u; ++e) {
    const int32_t ent = lst[e];
    const int32_t j = ent & 0xffffff;
    const uint32_t who = (uint32_t)ent >> 24;
    // prefetch the next key block (the last iteration reloads its own block
    // into the idle buffer, which keeps the loop free of divergent branches)
    stg.load(kh, vh, lst[min(e + 1, n_u - 1)] & 0xffffff, tid);

    const char* ks = lds + (e & 1) * C::kStageBytes;
    const char* vs = ks + C::kTileBytes;
    if (wave_has_rows && ((who >> qb) & 1u)) {
      // S^T[kv][q] = sum_d K[kv][d] Q[q][d]
      f32x16 sacc[C::kSTiles];
#pragma unroll
      for (int c = 0; c < C::kSTiles; ++c) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[c][r] = 0.f;
        const int row = 32 * c + l32;
        bf16x8 kf[kS];
#pragma unroll
        for (int s = 0; s < kS; ++s) {
          const int cc = 2 * s + hh;
          kf[s] = *reinterpret_cast<const bf16x8*>(ks + row * C::kRowBytes +
                                                   ((cc ^ k_swz<D>(row)) << 4));
        }
#pragma unroll
        for (int s = 0; s < kS; ++s)
          sacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qreg[s], sacc[c], 0, 0, 0);
      }
      // lane holds keys kv = 32 c + 8 (r / 4) + 4 hh + (r % 4) of query column l32
      if (j == nb - 1 && last_valid < BK) {
#pragma unroll
        for (int c = 0; c < C::kSTiles; ++c)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kv = 32 * c + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (kv >= last_valid) sacc[c][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int c = 0; c < C::kSTiles; ++c)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sacc[c][r], sacc[c][r + 1]));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mxs = mx * c_log2;
      // lazy rescale: move the running max only when it grows by > kLazy
      const bool need = mxs > m_run + kLazy;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float m_new = need ? mxs : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      }
      float rs = 0.f;
#pragma unroll
      for (int c = 0; c < C::kSTiles; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[c][r], c_log2, -m_run));
          sacc[c][r] = p;
          rs += p;
        }
      l_run += rs;
      // P^T as the bf16 B operand of step s: keys 16 s + 4 hh + {0..3, 8..11}
      bf16x8 pk[C::kPSteps];
#pragma unroll
      for (int s = 0; s < C::kPSteps; ++s)
#pragma unroll
        for (int x = 0; x < 8; ++x) pk[s][x] = (__bf16)sacc[s >> 1][8 * (s & 1) + x];
      // O^T[d][q] += sum_kv V^T[d][kv] P^T[kv][q]; the A operand of step s for
      // lane (d = 32 dt + l32, hh) is keys 16 s + 4 hh + {0..3} and {8..11},
      // two transposed 4x16 reads of the row-major V tile
      const int grp = lane >> 4, jj = lane & 15;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        const int dcol = 32 * dt + 16 * (grp & 1) + 4 * (jj & 3);
#pragma unroll
        for (int s = 0; s < C::kPSteps; ++s) {
          bf16x8 a;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int row = 16 * s + 8 * half + 4 * hh + (jj >> 2);
            const int lc = dcol >> 3;
            const int off = row * C::kRowBytes + ((lc ^ v_swz<D>(row)) << 4) + 2 * (dcol & 7);
            const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vs + off));
            const bf16x4 tb = __builtin_bit_cast(bf16x4, t);
#pragma unroll
            for (int x = 0; x < 4; ++x) a[4 * half + x] = tb[x];
          }
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[s], oacc[dt], 0, 0, 0);
        }
      }
    }
    stg.store(lds + ((e + 1) & 1) * C::kStageBytes, tid);
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
      bf16x4 o;
#pragma unroll
      for (int x = 0; x < 4; ++x) o[x] = (__bf16)(oacc[dt][4 * rq + x] * inv);
      *reinterpret_cast<bf16x4*>(orow + d0) = o;
    }
}

template <int D, int BK>
hipError_t launch_attn(const void* q, const void* k, const void* v, void* out, const int32_t* list,
                       const int32_t* count, const int32_t* order, const AttnWs& w, const Geom& g,
                       float c_log2, hipStream_t stream) {
  using C = Cfg<D, BK>;
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_kernel<D, BK>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::kLdsBytes);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int32_t last_valid = g.N - (g.nb - 1) * BK;
  hipLaunchKernelGGL((attn_kernel<D, BK>), dim3((uint32_t)w.items), dim3(kThreads), C::kLdsBytes,
                     stream, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)out,
                     list, count, order, w.groups, g.nb, g.Npad, last_valid, c_log2);
  return hipGetLastError();
}

}  // namespace

AttnWs attn_ws_layout(int32_t bh, int32_t nb, int32_t Bk) {
  AttnWs w{};
  w.group_size = kRowsPerItem / Bk;
  w.groups = (nb + w.group_size - 1) / w.group_size;
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
  if (g.Bk != 32 && g.Bk != 64) return hipErrorInvalidValue;
  if (head_dim != 64 && head_dim != 128) return hipErrorInvalidValue;
  const AttnWs w = attn_ws_layout(bh, g.nb, g.Bk);
  if (w.items > 0x7fffffff) return hipErrorInvalidValue;
  char* base = static_cast<char*>(ws);
  int32_t* list = reinterpret_cast<int32_t*>(base + w.list_off);
  int32_t* count = reinterpret_cast<int32_t*>(base + w.count_off);
  int32_t* order = reinterpret_cast<int32_t*>(base + w.order_off);

  hipLaunchKernelGGL(union_kernel, dim3((uint32_t)w.items), dim3(kSchedThreads),
                     (size_t)g.nb * sizeof(uint32_t), stream, row_ptr, col_idx, list, count, g.nb,
                     w.groups, w.group_size);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(order_kernel, dim3(1), dim3(kOrderThreads),
                     (size_t)(g.nb + 1) * sizeof(int32_t), stream, count, order, w.items, g.nb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const float c_log2 = scale * 1.4426950408889634f;
  if (head_dim == 128 && g.Bk == 64)
    return launch_attn<128, 64>(q, k, v, out, list, count, order, w, g, c_log2, stream);
  if (head_dim == 64 && g.Bk == 64)
    return launch_attn<64, 64>(q, k, v, out, list, count, order, w, g, c_log2, stream);
  if (head_dim == 128 && g.Bk == 32)
    return launch_attn<128, 32>(q, k, v, out, list, count, order, w, g, c_log2, stream);
  return launch_attn<64, 32>(q, k, v, out, list, count, order, w, g, c_log2, stream);
}

}  // namespace svsa
