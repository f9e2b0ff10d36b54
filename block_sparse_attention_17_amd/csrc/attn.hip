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
//  * The schedule sees the sequence as sub-blocks of 64 tokens (32 when the
//    block size is an odd multiple of 32, or for 32-aligned clusters); a block
//    of Bk tokens is Bk / 64 consecutive sub-blocks, each with the block's
//    list (so PSA-shaped 3x8x16 = 384-token blocks run unchanged).  Key tiles
//    are always 64 keys: with 32-token sub-blocks the kernel streams two list
//    entries per tile (paired mode), each half copied from its own block.
//  * A workgroup is 8 wavefronts (32 query rows each) and owns 256 consecutive
//    query rows of one (b, h): 4 sub-blocks of 64 tokens, or 8 of 32.
//    Neighbouring query blocks keep largely the same key blocks, so the
//    workgroup streams the UNION of their lists through LDS once and every
//    wavefront whose block keeps the current key block computes on it.
//  * The schedule kernel merges the group's CSR rows into that union list,
//    with a "who keeps it" bit mask per entry.  Items go to one work queue
//    per XCD, a quarter of a (b, h)'s consecutive query groups per queue
//    entry, so that the workgroups of one XCD share the head's key blocks in
//    its L2; a persistent kernel drains its own XCD's queue first, then the
//    others.
//  * V is transposed once per call (vt_kernel), or once per step straight
//    from natural-order V (stage_v_kernel, svsa_attn_stage_v), so both MFMA
//    A operands (K rows for S^T, V^T rows for O^T) are plain 16-byte LDS
//    reads.
//  * Key blocks reach LDS through a 4-slot ring filled by MUBUF buffer loads
//    with the LDS destination (no VGPR staging), issued two blocks ahead and
//    waited for with explicit vmcnt counts.  Tiles are XOR-swizzled by row so
//    that the operand reads are free of bank conflicts.
//  * Ping-pong: waves 0-3 and 4-7 form two groups (one wave of each per SIMD).
//    Each key block is two phases per wave: M (O += P V of the previous block
//    and S^T = K Q^T of this one, on the matrix cores) and V (online softmax
//    on the vector ALU).  Group 1 runs one phase behind group 0 and phases
//    are separated by workgroup barriers, so in every interval one wave per
//    SIMD feeds the matrix cores while the other runs the softmax.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane then owns one query column, so the
//    row max / row sum are lane-local plus one exchange between the two
//    32-lane halves.  The float32 probabilities convert in registers into the
//    bf16 B operand of O^T += V^T P^T; the key order inside each 16-key MFMA
//    step is permuted identically on both operands.
//  * Online softmax in base 2 with lazy rescaling: the running max only moves
//    (and O, l are only rescaled) when a tile raises it by more than 2^8, so
//    probabilities stay <= 256 and the O rescale is skipped on most tiles.
#include <algorithm>

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
constexpr int kMaxHeadDim = 128;
constexpr int kEnt = 7;                    // list entries used by one round of 8 intervals
constexpr int kWin = 10;  // LDS operand reads in flight ahead of the MFMA stream
constexpr int kPre = 4;   // P V operands read before the barrier that opens an M phase

// ---------------------------------------------------------------------------
// Schedule: per item (b, h, group of query sub-blocks) the union of the
// group's kept key sub-blocks, ascending from the group's own diagonal key
// sub-block and wrapping around (fixed-size blocks; cluster lists start at 0); entry = j | (valid << 13) | (mask << 24):
// j the key sub-block (< 8192), valid its valid tokens (its first slots; key
// sub-blocks with none are left out), bit m of mask set when the m-th query
// sub-block of the group keeps j.
// ---------------------------------------------------------------------------
constexpr int kSchedThreads = 256;

// The attention kernels work on sub-blocks of S = 64 (or 32) tokens; a block
// of Bk = ratio * S tokens is `ratio` consecutive sub-blocks, so block-level
// lists expand to sub-block lists here (nb: key sub-blocks, nq: query
// sub-blocks).  Two sources of blocks:
//   GeomSched   fixed-size tiles (packed or 3D-padded), CSR rows = blocks;
//   TableSched  clusters of any size, each starting on a sub-block boundary
//               (start[c], size[c] per head), CSR rows = query clusters and
//               columns = key clusters.
__device__ __forceinline__ int32_t clamp_valid(int32_t v, int32_t sub) {
  return v < 0 ? 0 : (v > sub ? sub : v);
}

struct GeomSched {
  // 3D-padded layouts hold sub-blocks of padding only inside a kept block
  static constexpr bool kSkipEmpty = true;
  Geom g;
  int32_t ratio, sub;
  __device__ int32_t ncols() const { return g.nb; }
  __device__ int32_t qvalid(int64_t, int32_t i) const {
    return clamp_valid(block_valid(g, i / ratio) - (i % ratio) * sub, sub);
  }
  __device__ int64_t row(int64_t bh, int32_t i) const { return bh * g.nb + i / ratio; }
  __device__ void keys(int64_t, int32_t jb, int32_t* j0, int32_t* j1) const {
    *j0 = jb * ratio;
    *j1 = *j0 + ratio;
  }
  __device__ int32_t kvalid(int64_t bh, int32_t j) const { return qvalid(bh, j); }
  __device__ int32_t rotation(int32_t i) const { return i; }   // same layout both sides
};

// last cluster c in [0, n) with start[c] <= pos (the one whose slots hold pos)
__device__ __forceinline__ int32_t owner_of(const int32_t* start, int32_t n, int32_t pos) {
  int32_t lo = 0, hi = n - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (start[mid] <= pos) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

struct TableSched {
  // clusters start on sub-block boundaries, so every sub-block of a kept key
  // cluster's range holds some of its keys (an empty cluster has no range)
  static constexpr bool kSkipEmpty = false;
  const int32_t *q_start, *q_size, *k_start, *k_size;
  int32_t nq, nk, sub;
  __device__ int32_t ncols() const { return nk; }
  __device__ int32_t qvalid(int64_t bh, int32_t i) const {
    const int32_t* st = q_start + bh * (nq + 1);
    const int32_t pos = i * sub;
    if (pos >= st[nq]) return 0;
    const int32_t c = owner_of(st, nq, pos);
    return clamp_valid(st[c] + q_size[bh * nq + c] - pos, sub);
  }
  __device__ int64_t row(int64_t bh, int32_t i) const {
    return bh * nq + owner_of(q_start + bh * (nq + 1), nq, i * sub);
  }
  __device__ void keys(int64_t bh, int32_t jc, int32_t* j0, int32_t* j1) const {
    const int32_t s0 = k_start[bh * (nk + 1) + jc];
    *j0 = s0 / sub;
    *j1 = (s0 + k_size[bh * nk + jc] + sub - 1) / sub;
  }
  __device__ int32_t kvalid(int64_t bh, int32_t j) const {
    const int32_t* st = k_start + bh * (nk + 1);
    const int32_t pos = j * sub;
    if (pos >= st[nk]) return 0;
    const int32_t c = owner_of(st, nk, pos);
    return clamp_valid(st[c] + k_size[bh * nk + c] - pos, sub);
  }
  __device__ int32_t rotation(int32_t) const { return 0; }
};

// Step lists.  With groups of four 64-token query sub-blocks (one per SIMD)
// the attention kernel walks STEPS of two list entries (a, b): a step costs
// one key block's time, and each wavefront works on the entry its sub-block
// keeps.  Two entries share a step when their keep masks are disjoint, so a
// union entry that only some sub-blocks keep no longer leaves the other
// SIMDs idle for a whole key block.  Over all items of a call (query blocks
// regrouped by their lists) this takes the steps to 0.886 of the union
// entries at Wan2.1-720p top-p 0.9 (kept pairs per step and sub-block 0.856
// -> 0.967) and to 0.759 in HunyuanVideo-720p fixed-fraction mode (0.721 ->
// 0.950).  A step holding two blocks keeps its copy and ring cost; pairing
// only within windows of 64 consecutive entries paired less and ran slower.
//
// Pairing: entries are bucketed by mask (1..15) and ranked in list order;
// the rules below, in order, pair the k-th free entry of the first bucket
// with the k-th free entry of the second: three keepers with the other one,
// two with the other two, two with one of the other two, one with one.  The
// entry from a rule's first bucket heads the step and keeps its place in the
// list order (wherever its partner stood); the partner leaves the list.  Ranks
// follow the list order, so the pairing is deterministic.
constexpr int kPairRules = 25;
constexpr int8_t kPairRule[kPairRules][2] = {
    {7, 8},  {11, 4}, {13, 2}, {14, 1},                                     // 3 + 1
    {3, 12}, {5, 10}, {6, 9},                                               // 2 + 2
    {3, 4},  {3, 8},  {5, 2},  {5, 8}, {6, 1}, {6, 8}, {9, 2}, {9, 4},      // 2 + 1
    {10, 1}, {10, 4}, {12, 1}, {12, 2},
    {1, 2},  {1, 4},  {1, 8},  {2, 4}, {2, 8}, {4, 8}};                     // 1 + 1
constexpr int32_t kPairMaxNb = 4096;   // staging in LDS: 3 words per key sub-block

// out_mode: 0 = one word per entry (the entry walks), 2 = steps paired as
// above (nb <= kPairMaxNb).
template <typename Sched, int out_mode>
__global__ void __launch_bounds__(kSchedThreads)
union_kernel(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
             int32_t* __restrict__ list, int32_t* __restrict__ count, int32_t nb, int32_t nq,
             int32_t groups, int32_t group_size, Sched sc, const int32_t* __restrict__ perm) {
  const int32_t ncols = sc.ncols();
  extern __shared__ uint32_t mask[];  // [nb]; out_mode 2: then entw[nb], pos[nb]
  __shared__ int32_t wave_tot[kSchedThreads / 64];
  __shared__ int32_t s_base[16], s_rule[kPairRules][3];
  const int64_t item = blockIdx.x;
  const int64_t bh = item / groups;
  const int32_t g = (int32_t)(item % groups);
  const int t = threadIdx.x;
  for (int32_t j = t; j < nb; j += kSchedThreads) mask[j] = 0u;
  __syncthreads();
  // the group's query sub-blocks: consecutive, or as regrouped (perm, with
  // -1 for empty slots)
  const int32_t* gp = perm ? perm + item * group_size : nullptr;
  for (int m = 0; m < group_size; ++m) {
    const int32_t i = gp ? gp[m] : g * group_size + m;   // query sub-block
    if (i < 0 || i >= nq) continue;
    if (sc.qvalid(bh, i) == 0) continue;     // padding only: nothing to compute
    const int64_t row = sc.row(bh, i);
    const int32_t e0 = row_ptr[row], e1 = row_ptr[row + 1];
    for (int32_t e = e0 + t; e < e1; e += kSchedThreads) {
      const int32_t jb = col_idx[e];
      if (jb < 0 || jb >= ncols) continue;
      int32_t j0, j1;
      sc.keys(bh, jb, &j0, &j1);
      for (int32_t j = j0; j < j1; ++j)
        if (j < nb && (!Sched::kSkipEmpty || sc.kvalid(bh, j) > 0)) atomicOr(&mask[j], 1u << m);
    }
  }
  __syncthreads();
  int32_t* out = list + item * (out_mode == 0 ? nb : 2 * nb);
  uint32_t* entw = mask + nb;   // out_mode 2: the list in LDS
  int32_t off = 0;
  const int lane = t & 63, wv = t >> 6;
  // the list starts at the group's own diagonal key sub-block and wraps
  // around, so neighbouring query groups walk the same keys at the same time
  int32_t j0 = sc.rotation(gp ? max(gp[0], 0) : g * group_size);
  j0 = j0 < nb ? j0 : 0;
  for (int32_t base = 0; base < nb; base += kSchedThreads) {
    const int32_t jj = base + t;
    const int32_t j = jj < nb ? (jj + j0 < nb ? jj + j0 : jj + j0 - nb) : nb;
    const uint32_t m = jj < nb ? mask[j] : 0u;
    const unsigned long long bal = __ballot(m != 0u);
    const int32_t before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wv] = __popcll(bal);
    __syncthreads();
    int32_t wbase = 0, tot = 0;
    for (int k = 0; k < kSchedThreads / 64; ++k) {
      if (k < wv) wbase += wave_tot[k];
      tot += wave_tot[k];
    }
    if (m != 0u) {
      const int32_t word = j | (sc.kvalid(bh, j) << 13) | (int32_t)(m << 24);
      const int32_t at = off + wbase + before;
      if constexpr (out_mode == 0) out[at] = word;
      else entw[at] = (uint32_t)word;
    }
    off += tot;
    __syncthreads();
  }
  if constexpr (out_mode == 0) {
    if (t == 0) count[item] = off;
    return;
  }

  // ---- pairing (out_mode 2); mask[] is free from here on
  const int32_t n = off;
  uint32_t* key = mask;          // (bucket << 16) | rank in the bucket
  uint32_t* pos = mask + 2 * nb; // entry index by (bucket start + rank)
  if (wv == 0) {
    int32_t cnt[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) cnt[b] = 0;
    for (int32_t c0 = 0; c0 < n; c0 += 64) {
      const int32_t e = c0 + lane;
      const uint32_t m = e < n ? (entw[e] >> 24) & 15u : 0u;
      int32_t rank = 0;
#pragma unroll
      for (int b = 1; b < 16; ++b) {
        const unsigned long long bal = __ballot(m == (uint32_t)b);
        if (m == (uint32_t)b) rank = cnt[b] + __popcll(bal & ((1ull << lane) - 1ull));
        cnt[b] += __popcll(bal);
      }
      if (e < n) key[e] = (m << 16) | (uint32_t)rank;
    }
    if (lane == 0) {
      int32_t rem[16], base = 0;
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        s_base[b] = base;
        base += cnt[b];
        rem[b] = cnt[b];
      }
#pragma unroll
      for (int r = 0; r < kPairRules; ++r) {
        const int c1 = kPairRule[r][0], c2 = kPairRule[r][1];
        const int32_t k = min(rem[c1], rem[c2]);
        s_rule[r][0] = k;
        s_rule[r][1] = cnt[c1] - rem[c1];
        s_rule[r][2] = cnt[c2] - rem[c2];
        rem[c1] -= k;
        rem[c2] -= k;
      }
    }
  }
  __syncthreads();
  for (int32_t e = t; e < n; e += kSchedThreads) {
    const uint32_t k = key[e];
    pos[s_base[k >> 16] + (int32_t)(k & 0xffffu)] = (uint32_t)e;
  }
  __syncthreads();
  // steps: the heads in list order, each with its partner (or none)
  int32_t soff = 0;
  for (int32_t base = 0; base < n; base += kSchedThreads) {
    const int32_t e = base + t;
    bool head = e < n;
    int32_t partner = -1;
    if (e < n) {
      const uint32_t k = key[e];
      const int c = (int)(k >> 16);
      const int32_t r = (int32_t)(k & 0xffffu);
#pragma unroll
      for (int ri = 0; ri < kPairRules; ++ri) {
        const int c1 = kPairRule[ri][0], c2 = kPairRule[ri][1];
        const int32_t kk = s_rule[ri][0], sa = s_rule[ri][1], sb = s_rule[ri][2];
        if (c == c1 && r >= sa && r < sa + kk) partner = (int32_t)pos[s_base[c2] + sb + (r - sa)];
        if (c == c2 && r >= sb && r < sb + kk) head = false;
      }
    }
    const unsigned long long bal = __ballot(head);
    const int32_t before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wv] = __popcll(bal);
    __syncthreads();
    int32_t wbase = 0, tot = 0;
    for (int k = 0; k < kSchedThreads / 64; ++k) {
      if (k < wv) wbase += wave_tot[k];
      tot += wave_tot[k];
    }
    if (head) {
      const int32_t at = soff + wbase + before;
      out[2 * at] = (int32_t)entw[e];
      out[2 * at + 1] = partner >= 0 ? (int32_t)entw[partner] : 0;
    }
    soff += tot;
    __syncthreads();
  }
  if (t == 0) count[item] = soff;
}

// ---------------------------------------------------------------------------
// Regrouping of query blocks (fixed-size blocks of one 64-token sub-block):
// the workgroup of an item streams the union of its four query blocks'
// lists, and a union entry costs the whole workgroup a key block whether one
// or four of the blocks keep it, so grouping blocks whose lists overlap
// shortens the unions.  Per window of WIN consecutive query blocks of a
// head, greedily: the lowest block not yet taken anchors a group, then three
// times the free block of the window that maximises 3 |L n U| - |L| (U: the
// union of the group so far, L: the candidate's list; ties to the lower
// block) joins it.  perm[(bh * groups + g) * 4 + m] = the m-th block of group
// g (-1 for the empty slots of the last group), the groups of a window in
// anchor order, so that neighbouring items still work on neighbouring blocks.
// One workgroup per window; thread t holds block t's list as a bitmap in
// registers, the group's union in registers too.  Windows of 512 blocks
// shorten the unions of fixed-fraction masks by a further 2.4% (top-p masks:
// 0.2-0.4%), but each pick then costs ~3x as long (twice the candidates per
// SIMD), 0.57 instead of 0.25 ms at HunyuanVideo 720p: 256 is the default.
// ---------------------------------------------------------------------------
constexpr int kGWin = 256;   // query blocks per window = threads per workgroup

// Maximum of an unsigned value over the wavefront, returned to every lane:
// running maxima within each row of 16 lanes (DPP row shifts), then across
// rows (row broadcasts of lanes 15 and 31); lane 63 holds the result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

template <int WORDS, int WIN>
__global__ void __launch_bounds__(WIN)
group_kernel(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
             int32_t* __restrict__ perm, int32_t nq, int32_t groups, int32_t windows) {
  // row stride: a whole number of 16-byte units (the union update reads the
  // winner's row four words at a time, the same address in every lane)
  constexpr int kStride = WORDS + 4;
  static_assert(WORDS <= 64 && WORDS % 4 == 0, "scores must fit 14 bits");
  constexpr int kNW = WIN / 64;          // 64-bit words of the taken mask
  constexpr int kTB = WIN == 512 ? 9 : 8; // bits of the thread index in a key
  static_assert(WIN == 256 || WIN == 512, "window of 256 or 512 blocks");
  __shared__ __align__(16) uint32_t bs[WIN * kStride];
  __shared__ uint32_t red[2][kNW];
  const int64_t bh = blockIdx.x / windows;
  const int32_t w0 = (int32_t)(blockIdx.x % windows) * WIN;
  const int32_t nrow = min(WIN, nq - w0);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int32_t* out = perm + (bh * groups + w0 / 4) * 4;   // this window's groups
  // every row keeps every key block: no grouping changes a union, so the
  // groups stay positional (the all-kept launch pays no search)
  {
    const int64_t r0 = bh * nq + w0;
    const int64_t kept = (int64_t)row_ptr[r0 + nrow] - row_ptr[r0];
    if (kept == (int64_t)nrow * nq) {
      for (int32_t x = t; x < 4 * ((nrow + 3) / 4); x += WIN) out[x] = x < nrow ? w0 + x : -1;
      return;
    }
  }
  // the window's bitmaps: thread t builds row t's in its own LDS row.  The
  // row's column indices are read as 16-byte vectors from the 16-byte aligned
  // address at or below its first entry, sixteen vectors (64 entries) at a
  // time so that their latencies overlap; a vector that would start before
  // the array or pass the row's end is read as single words.  Every entry's
  // bit is OR-ed into the row with an LDS atomic that returns nothing (no
  // wait; any column order works); entries outside the row OR zero into the
  // row's padding word.
  for (int w = 0; w < kStride; ++w) bs[t * kStride + w] = 0u;
  if (t < nrow) {
    const int64_t r = bh * nq + w0 + t;
    const int32_t e0 = row_ptr[r], e1 = row_ptr[r + 1];
    uint32_t* row = bs + t * kStride;
    // col_idx + x is 16-byte aligned when (x + mis) % 4 == 0
    const int32_t mis = (int32_t)((reinterpret_cast<uintptr_t>(col_idx) >> 2) & 3);
    for (int32_t e = ((e0 + mis) & ~3) - mis; e < e1; e += 64) {
      int4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int32_t x = e + 4 * u;
        if (x >= 0 && x + 3 < e1) {
          v[u] = *reinterpret_cast<const int4*>(col_idx + x);
        } else {
          v[u].x = x >= e0 && x < e1 ? col_idx[x] : -1;
          v[u].y = x + 1 >= e0 && x + 1 < e1 ? col_idx[x + 1] : -1;
          v[u].z = x + 2 >= e0 && x + 2 < e1 ? col_idx[x + 2] : -1;
          v[u].w = x + 3 >= e0 && x + 3 < e1 ? col_idx[x + 3] : -1;
        }
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int32_t x = e + 4 * u + c;
          const int32_t j = c == 0 ? v[u].x : c == 1 ? v[u].y : c == 2 ? v[u].z : v[u].w;
          const bool ok = x >= e0 && j >= 0 && j < 32 * WORDS;
          atomicOr(row + (ok ? (j >> 5) : WORDS), ok ? 1u << (j & 31) : 0u);
        }
      }
    }
  }
  __syncthreads();
  uint32_t mine[WORDS], un[WORDS];
  int32_t cnt = 0;
#pragma unroll
  for (int w = 0; w < WORDS; ++w) {
    mine[w] = bs[t * kStride + w];
    cnt += __popc(mine[w]);
  }
  // blocks taken so far, as a WIN-bit mask that every thread keeps alike
  // (every winner is known to all threads), so the anchor scan needs no
  // barrier; bits past nrow start set.  Indexed only with compile-time word
  // numbers (selects), so the mask stays in registers.
  uint64_t tk[kNW];
#pragma unroll
  for (int x = 0; x < kNW; ++x) {
    const int32_t lo = 64 * x;
    tk[x] = nrow >= lo + 64 ? 0ull : (nrow <= lo ? ~0ull : ~((1ull << (nrow - lo)) - 1ull));
  }
#define SVSA_TAKE(b)                                   \
  do {                                                 \
    const uint64_t bit_ = 1ull << ((b) & 63);          \
    const int32_t x_ = (b) >> 6;                       \
    _Pragma("unroll") for (int x = 0; x < kNW; ++x) tk[x] |= x_ == x ? bit_ : 0ull; \
  } while (0)
#define SVSA_TAKEN(b)                                                            \
  ({                                                                             \
    const int32_t b_ = (b);                                                      \
    uint64_t w_ = 0ull;                                                          \
    _Pragma("unroll") for (int x = 0; x < kNW; ++x) w_ = (b_ >> 6) == x ? tk[x] : w_; \
    (w_ >> (b_ & 63)) & 1ull;                                                    \
  })
  int32_t g = 0;
  int buf = 0;
  for (int32_t a = 0; a < nrow; ++a) {
    if (SVSA_TAKEN(a)) continue;   // uniform: the masks agree
    SVSA_TAKE(a);
    if (t == 0) out[4 * g] = w0 + a;
#pragma unroll
    for (int w = 0; w < WORDS; w += 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(&bs[a * kStride + w]);
      un[w] = q.x;
      un[w + 1] = q.y;
      un[w + 2] = q.z;
      un[w + 3] = q.w;
    }
    for (int m = 1; m < 4; ++m) {
      uint32_t key = 0u;
      if (!SVSA_TAKEN(t)) {
        int32_t inter = 0;
        // four independent sums (a single chain of dependent adds is latency bound)
        int32_t i4[4] = {0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < WORDS; ++w) i4[w & 3] += __popc(mine[w] & un[w]);
        inter = (i4[0] + i4[1]) + (i4[2] + i4[3]);
        // 3 |L n U| - |L| made positive (< 2^14), ties to the lower t
        const uint32_t score = (uint32_t)(3 * inter - cnt + 32 * WORDS + 1);
        key = (score << kTB) | (uint32_t)(WIN - 1 - t);
      }
      key = wave_max_u32(key);
      if (lane == 0) red[buf][wave] = key;
      __syncthreads();
      uint32_t best = red[buf][0];
#pragma unroll
      for (int x = 1; x < kNW; ++x) best = max(best, red[buf][x]);
      buf ^= 1;                  // red[buf] is rewritten only after the next barrier
      const int32_t win = best == 0u ? -1 : (int32_t)(WIN - 1 - (best & ((1u << kTB) - 1u)));
      if (t == 0) out[4 * g + m] = win < 0 ? -1 : w0 + win;
      if (win < 0) continue;     // uniform: no free block left (the slot stays -1)
      SVSA_TAKE(win);
#pragma unroll
      for (int w = 0; w < WORDS; w += 4) {
        const uint4 q = *reinterpret_cast<const uint4*>(&bs[win * kStride + w]);
        un[w] |= q.x;
        un[w + 1] |= q.y;
        un[w + 2] |= q.z;
        un[w + 3] |= q.w;
      }
    }
    ++g;
  }
#undef SVSA_TAKE
#undef SVSA_TAKEN
}

// Work queues.  The query groups of one (b, h) are cut into kHeadParts runs
// of consecutive groups (units); the items of a unit all go to one of kQueues
// queues (one per XCD of the chip) and, inside it, stay in query group order,
// so the workgroups running on one XCD at a time work on neighbouring query
// groups of the same head and share its key blocks in that XCD's L2.  Units
// are taken heaviest first (work = union lengths plus a per-item constant)
// and each goes to the queue with the least work so far, so every queue ends
// with its lightest units and the last items of the launch are short.  Four
// parts per head beat whole heads per queue by 3-4% at Wan2.1 and
// HunyuanVideo 720p (A/B on one box; 3 to 8 parts, or units of 64 groups,
// within 0.5% of each other): the parts of a head run at the same time on
// several XCDs, which then share its K / V^T in the Infinity Cache, and the
// finer units balance the queues' ends.
// meta = {base[8], len[8], take[8]}; take[] is zeroed here, before every
// attention launch.
constexpr int kQueues = 8;
constexpr int kQueueThreads = 1024;
constexpr int kQueueMaxBh = 2048;   // units placed by work; beyond, whole heads by bh % 8
constexpr int kItemCost = 4;        // fixed cost of one item, in key blocks
constexpr int kHeadParts = 4;       // units one (b, h) is cut into

__global__ void __launch_bounds__(kQueueThreads)
queue_kernel(const int32_t* __restrict__ count, int32_t* __restrict__ queue,
             int32_t* __restrict__ meta, int32_t bh_count, int32_t groups, int32_t parts) {
  // units: each (b, h) split into `parts` runs of consecutive query groups
  // (gpu groups each, the last one shorter), placed like whole heads
  __shared__ unsigned long long work[kQueueMaxBh];
  __shared__ int32_t qof[kQueueMaxBh];   // queue of each unit
  __shared__ int32_t off[kQueueMaxBh];   // its first position inside that queue
  __shared__ int32_t by_rank[kQueueMaxBh];  // units, heaviest first
  __shared__ int32_t len[kQueues], base[kQueues];
  const int t = threadIdx.x;
  parts = max(1, min(parts, groups));
  const int32_t gpu = max(1, (groups + parts - 1) / parts);   // query groups per unit
  parts = max(1, (groups + gpu - 1) / gpu);                    // no empty unit
  const int32_t units = bh_count * parts;
  const bool by_work = units <= kQueueMaxBh;
  if (by_work) {
    // work per unit: every thread adds a strided share of all items (loads
    // independent and coalesced), integer sums so the order does not matter
    for (int32_t u = t; u < units; u += kQueueThreads) work[u] = 0ull;
    __syncthreads();
    // each thread sums a contiguous run of items (one division to find where
    // it starts, then (b, g, part) advance by one), adding to a unit's work
    // once per unit it touches
    const int64_t n_items = (int64_t)bh_count * groups;
    const int64_t per = (n_items + kQueueThreads - 1) / kQueueThreads;
    const int64_t it0 = min(n_items, (int64_t)t * per), it1 = min(n_items, it0 + per);
    if (it0 < it1) {
      int32_t b = (int32_t)(it0 / groups), g = (int32_t)(it0 % groups);
      int32_t part = g / gpu, next = min(groups, (part + 1) * gpu);
      unsigned long long acc = 0ull;
      for (int64_t c0 = it0; c0 < it1; c0 += 16) {
        int32_t cb[16];   // sixteen counts in flight at a time
#pragma unroll
        for (int j = 0; j < 16; ++j) cb[j] = c0 + j < it1 ? count[c0 + j] : 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int64_t it = c0 + j;
          if (it >= it1) break;
          acc += (unsigned long long)(cb[j] + kItemCost);
          if (++g == next || it + 1 == it1) {   // the unit ends here (or the run does)
            atomicAdd(&work[b * parts + part], acc);
            acc = 0ull;
            if (g == groups) { g = 0; ++b; part = 0; } else { ++part; }
            next = min(groups, (part + 1) * gpu);
          }
        }
      }
    }
    __syncthreads();
    for (int32_t u = t; u < units; u += kQueueThreads) {
      const unsigned long long wu = work[u];
      int32_t rank = 0;
#pragma unroll 8
      for (int32_t o = 0; o < units; ++o) {
        const unsigned long long wo = work[o];   // same address in every lane
        rank += (wo > wu) || (wo == wu && o < u);
      }
      by_rank[rank] = u;
    }
  }
  __syncthreads();
  if (t < 64) {
    // wavefront 0 places the units in rank order (each choice depends on the
    // ones before).  Lane j loads unit k0 + j of a batch of 64 (one LDS read
    // for the batch); the loop takes each unit's values with readlane, so
    // they, the queue loads and the choice are wave-uniform (scalar unit)
    // and no step waits on LDS.
    const int lane = t;
    unsigned long long load[kQueues];
    int32_t lenr[kQueues];
#pragma unroll
    for (int x = 0; x < kQueues; ++x) { load[x] = 0ull; lenr[x] = 0; }
    const int32_t n_place = by_work ? units : 0;
    for (int32_t k0 = 0; k0 < n_place; k0 += 64) {
      const int32_t kj = k0 + lane;
      const int32_t uj = kj < n_place ? by_rank[kj] : 0;
      const unsigned long long wj = kj < n_place ? work[uj] : 0ull;
      const int32_t pj = uj % parts;                                   // the unit's part
      const int32_t nj = min(groups, (pj + 1) * gpu) - pj * gpu;       // and its groups
      const int32_t cnt = min(64, n_place - k0);
      for (int32_t j = 0; j < cnt; ++j) {
        const int32_t u = __builtin_amdgcn_readlane(uj, j);
        const uint32_t wlo = (uint32_t)__builtin_amdgcn_readlane((int32_t)(uint32_t)wj, j);
        const uint32_t whi = (uint32_t)__builtin_amdgcn_readlane((int32_t)(uint32_t)(wj >> 32), j);
        const unsigned long long w = ((unsigned long long)whi << 32) | wlo;
        const int32_t n = __builtin_amdgcn_readlane(nj, j);
        int best = 0;
        unsigned long long best_load = load[0];
        int32_t best_len = lenr[0];
#pragma unroll
        for (int x = 1; x < kQueues; ++x)
          if (load[x] < best_load) { best = x; best_load = load[x]; best_len = lenr[x]; }
        if (lane == 0) {
          qof[u] = best;
          off[u] = best_len;
        }
#pragma unroll
        for (int x = 0; x < kQueues; ++x)
          if (x == best) { lenr[x] += n; load[x] += w; }
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int x = 0; x < kQueues; ++x)
        len[x] = by_work ? lenr[x] : ((bh_count - x + kQueues - 1) / kQueues) * groups;
    }
  }
  if (t == 0) {
    int32_t acc = 0;
    for (int x = 0; x < kQueues; ++x) { base[x] = acc; acc += len[x]; }
    for (int x = 0; x < kQueues; ++x) {
      meta[x] = base[x];
      meta[kQueues + x] = len[x];
      meta[2 * kQueues + x] = 0;
    }
  }
  __syncthreads();
  // every item into its unit's place: contiguous runs per thread again, with
  // (b, g, part) advanced by one per item
  const int64_t items = (int64_t)bh_count * groups;
  const int64_t per_t = (items + kQueueThreads - 1) / kQueueThreads;
  const int64_t i0 = min(items, (int64_t)t * per_t), i1 = min(items, i0 + per_t);
  if (i0 < i1) {
    int32_t b = (int32_t)(i0 / groups), g = (int32_t)(i0 % groups);
    int32_t part = g / gpu;
    for (int64_t it = i0; it < i1; ++it) {
      if (by_work) {
        const int32_t u = b * parts + part;
        queue[base[qof[u]] + off[u] + (g - part * gpu)] = (int32_t)it;
      } else {
        queue[base[b % kQueues] + (b / kQueues) * groups + g] = (int32_t)it;
      }
      if (++g == groups) { g = 0; ++b; part = 0; }
      else if (g == (part + 1) * gpu) { ++part; }
    }
  }
}

// ---------------------------------------------------------------------------
// V^T per key block: vt[bh][j][d][pos(kv)] = v[bh][j * BK + kv][d], with the
// key order inside each 16-key MFMA step permuted (pos, below) so that the
// 8 keys one lane-half feeds to an MFMA step are 16 contiguous bytes.  One
// workgroup per key block; the block goes through LDS so that both the reads
// and the writes are whole coalesced rows.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int vt_pos(int kv) {
  // kv = 16 s + 8 a + 4 h + e  ->  16 s + 8 h + 4 a + e
  return (kv & ~15) | ((kv & 4) << 1) | ((kv & 8) >> 1) | (kv & 3);
}

constexpr int kVtThreads = 256;

// Second half of the transpose: the key block staged row-major in LDS goes
// out as D rows of BK keys in vt_pos order; output word i holds positions
// 2p, 2p+1 of row d.
template <int D, int BK>
__device__ __forceinline__ void vt_store(const uint16_t (*tile)[D + 2], uint16_t* dst) {
  for (int i = threadIdx.x; i < BK * D / 2; i += kVtThreads) {
    const int d = (2 * i) / BK, p = (2 * i) % BK;
    // positions p, p+1 hold keys vt_pos^-1(p), vt_pos^-1(p+1) (vt_pos is an involution)
    const uint32_t lo = tile[vt_pos(p)][d], hi = tile[vt_pos(p + 1)][d];
    reinterpret_cast<uint32_t*>(dst)[i] = lo | (hi << 16);
  }
}

template <int D, int BK>
__global__ void __launch_bounds__(kVtThreads)
vt_kernel(const __bf16* __restrict__ v, __bf16* __restrict__ vt, int32_t nb, int32_t Npad) {
  __shared__ uint16_t tile[BK][D + 2];  // +2: odd word stride, conflict-free column reads
  const int64_t bh = blockIdx.x / nb;
  const int32_t j = blockIdx.x % nb;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(v) + (bh * Npad + (int64_t)j * BK) * D;
  uint16_t* dst = reinterpret_cast<uint16_t*>(vt) + (bh * Npad + (int64_t)j * BK) * D;
  for (int i = threadIdx.x; i < BK * D / 2; i += kVtThreads) {
    const int kv = (2 * i) / D, d = (2 * i) % D;
    const uint32_t w = reinterpret_cast<const uint32_t*>(src)[i];
    tile[kv][d] = (uint16_t)(w & 0xffffu);
    tile[kv][d + 1] = (uint16_t)(w >> 16);
  }
  __syncthreads();
  vt_store<D, BK>(tile, dst);
}

// The same V^T from natural-order V: the rows of key sub-block j are gathered
// from their natural positions (the tile reorder of [PSA] Sec. 3.2, inverted
// per row) and padding slots become zeros, so the result equals vt_kernel run
// on the reordered V without that tensor ever being written.  nbs sub-blocks
// of BK rows per (b, h).
template <int D, int BK>
__global__ void __launch_bounds__(kVtThreads)
stage_v_kernel(const __bf16* __restrict__ v, __bf16* __restrict__ vt, int32_t nbs, Geom g) {
  static_assert(BK <= kVtThreads, "one thread per row for the row map");
  __shared__ __align__(16) uint16_t tile[BK][D + 2];
  __shared__ int32_t nat[BK];
  const int64_t bh = blockIdx.x / nbs;
  const int32_t j = blockIdx.x % nbs;
  if (threadIdx.x < BK) {
    const int32_t p = j * BK + (int32_t)threadIdx.x;  // tiled row
    const int32_t blk = p / g.Bk, slot = p - blk * g.Bk;
    nat[threadIdx.x] =
        (blk < g.nb && slot < block_valid(g, blk)) ? natural_row(g, blk, slot) : -1;
  }
  __syncthreads();
  constexpr int kChunks = D / 8;  // 16-byte chunks per row
  const uint4* src = reinterpret_cast<const uint4*>(v) + bh * g.N * kChunks;
  for (int i = threadIdx.x; i < BK * kChunks; i += kVtThreads) {
    const int kv = i / kChunks, c = i % kChunks;
    const int32_t n = nat[kv];
    const uint4 u = n >= 0 ? src[(int64_t)n * kChunks + c] : make_uint4(0u, 0u, 0u, 0u);
    uint32_t* row = reinterpret_cast<uint32_t*>(&tile[kv][8 * c]);  // rows are 4-byte aligned
    row[0] = u.x;
    row[1] = u.y;
    row[2] = u.z;
    row[3] = u.w;
  }
  __syncthreads();
  vt_store<D, BK>(tile, reinterpret_cast<uint16_t*>(vt) + (bh * g.Npad + (int64_t)j * BK) * D);
}

// ---------------------------------------------------------------------------
// Attention kernel.
// ---------------------------------------------------------------------------
template <int D, int BK>
struct Cfg {
  static constexpr int kTileBytes = BK * D * 2;  // one K (or V) tile
  static constexpr int kRowBytes = 2 * D;    // K row
  static constexpr int kVtRowBytes = 2 * BK;  // V^T row
  static constexpr int kDmaPerTile = kTileBytes / 1024;          // 1 KB per wavefront copy
  static constexpr int kDmaPerWave = 2 * kDmaPerTile / kWaves;   // K + V, split over the waves
  static constexpr int kSTiles = BK / 32;    // 32-key tiles of S^T
  static constexpr int kPSteps = BK / 16;    // 16-key MFMA steps of P V
  static_assert(kDmaPerWave >= 1 && kDmaPerWave <= 4 && (2 * kDmaPerTile) % kWaves == 0,
                "copies must split");
};

// K tile: row-major, 16-byte chunks XOR-swizzled by row so that the S^T
// A-operand reads (32 consecutive rows at one column) hit distinct banks.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
// V^T tile: one row per head-dimension index (2 BK bytes), 16-byte chunks
// XOR-swizzled by row so that 16 consecutive rows read at one column (the
// V^T A-operand pattern) hit distinct banks.
template <int BK>
__device__ __forceinline__ int vt_swz(int row) {
  static_assert(BK == 64, "key tiles are 64 keys");
  return (row >> 1) & 7;
}

// Cross-half exchange: the value held by lane (lane ^ 32).
__device__ __forceinline__ float swap_halves(float x, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

// s_waitcnt immediates (gfx9 layout: vmcnt[3:0,15:14], expcnt[6:4], lgkmcnt[11:8])
constexpr int waitcnt_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kWaitLgkm0 = 0xC07F;

// Workgroup barrier without an implied memory fence: LDS reads are drained
// (lgkmcnt) and HBM->LDS copies are waited for explicitly, so copies of later
// key blocks stay in flight across the barrier.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per-wave state of the online softmax.
template <int D, int BK>
struct WaveState {
  static constexpr int kDT = D / 32;
  f32x16 oacc[kDT];
  f32x16 sacc[BK / 32];
  bf16x8 pk[BK / 16];
  bf16x8 qreg[D / 16];
  bf16x8 pre[kPre];
  float m_run, l_run, o_alpha;
  bool o_rescale;
};

// Where the epilogue writes O: tile order (natural == 0; the cluster path
// always), or the natural (t, h, w) order of the fixed-block geometry g
// (natural == 1), where padding slots have no row and are not written.
struct OutMap {
  Geom g;
  int32_t natural;
};

struct Ctx {
  __amdgpu_buffer_rsrc_t k_rsrc;   // K of this (b, h)
  __amdgpu_buffer_rsrc_t vt_rsrc;  // V^T blocks of this (b, h)
  const int32_t* lst;
  int32_t n_u, T, nb;   // n_u: key tiles streamed (list entries, or pairs of them)
  int32_t n_list;       // list entries
  float c_log2;
  int wave, lane, qb, l32, hh;
  uint32_t dma_off[4];  // per-lane source offsets of this wave's copies
  uint32_t vt_sel[4];   // paired mode: all ones where a lane's V^T copy comes from entry b
  bool has_rows;
};

// List data of one key tile.  Plain mode: one entry (a) per tile of BK keys.
// Paired mode (32-token list entries streamed two at a time as the halves of
// a 64-key tile, query sub-blocks of 32 rows, one per wavefront): entries a
// and b; an entry past the end of the list has its keep mask cleared.
struct TileEnt {
  int32_t a, b;
};

// Per-lane source byte offset, inside one key block, of this wavefront's u-th
// HBM -> LDS copy (each copy is 64 lanes x 16 contiguous LDS bytes; the LDS
// swizzle is applied on the source side).  Copies 0 .. kDmaPerTile-1 fill the
// K tile, the rest the V^T tile.
template <int D, int BK>
__device__ __forceinline__ uint32_t copy_src_off(int wave, int lane, int u) {
  using C = Cfg<D, BK>;
  const int ld = wave + u * kWaves;
  const bool is_v = ld >= C::kDmaPerTile;
  const int byte = (is_v ? ld - C::kDmaPerTile : ld) * 1024 + lane * 16;
  const int rb = is_v ? C::kVtRowBytes : C::kRowBytes;
  const int row = byte / rb;
  const int lc = ((byte % rb) >> 4) ^ (is_v ? vt_swz<BK>(row) : k_swz<D>(row));
  return (uint32_t)(row * rb + lc * 16);
}

// Issue this wavefront's copies of key block j into (kdst, vdst): buffer
// loads with the LDS destination (MUBUF "lds"), addressed by the head's buffer
// resource, a wave-uniform block offset and a loop-invariant per-lane offset.
// (A MUBUF copy, unlike the FLAT global_load_lds form, leaves the compiler's
// counting of LDS reads exact: with a FLAT copy in flight it would wait for
// every outstanding LDS read before each use.)
template <int D, int BK, bool PR>
__device__ __forceinline__ void issue_copies(const Ctx& cx, TileEnt te, char* kdst, char* vdst,
                                             int32_t wave_off) {
  using C = Cfg<D, BK>;
  if constexpr (PR) {
    // Paired mode: K copies lie within one half of the tile, so their block
    // offset is wave-uniform (the half's row offset is folded into dma_off);
    // each lane of a V^T copy takes its 16 bytes from entry a's or b's block.
    static_assert(BK == 64 && C::kDmaPerTile % kWaves == 0, "paired tiles are 64 keys");
    constexpr int32_t kHalfBytes = 32 * D * 2;
    constexpr int kPerWaveK = C::kDmaPerTile / kWaves;
    const int32_t ja = (te.a & 0x1fff) * kHalfBytes, jb = (te.b & 0x1fff) * kHalfBytes;
#pragma unroll
    for (int u = 0; u < C::kDmaPerWave; ++u) {
      if (u < kPerWaveK) {
        const bool hb = (cx.wave + u * kWaves) * 1024 >= kHalfBytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            cx.k_rsrc, (__attribute__((address_space(3))) void*)(kdst + wave_off + u * kWaves * 1024), 16,
            (int)cx.dma_off[u], hb ? jb : ja, 0, 0);
      } else {
        const uint32_t base = (cx.vt_sel[u] & (uint32_t)jb) | (~cx.vt_sel[u] & (uint32_t)ja);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            cx.vt_rsrc,
            (__attribute__((address_space(3))) void*)(vdst + wave_off + (u * kWaves - C::kDmaPerTile) * 1024), 16,
            (int)(cx.dma_off[u] + base), 0, 0, 0);
      }
    }
    return;
  }
  const int32_t boff = (te.a & 0x1fff) * C::kTileBytes;
#pragma unroll
  for (int u = 0; u < C::kDmaPerWave; ++u) {
    const int ld = cx.wave + u * kWaves;
    if constexpr (C::kDmaPerTile % kWaves == 0) {
      // K or V is known per copy at compile time, so every copy targets one
      // LDS object and the compiler can tell copies and reads of different
      // ring slots apart
      constexpr int kPerWaveK = C::kDmaPerTile / kWaves;
      if (u < kPerWaveK)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            cx.k_rsrc, (__attribute__((address_space(3))) void*)(kdst + wave_off + u * kWaves * 1024), 16,
            (int)cx.dma_off[u], boff, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            cx.vt_rsrc,
            (__attribute__((address_space(3))) void*)(vdst + wave_off + (u * kWaves - C::kDmaPerTile) * 1024), 16,
            (int)cx.dma_off[u], boff, 0, 0);
    } else {
      if (ld < C::kDmaPerTile)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            cx.k_rsrc, (__attribute__((address_space(3))) void*)(kdst + wave_off + u * kWaves * 1024), 16,
            (int)cx.dma_off[u], boff, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            cx.vt_rsrc,
            (__attribute__((address_space(3))) void*)(vdst + wave_off + (u * kWaves - C::kDmaPerTile) * 1024), 16,
            (int)cx.dma_off[u], boff, 0, 0);
    }
  }
}

// Does this wavefront's query block keep the key block of list entry `ent`?
__device__ __forceinline__ bool keeps(const Ctx& cx, int32_t ent) {
  return ((((uint32_t)ent) >> 24) >> cx.qb) & 1u;
}
// ... any key of the tile (paired mode: either half)?
// (step lists: the wave keeps at most one of a and b; b = 0 keeps nothing)
template <bool PR>
__device__ __forceinline__ bool active(const Ctx& cx, TileEnt te) {
  return keeps(cx, te.a) || keeps(cx, te.b);
}

// V^T A operand of P V job i (step s = i / (D / 32), d tile dt = i % (D / 32);
// consecutive jobs accumulate into different tiles) for lane (d = 32 dt + l32,
// hh): positions 16 s + 8 hh .. + 7 of V^T row d, i.e. keys
// 16 s + 4 hh + {0..3, 8..11}.
template <int D, int BK>
__device__ __forceinline__ bf16x8 v_operand(const Ctx& cx, const char* vt, int i) {
  using C = Cfg<D, BK>;
  const int s = i / (D / 32), dt = i % (D / 32);
  const int row = 32 * dt + cx.l32;
  return *reinterpret_cast<const bf16x8*>(vt + row * C::kVtRowBytes +
                                          (((2 * s + cx.hh) ^ vt_swz<BK>(row)) << 4));
}

// K A operand of S^T job j (step s = j / kSTiles over D, key tile c = j % kSTiles).
template <int D, int BK>
__device__ __forceinline__ bf16x8 k_operand(const Ctx& cx, const char* kt, int j) {
  using C = Cfg<D, BK>;
  const int s = j / C::kSTiles, c = j % C::kSTiles;
  const int row = 32 * c + cx.l32;
  return *reinterpret_cast<const bf16x8*>(kt + row * C::kRowBytes +
                                          (((2 * s + cx.hh) ^ k_swz<D>(row)) << 4));
}

// One stream of MFMA jobs: the P V jobs (if PV) followed by the S^T jobs (if
// QK), with LDS operand reads kWin jobs ahead of their MFMA.  The operands of
// the first kPre P V jobs were read at the end of the previous phase.
template <int D, int BK, bool PV, bool QK, bool PR, int PRE>
__device__ __forceinline__ void mfma_stream(WaveState<D, BK>& st, const Ctx& cx, const char* vprev,
                                            const char* kcur) {
  using C = Cfg<D, BK>;
  constexpr int kNpv = PV ? (D / 32) * C::kPSteps : 0;
  constexpr int kNqk = QK ? (D / 16) * C::kSTiles : 0;
  constexpr int kN = kNpv + kNqk;
  auto rd = [&](int i) {
    return i < kNpv ? v_operand<D, BK>(cx, vprev, i) : k_operand<D, BK>(cx, kcur, i - kNpv);
  };
  // sched_barrier(0) fences keep this source order: the compiler's schedulers
  // would otherwise either issue every read up front (spilling) or move each
  // read next to its MFMA (exposing the LDS latency).
  bf16x8 win[kWin];
#pragma unroll
  for (int i = 0; i < kWin; ++i)
    if (i < kN) win[i] = (PV && i < PRE) ? st.pre[i] : rd(i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kN; ++i) {
    const bf16x8 a = win[i % kWin];
    if (i + kWin < kN) win[i % kWin] = rd(i + kWin);
    // paired mode: a half of the tile the wave does not keep is not skipped
    // on the matrix cores: its scores are masked in the softmax, so its P is
    // zero and its P V MFMAs add nothing, and a branch per MFMA would cost
    // registers that the paired variant does not have
    if (i < kNpv) {
      const int s = i / (D / 32), dt = i % (D / 32);
      st.oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, st.pk[s], st.oacc[dt], 0, 0, 0);
    } else {
      const int j = i - kNpv;
      const int s = j / C::kSTiles, c = j % C::kSTiles;
      const f32x16 acc = s == 0 ? f32x16{} : st.sacc[c];  // S^T starts at 0
      st.sacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, st.qreg[s], acc, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// M phase for key block e: O += P(e-1) V(e-1); S(e) = K(e) Q^T.  The first
// PRE operands of P V were read at the end of the wave's softmax phase.
template <int D, int BK, bool PR, int PRE>
__device__ __forceinline__ void m_phase(WaveState<D, BK>& st, const Ctx& cx, int32_t e,
                                        TileEnt ent_prev, TileEnt ent, const char* vprev,
                                        const char* kcur) {
  using C = Cfg<D, BK>;
  constexpr int kDT = D / 32;
  const bool pv = e >= 1 && e <= cx.n_u && active<PR>(cx, ent_prev);
  const bool qk = e < cx.n_u && active<PR>(cx, ent);
  __builtin_amdgcn_s_setprio(1);
  if (pv && st.o_rescale) {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) st.oacc[dt] = st.oacc[dt] * st.o_alpha;
  }
  if (pv) mfma_stream<D, BK, true, false, PR, PRE>(st, cx, vprev, kcur);
  if (qk) mfma_stream<D, BK, false, true, PR, PRE>(st, cx, vprev, kcur);
  __builtin_amdgcn_s_setprio(0);
}

// V phase for key block e: online softmax of S(e) -> P(e).
template <int D, int BK, bool PR, int PRE>
__device__ __forceinline__ void v_phase(WaveState<D, BK>& st, const Ctx& cx, int32_t e,
                                        TileEnt te, const char* vcur) {
  using C = Cfg<D, BK>;
  if (!(e < cx.n_u && active<PR>(cx, te))) return;
  // lane holds keys kv = 32 c + 8 (r / 4) + 4 hh + (r % 4) of query column l32
  if constexpr (PR) {
    // per 32-key half: its valid keys (the first ones) if the wave keeps it, else none
    const int32_t la = keeps(cx, te.a) ? (te.a >> 13) & 127 : 0;
    const int32_t lb = keeps(cx, te.b) ? (te.b >> 13) & 127 : 0;
    if (la < 32 || lb < 32) {
      int lim0 = la - 4 * cx.hh, lim1 = lb - 4 * cx.hh;
      asm volatile("" : "+v"(lim0), "+v"(lim1));
#pragma unroll
      for (int c = 0; c < C::kSTiles; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kv = 8 * (r >> 2) + (r & 3);  // key index in the half minus 4 hh
          if (kv >= (c ? lim1 : lim0)) st.sacc[c][r] = -INFINITY;
        }
    }
  }
  // valid keys: the first nvalid (step lists: of the entry this wave keeps)
  const int32_t nvalid = PR ? BK : ((keeps(cx, te.b) ? te.b : te.a) >> 13) & 127;
  if (!PR && nvalid < BK) {
    // lane-dependent limit, computed here (an opaque value keeps the 32
    // compares out of loop-invariant code motion, where they would pin 32
    // SGPR-pair lane masks for the whole loop)
    int lim = nvalid - 4 * cx.hh;
    asm volatile("" : "+v"(lim));
#pragma unroll
    for (int c = 0; c < C::kSTiles; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kv = 32 * c + 8 * (r >> 2) + (r & 3);  // key index minus 4 hh
        if (kv >= lim) st.sacc[c][r] = -INFINITY;
      }
  }
  // row max: two chains of 3-input maxima
  float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
  for (int c = 0; c < C::kSTiles; ++c)
#pragma unroll
    for (int r = 0; r < 16; r += 4) {
      m0 = fmaxf(fmaxf(m0, st.sacc[c][r]), st.sacc[c][r + 1]);
      m1 = fmaxf(fmaxf(m1, st.sacc[c][r + 2]), st.sacc[c][r + 3]);
    }
  float mx = fmaxf(m0, m1);
  mx = fmaxf(mx, swap_halves(mx, cx.lane));
  const float mxs = mx * cx.c_log2;
  // lazy rescale: the running max moves only when it grows by > kLazy; O itself
  // is rescaled by o_alpha at the start of the next P V
  const bool need = mxs > st.m_run + kLazy;
  st.o_rescale = __builtin_amdgcn_ballot_w64(need) != 0;
  if (st.o_rescale) {
    const float m_new = need ? mxs : st.m_run;
    st.o_alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
    st.m_run = m_new;
    st.l_run *= st.o_alpha;
  }
  float rs = 0.f;
#pragma unroll
  for (int c = 0; c < C::kSTiles; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(st.sacc[c][r], cx.c_log2, -st.m_run));
      st.sacc[c][r] = p;
      rs += p;
    }
  st.l_run += rs;
  // P^T as the bf16 B operand of step s: keys 16 s + 4 hh + {0..3, 8..11}
#pragma unroll
  for (int s = 0; s < C::kPSteps; ++s)
#pragma unroll
    for (int x = 0; x < 8; ++x) st.pk[s][x] = (__bf16)st.sacc[s >> 1][8 * (s & 1) + x];
  // The next phase of this wave is M(e + 1), whose P V reads V^T(e): where the
  // schedule has V^T(e) complete in LDS by now (PRE > 0), its first operands
  // are read ahead of the barrier.
  if constexpr (PRE > 0) {
#pragma unroll
    for (int i = 0; i < PRE; ++i) st.pre[i] = v_operand<D, BK>(cx, vcur, i);
  }
}

// LDS ring: key block e lives in slot e % 4 (separate LDS objects, so the
// compiler can tell the copies into one slot from the reads of another).
template <int D, int BK>
struct Ring {
  char* k[4];
  char* v[4];
};

// One interval t = t0 + I of group G (t0 is a multiple of 8, so every ring
// slot and every index into ent[] below is a compile-time constant).
//  * even t: every wave issues its copies of key block t / 2 + 2;
//  * phase ph = t - G: even -> M phase of block ph / 2, odd -> V phase;
//  * odd t: wait for this wave's copies of block (t + 1) / 2 before the
//    barrier, so the block is complete when group 0 reads it at t + 1.
// ent[x] is the list data of key tile t0 / 2 - 1 + x (one list entry, or two
// in paired mode).
template <int D, int BK, bool PR, int G, int I>
__device__ __forceinline__ void interval(WaveState<D, BK>& st, const Ctx& cx, const Ring<D, BK>& rg,
                                         int32_t t0, const TileEnt (&ent)[kEnt], int32_t wave_off) {
  using C = Cfg<D, BK>;
  const int32_t t = t0 + I;
  if ((I & 1) == 0) {
    // Past the end of the list this copies the last block again (ent[] is
    // clamped) into a slot that is no longer read: unconditional copies keep
    // the per-wave count of copies in flight fixed.
    constexpr int slot = (I / 2 + 2) & 3;
    issue_copies<D, BK, PR>(cx, ent[I / 2 + 3], rg.k[slot], rg.v[slot], wave_off);
  }
  const int32_t ph = t - G;
  if (ph >= 0 && cx.has_rows) {
    const int32_t e = ph >> 1;
    constexpr int x = ((I - G) >> 1) + 1;  // ent[] index of entry e
    if constexpr (((I - G) & 1) == 0) {
      constexpr int sc = (((I - G) >> 1) + 4) & 3;
      constexpr int sp = (sc + 3) & 3;
      m_phase<D, BK, PR, kPre>(st, cx, e, ent[x - 1], ent[x], rg.v[sp], rg.k[sc]);
    } else {
      constexpr int se = ((I - G) >> 1) & 3;  // ring slot of block e
      v_phase<D, BK, PR, kPre>(st, cx, e, ent[x], rg.v[se]);
    }
  }
  if (I & 1) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(C::kDmaPerWave));
    wg_barrier();
  }
}

template <int D, int BK, bool PR, int G>
__device__ __forceinline__ void run_group(WaveState<D, BK>& st, const Ctx& cx,
                                          const Ring<D, BK>& rg) {
  // The first round (t0 = -8) only issues the copies of key blocks 0 and 1
  // (and, harmlessly, of block 0 into the two other slots): all copies come
  // from this one loop body.
  for (int32_t t0 = -8; t0 < cx.T; t0 += 8) {
    // The list entries of these 8 intervals, loaded (scalar) and waited for
    // up front, so that no scalar load is outstanding while the phases wait
    // on their LDS reads (the shared counter would force full waits).
    TileEnt ent[kEnt];
#pragma unroll
    for (int x = 0; x < kEnt; ++x) {
      const int32_t tile = t0 / 2 - 1 + x;
      if constexpr (PR) {
        const int32_t ia = 2 * tile, ib = 2 * tile + 1;
        ent[x].a = cx.lst[min(max(ia, 0), cx.n_list - 1)];
        const int32_t eb = cx.lst[min(max(ib, 0), cx.n_list - 1)];
        ent[x].b = ib >= 0 && ib < cx.n_list ? eb : eb & 0x00ffffff;  // past the end: kept by none
      } else {
        ent[x].a = cx.lst[min(max(tile, 0), cx.n_u - 1)];
        ent[x].b = 0;
      }
    }
#pragma unroll
    for (int x = 0; x < kEnt; ++x) {
      if constexpr (PR) asm volatile("" : "+s"(ent[x].a), "+s"(ent[x].b));
      else asm volatile("" : "+s"(ent[x].a));
    }
    // LDS offset of this wave's copies, re-materialised every round (kept
    // out of loop-invariant code motion, which would pin one SGPR per copy
    // destination and spill)
    int32_t wave_off = cx.wave * 1024;
    asm volatile("" : "+s"(wave_off));
    interval<D, BK, PR, G, 0>(st, cx, rg, t0, ent, wave_off);
    interval<D, BK, PR, G, 1>(st, cx, rg, t0, ent, wave_off);
    interval<D, BK, PR, G, 2>(st, cx, rg, t0, ent, wave_off);
    interval<D, BK, PR, G, 3>(st, cx, rg, t0, ent, wave_off);
    interval<D, BK, PR, G, 4>(st, cx, rg, t0, ent, wave_off);
    interval<D, BK, PR, G, 5>(st, cx, rg, t0, ent, wave_off);
    interval<D, BK, PR, G, 6>(st, cx, rg, t0, ent, wave_off);
    interval<D, BK, PR, G, 7>(st, cx, rg, t0, ent, wave_off);
  }
}

// ---------------------------------------------------------------------------
// Step schedule (64-token sub-blocks): the list holds steps {a, b} of one or
// two entries with disjoint keep masks (union_kernel), and each wave works on
// the entry its query sub-block keeps.  The ring holds two steps, each with an
// a and a b tile of K and of V^T (8 x 16 KB at D = 128, as the 4-slot ring):
// step s lives in slot s % 2, one LDS object per slot and operand with the b
// tile after the a tile, so a wave picks its tile by an offset and the
// compiler still tells the copies into one slot from the reads of the other
// (a pointer chosen between two objects would make it wait for every copy in
// flight before each read).  Copies run one step ahead: at even interval t
// every wave issues its share of K(t / 2 + 1) and V^T(t / 2) (a tiles, and b
// tiles where the step has a b entry), and before the barrier closing
// interval t + 1 it waits for all of them.  Slot safety: K(s) is read in M(s) (intervals
// 2 s, 2 s + 1), so its slot takes K(s + 2) from interval 2 s + 2 on; V^T(s)
// is read in M(s + 1) (up to 2 s + 3), so its slot takes V^T(s + 2) from 2 s
// + 4 on; both after the barrier closing the last read.
// ---------------------------------------------------------------------------
template <int D, int BK>
struct PairRing {
  char* k[2];   // 2 tiles each: a, then b
  char* v[2];
};

// This wave's copies of the K (PART 0) or V^T (PART 1) tiles of step te into
// slot dst: the a tile, then the b tile when the step has one (the count of
// copies in flight may vary: they are waited for with vmcnt 0).
template <int D, int BK, int PART>
__device__ __forceinline__ void issue_step_copies(const Ctx& cx, TileEnt te, char* slot,
                                                  int32_t wave_off) {
  using C = Cfg<D, BK>;
  char* const da = slot;
  char* const db = slot + C::kTileBytes;
  static_assert(C::kDmaPerTile % kWaves == 0, "copies of a tile split evenly over the waves");
  constexpr int kPer = C::kDmaPerTile / kWaves;  // copies per wave per tile
  const __amdgpu_buffer_rsrc_t rs = PART == 0 ? cx.k_rsrc : cx.vt_rsrc;
  const int32_t oa = (te.a & 0x1fff) * C::kTileBytes;
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(da + wave_off + u * kWaves * 1024), 16,
        (int)cx.dma_off[PART * kPer + u], oa, 0, 0);
  if (te.b != 0) {  // wave-uniform
    const int32_t ob = (te.b & 0x1fff) * C::kTileBytes;
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(db + wave_off + u * kWaves * 1024), 16,
          (int)cx.dma_off[PART * kPer + u], ob, 0, 0);
  }
}

// One interval t = t0 + I of group G in the step schedule (t0 a multiple of
// 8, so every slot and ent[] index is a compile-time constant; ent[x] is step
// t0 / 2 - 1 + x).
template <int D, int BK, int G, int I>
__device__ __forceinline__ void interval_step(WaveState<D, BK>& st, const Ctx& cx,
                                              const PairRing<D, BK>& rg, int32_t t0,
                                              const TileEnt (&ent)[kEnt], int32_t wave_off) {
  const int32_t t = t0 + I;
  if ((I & 1) == 0) {
    constexpr int sk = (I / 2 + 1) & 1, sv = (I / 2) & 1;
    issue_step_copies<D, BK, 0>(cx, ent[I / 2 + 2], rg.k[sk], wave_off);
    issue_step_copies<D, BK, 1>(cx, ent[I / 2 + 1], rg.v[sv], wave_off);
  }
  const int32_t ph = t - G;
  if (ph >= 0 && cx.has_rows) {
    const int32_t e = ph >> 1;
    constexpr int x = ((I - G) >> 1) + 1;  // ent[] index of step e
    if constexpr (((I - G) & 1) == 0) {
      constexpr int sc = ((I - G) >> 1) & 1;  // slot of step e; e - 1 in the other
      const TileEnt ep = ent[x - 1], ec = ent[x];
      constexpr int32_t kTB = Cfg<D, BK>::kTileBytes;
      const char* vprev = rg.v[sc ^ 1] + (keeps(cx, ep.b) ? kTB : 0);
      const char* kcur = rg.k[sc] + (keeps(cx, ec.b) ? kTB : 0);
      m_phase<D, BK, false, G == 1 ? kPre : 0>(st, cx, e, ep, ec, vprev, kcur);
    } else {
      // Group 1's softmax of step e runs in interval 2 e + 2, after the
      // barrier that completed V^T(e) (copied in 2 e): it reads the first
      // operands of its next P V ahead.  Group 0's runs in 2 e + 1, while
      // that copy may still be in flight.
      constexpr int se = ((I - G) >> 1) & 1;  // slot of step e
      const char* vcur = rg.v[se] + (keeps(cx, ent[x].b) ? Cfg<D, BK>::kTileBytes : 0);
      v_phase<D, BK, false, G == 1 ? kPre : 0>(st, cx, e, ent[x], vcur);
    }
  }
  if (I & 1) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    wg_barrier();
  }
}

template <int D, int BK, int G>
__device__ __forceinline__ void run_group_steps(WaveState<D, BK>& st, const Ctx& cx,
                                                const PairRing<D, BK>& rg) {
  // The first round (t0 = -8) only issues copies (of step 0 where the index
  // is negative); its last even interval brings K(0).
  for (int32_t t0 = -8; t0 < cx.T; t0 += 8) {
    TileEnt ent[kEnt];   // the step schedule uses ent[0 .. 5]
#pragma unroll
    for (int x = 0; x < kEnt; ++x) {
      if (x > 5) {
        ent[x] = ent[5];
        continue;
      }
      const int32_t step = min(max(t0 / 2 - 1 + x, 0), cx.n_u - 1);
      ent[x].a = cx.lst[2 * step];
      ent[x].b = cx.lst[2 * step + 1];
    }
#pragma unroll
    for (int x = 0; x < 6; ++x) asm volatile("" : "+s"(ent[x].a), "+s"(ent[x].b));
    int32_t wave_off = cx.wave * 1024;
    asm volatile("" : "+s"(wave_off));
    interval_step<D, BK, G, 0>(st, cx, rg, t0, ent, wave_off);
    interval_step<D, BK, G, 1>(st, cx, rg, t0, ent, wave_off);
    interval_step<D, BK, G, 2>(st, cx, rg, t0, ent, wave_off);
    interval_step<D, BK, G, 3>(st, cx, rg, t0, ent, wave_off);
    interval_step<D, BK, G, 4>(st, cx, rg, t0, ent, wave_off);
    interval_step<D, BK, G, 5>(st, cx, rg, t0, ent, wave_off);
    interval_step<D, BK, G, 6>(st, cx, rg, t0, ent, wave_off);
    interval_step<D, BK, G, 7>(st, cx, rg, t0, ent, wave_off);
  }
}

// Ping-pong schedule.  The 8 wavefronts form two groups (waves 0-3 and 4-7;
// each SIMD holds one wave of each).  Per key block e a wave runs an MFMA
// phase M(e) = { O += P(e-1) V(e-1) ; S(e) = K(e) Q^T } and a VALU phase
// V(e) = { online softmax of S(e) -> P(e) }.  Group 1 runs one phase behind
// group 0 and phases are separated by workgroup barriers, so in every
// interval one wave per SIMD issues matrix work while the other issues the
// softmax.  Key block e is copied HBM -> LDS at interval 2e - 4, two key
// blocks ahead of its first use, and is read during intervals 2e .. 2e+3.
// One work item: query group gi of head bh, whose union list is list[item].
template <int D, int BK, bool PR, bool STEPS, typename RingT>
__device__ __forceinline__ void run_item(const __bf16* __restrict__ q,
                                         const __bf16* __restrict__ k,
                                         const __bf16* __restrict__ vt, __bf16* __restrict__ out,
                                         const int32_t* __restrict__ list,
                                         const int32_t* __restrict__ count, int64_t item,
                                         int32_t groups, int32_t nb, int32_t nq,
                                         int32_t npad_q, int32_t npad_k, float c_log2,
                                         const OutMap& om, const int32_t* __restrict__ perm,
                                         const RingT& rg) {
  using C = Cfg<D, BK>;
  constexpr int kS = D / 16, kDT = D / 32;

  const int tid = threadIdx.x;
  Ctx cx;
  cx.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  cx.lane = tid & 63;
  const int grp = cx.wave >> 2;                             // ping-pong group
  // query block inside the item (paired mode: one 32-row block per wave) and
  // the wave's 32-row slice inside it
  constexpr bool kSplitBlock = !PR;
  cx.qb = kSplitBlock ? (cx.wave & 3) : cx.wave;
  const int sub = kSplitBlock ? grp : 0;
  constexpr int kQRows = kSplitBlock ? 64 : 32;             // rows of one query block
  constexpr int kQGroup = kRowsPerItem / kQRows;            // query blocks per item
  cx.l32 = cx.lane & 31;
  cx.hh = cx.lane >> 5;

  const int64_t bh = item / groups;
  const int32_t gi = (int32_t)(item % groups);
  // the wave's query block: consecutive in the group, or as regrouped by
  // group_kernel (-1: an empty slot of the head's last group)
  const int32_t iq = perm ? perm[item * kQGroup + cx.qb] : gi * kQGroup + cx.qb;
  cx.has_rows = iq >= 0 && iq < nq;
  cx.n_list = count[item];
  cx.n_u = PR ? (cx.n_list + 1) / 2 : cx.n_list;            // key tiles streamed
  // intervals 0 .. 2 n_u + 1 carry work; the count is rounded up to whole
  // rounds of 8 (the extra intervals do nothing)
  cx.T = (2 * cx.n_u + 2 + 7) & ~7;
  cx.nb = nb;
  cx.c_log2 = c_log2;
  cx.lst = list + item * (STEPS ? 2 * nb : nb);   // entries, or steps of two words
  // raw buffer resources over this head's K and V^T (byte range npad_k * D * 2,
  // below 2^31 by the host checks; dword 3 = 0x00020000: raw 32-bit data)
  const int32_t head_bytes = npad_k * D * 2;
  cx.k_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(k + bh * (int64_t)npad_k * D), (short)0,
                                                head_bytes, 0x00020000);
  cx.vt_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(vt + bh * (int64_t)npad_k * D),
                                                 (short)0, head_bytes, 0x00020000);
  const __bf16* qh = q + bh * (int64_t)npad_q * D;
  __bf16* oh = out + bh * (int64_t)npad_q * D;

#pragma unroll
  for (int u = 0; u < C::kDmaPerWave; ++u) {
    cx.dma_off[u] = copy_src_off<D, BK>(cx.wave, cx.lane, u);
    cx.vt_sel[u] = 0u;
    if constexpr (PR) {
      // paired mode: the source of each 32-key half is its own list entry's
      // block of 32 keys (K: 32 rows of 2 D bytes; V^T: D rows of 64 bytes)
      constexpr int32_t kHalfBytes = 32 * D * 2;
      const int ld = cx.wave + u * kWaves;
      if (ld < C::kDmaPerTile) {
        if (ld * 1024 >= kHalfBytes) cx.dma_off[u] -= kHalfBytes;   // rows 32..63: entry b
      } else {
        const int byte = (ld - C::kDmaPerTile) * 1024 + cx.lane * 16;
        const int row = byte / C::kVtRowBytes;
        const int lc = ((byte % C::kVtRowBytes) >> 4) ^ vt_swz<BK>(row);  // source chunk 0..7
        cx.dma_off[u] = (uint32_t)(row * 64 + (lc & 3) * 16);
        cx.vt_sel[u] = lc >= 4 ? ~0u : 0u;
      }
    }
  }

  WaveState<D, BK> st;
  const int32_t qrow = (cx.has_rows ? iq : nq - 1) * kQRows + sub * 32 + cx.l32;
#pragma unroll
  for (int s = 0; s < kS; ++s)
    st.qreg[s] = *reinterpret_cast<const bf16x8*>(qh + (int64_t)qrow * D + 16 * s + 8 * cx.hh);
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.oacc[dt][r] = 0.f;
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  st.o_alpha = 1.f;
  st.o_rescale = false;
  // Q operands are in place before the loop
#pragma unroll
  for (int s = 0; s < kS; ++s) asm volatile("" ::"v"(st.qreg[s]));
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  wg_barrier();

  // An item whose union list is empty (every row of its group is empty, or
  // the group holds padding only) streams nothing: its output rows are zeros.
  // The count is uniform over the workgroup, so every wave skips the loop and
  // its barriers together; the loop's list reads need n_list >= 1.
  if (cx.n_u > 0) {
    if constexpr (STEPS) {
      if (grp == 0) run_group_steps<D, BK, 0>(st, cx, rg);
      else run_group_steps<D, BK, 1>(st, cx, rg);
    } else {
      if (grp == 0) run_group<D, BK, PR, 0>(st, cx, rg);
      else run_group<D, BK, PR, 1>(st, cx, rg);
    }
  }

  if (!cx.has_rows) return;
  const float l_tot = st.l_run + swap_halves(st.l_run, cx.lane);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  __bf16* orow = oh + (int64_t)qrow * D;
  if (om.natural) {  // natural (t, h, w) order; padding slots have no row there
    const int32_t blk = qrow / om.g.Bk, slot = qrow - blk * om.g.Bk;
    if (blk >= om.g.nb || slot >= block_valid(om.g, blk)) return;
    orow = out + (bh * (int64_t)om.g.N + natural_row(om.g, blk, slot)) * D;
  }
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = 32 * dt + 8 * rq + 4 * cx.hh;
      bf16x4 o;
#pragma unroll
      for (int x = 0; x < 4; ++x) o[x] = (__bf16)(st.oacc[dt][4 * rq + x] * inv);
      *reinterpret_cast<bf16x4*>(orow + d0) = o;
    }
}

// Persistent kernel: one workgroup per CU slot takes items from the queue of
// the XCD it runs on (hardware register XCC_ID), then from the other queues;
// it exits once every queue is drained.
template <int D, int BK, bool PR, bool STEPS>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
            const __bf16* __restrict__ vt, __bf16* __restrict__ out,
            const int32_t* __restrict__ list, const int32_t* __restrict__ count,
            const int32_t* __restrict__ queue, int32_t* __restrict__ meta, int32_t groups,
            int32_t nb, int32_t nq, int32_t npad_q, int32_t npad_k, float c_log2, OutMap om,
            const int32_t* __restrict__ perm) {
  using C = Cfg<D, BK>;
  __shared__ int32_t s_item;
  const int home = __builtin_amdgcn_s_getreg((3 << 11) | 20) & (kQueues - 1);  // XCC_ID
  int probe = 0;  // thread 0: queues home, home + 1, ... found empty so far
  // thread 0 takes the next item (-1: every queue drained), broadcast via LDS
  auto next_item = [&]() {
    if (threadIdx.x == 0) {
      int32_t it = -1;
      while (probe < kQueues) {
        const int x = (home + probe) & (kQueues - 1);
        const int32_t pos = atomicAdd(&meta[2 * kQueues + x], 1);
        if (pos < meta[kQueues + x]) {
          it = queue[meta[x] + pos];
          break;
        }
        ++probe;
      }
      s_item = it;
    }
    __syncthreads();
    const int32_t item = s_item;
    __syncthreads();
    return item;
  };
  if constexpr (!STEPS) {
    // entries (paired 32-key tiles or 64-key blocks): 4-slot ring, one object per tile
    __shared__ __attribute__((aligned(1024))) char k0[C::kTileBytes], k1[C::kTileBytes],
        k2[C::kTileBytes], k3[C::kTileBytes];
    __shared__ __attribute__((aligned(1024))) char v0[C::kTileBytes], v1[C::kTileBytes],
        v2[C::kTileBytes], v3[C::kTileBytes];
    const Ring<D, BK> rg{{k0, k1, k2, k3}, {v0, v1, v2, v3}};
    for (int32_t item = next_item(); item >= 0; item = next_item())
      run_item<D, BK, PR, STEPS>(q, k, vt, out, list, count, item, groups, nb, nq, npad_q, npad_k,
                          c_log2, om, perm, rg);
  } else {
    static_assert(!PR, "step lists hold 64-key entries");
    // steps: 2-step ring, one object per slot holding the a and b tiles
    __shared__ __attribute__((aligned(1024))) char k0[2 * C::kTileBytes], k1[2 * C::kTileBytes];
    __shared__ __attribute__((aligned(1024))) char v0[2 * C::kTileBytes], v1[2 * C::kTileBytes];
    const PairRing<D, BK> rg{{k0, k1}, {v0, v1}};
    for (int32_t item = next_item(); item >= 0; item = next_item())
      run_item<D, BK, PR, STEPS>(q, k, vt, out, list, count, item, groups, nb, nq, npad_q, npad_k,
                          c_log2, om, perm, rg);
  }
}

// Workgroups of the persistent attention kernel: every CU slot of the current
// device (CU count x resident workgroups per CU), at most one per item.  Both
// figures are queried on every call: the library keeps no state between calls.
template <int D, int BK, bool PR, bool STEPS>
hipError_t attn_grid(int64_t items, uint32_t* grid) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_kernel<D, BK, PR, STEPS>, kThreads,
                                                   0);
  if (e != hipSuccess) return e;
  int64_t slots = (int64_t)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
  *grid = (uint32_t)(items < slots ? items : slots);
  return hipSuccess;
}

// nb / nq: key / query sub-blocks per head (nb is also the list stride);
// npad_q / npad_k: rows per head of Q and O / of K and V.
// PR: paired mode (32-key schedule entries streamed two per 64-key tile; V^T
// is laid out per 32-key sub-block)
template <int D, int BK, bool PR, bool STEPS>
hipError_t launch_attn(const void* q, const void* k, const void* v, void* out, const int32_t* list,
                       const int32_t* count, const int32_t* queue, int32_t* meta, __bf16* vt,
                       int32_t bh, const AttnWs& w, int32_t nb, int32_t nq, int32_t npad_q,
                       int32_t npad_k, float c_log2, const OutMap& om, const int32_t* perm,
                       hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (v) {  // else V^T is already in the workspace (launch_attn_stage_v)
    hipLaunchKernelGGL((vt_kernel<D, PR ? 32 : BK>), dim3((uint32_t)((int64_t)bh * nb)),
                       dim3(kVtThreads), 0, stream, (const __bf16*)v, vt, nb, npad_k);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  uint32_t grid = 0;
  e = attn_grid<D, BK, PR, STEPS>(w.items, &grid);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_kernel<D, BK, PR, STEPS>), dim3(grid), dim3(kThreads), 0, stream,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)vt, (__bf16*)out, list,
                     count, queue, meta, w.groups, nb, nq, npad_q, npad_k, c_log2, om, perm);
  return hipGetLastError();
}

}  // namespace

namespace {
AttnWs ws_common(int32_t bh, int32_t sub, int32_t nbs_q, int32_t nbs_k, int64_t npad_k,
                 bool groupable) {
  AttnWs w{};
  w.groupable = groupable;
  w.sub = sub;
  w.nbs = nbs_k;
  w.nbs_q = nbs_q;
  w.group_size = kRowsPerItem / w.sub;
  w.groups = (nbs_q + w.group_size - 1) / w.group_size;
  w.items = (int64_t)bh * w.groups;
  size_t off = 0;
  w.list_off = off;   // per item: nbs entries, or nbs steps of two words
  off = align_up(off + (size_t)w.items * w.nbs * 2 * sizeof(int32_t), 256);
  w.count_off = off;
  off = align_up(off + (size_t)w.items * sizeof(int32_t), 256);
  w.queue_off = off;
  off = align_up(off + (size_t)w.items * sizeof(int32_t), 256);
  w.meta_off = off;
  off = align_up(off + 3 * kQueues * sizeof(int32_t), 256);
  w.vt_off = off;
  off = align_up(off + (size_t)bh * npad_k * kMaxHeadDim * 2, 256);  // V^T (bf16)
  w.perm_off = off;
  if (groupable) off = align_up(off + (size_t)w.items * w.group_size * sizeof(int32_t), 256);
  w.total = off;
  return w;
}

// union lists, work queues, then the kernels for this head_dim / sub-block size
template <typename Sched>
hipError_t run_attention(const void* q, const void* k, const void* v, void* out, int32_t bh,
                         int32_t head_dim, const AttnWs& w, const Sched& sc, int32_t npad_q,
                         int32_t npad_k, float scale, const int32_t* row_ptr,
                         const int32_t* col_idx, void* ws, const OutMap& om, int regroup,
                         bool steps, hipStream_t stream) {
  if (w.items > 0x7fffffff) return hipErrorInvalidValue;
  char* base = static_cast<char*>(ws);
  int32_t* list = reinterpret_cast<int32_t*>(base + w.list_off);
  int32_t* count = reinterpret_cast<int32_t*>(base + w.count_off);
  int32_t* queue = reinterpret_cast<int32_t*>(base + w.queue_off);
  int32_t* meta = reinterpret_cast<int32_t*>(base + w.meta_off);
  __bf16* vt = reinterpret_cast<__bf16*>(base + w.vt_off);
  int32_t* perm = nullptr;
  hipError_t e = hipSuccess;
  // regroup: 0 never, 2 always (when groupable), 1 when the work is large
  // enough to pay for the search (~0.3 ms, against ~1.5% of the attention
  // time): batch * heads * nb^2 * head_dim >= 2^32 (Wan-720p: 1.7 * 2^32)
  const bool big = (double)bh * w.nbs * w.nbs * head_dim >= 4294967296.0;
  if (w.groupable && (regroup == 2 || (regroup == 1 && big))) {
    perm = reinterpret_cast<int32_t*>(base + w.perm_off);
    const int32_t windows = (w.nbs_q + kGWin - 1) / kGWin;
    const dim3 ggrid((uint32_t)((int64_t)bh * windows)), gblk(kGWin);
    if (w.nbs <= 512)
      hipLaunchKernelGGL((group_kernel<16, kGWin>), ggrid, gblk, 0, stream, row_ptr, col_idx, perm,
                         w.nbs_q, w.groups, windows);
    else if (w.nbs <= 1024)
      hipLaunchKernelGGL((group_kernel<32, kGWin>), ggrid, gblk, 0, stream, row_ptr, col_idx, perm,
                         w.nbs_q, w.groups, windows);
    else if (w.nbs <= 1536)
      hipLaunchKernelGGL((group_kernel<48, kGWin>), ggrid, gblk, 0, stream, row_ptr, col_idx, perm,
                         w.nbs_q, w.groups, windows);
    else
      hipLaunchKernelGGL((group_kernel<64, kGWin>), ggrid, gblk, 0, stream, row_ptr, col_idx, perm,
                         w.nbs_q, w.groups, windows);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  // step lists: 64-token sub-blocks and a staging that fits in LDS; otherwise
  // the entry walk (one word per entry)
  steps = steps && w.sub == 64 && w.nbs <= kPairMaxNb;
  const int32_t out_mode = steps ? 2 : 0;
  const dim3 ugrid((uint32_t)w.items), ublk(kSchedThreads);
  const size_t ushm = (size_t)w.nbs * sizeof(uint32_t) * (out_mode == 2 ? 3 : 1);
  if (out_mode == 2)
    hipLaunchKernelGGL((union_kernel<Sched, 2>), ugrid, ublk, ushm, stream, row_ptr, col_idx, list,
                       count, w.nbs, w.nbs_q, w.groups, w.group_size, sc, (const int32_t*)perm);
  else
    hipLaunchKernelGGL((union_kernel<Sched, 0>), ugrid, ublk, ushm, stream, row_ptr, col_idx, list,
                       count, w.nbs, w.nbs_q, w.groups, w.group_size, sc, (const int32_t*)perm);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // fewer runs per head when there are many heads, so that every unit is still
  // placed by its work (kQueueMaxBh units at most)
  const int32_t parts = (int32_t)std::max<int64_t>(1, std::min<int64_t>(kHeadParts, kQueueMaxBh / bh));
  hipLaunchKernelGGL(queue_kernel, dim3(1), dim3(kQueueThreads), 0, stream, count, queue, meta, bh,
                     w.groups, parts);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const float c_log2 = scale * 1.4426950408889634f;
#define SVSA_LAUNCH(DD, PR, ST)                                                                  \
  return launch_attn<DD, 64, PR, ST>(q, k, v, out, list, count, queue, meta, vt, bh, w, w.nbs,  \
                                     w.nbs_q, npad_q, npad_k, c_log2, om, perm, stream)
  if (w.sub == 64) {
    if (head_dim == 128) {
      if (steps) SVSA_LAUNCH(128, false, true);
      SVSA_LAUNCH(128, false, false);
    }
    if (steps) SVSA_LAUNCH(64, false, true);
    SVSA_LAUNCH(64, false, false);
  }
  if (head_dim == 128) SVSA_LAUNCH(128, true, false);
  SVSA_LAUNCH(64, true, false);
#undef SVSA_LAUNCH
}
}  // namespace

AttnWs attn_ws_layout(int32_t bh, const Geom& g) {
  const int32_t sub = g.Bk % 64 == 0 ? 64 : 32;
  const int32_t ratio = g.Bk / sub;
  const int32_t nbs = g.pad3d ? g.nb * ratio : (g.N + sub - 1) / sub;
  // query blocks can be regrouped when a block is one 64-token sub-block and
  // a list fits group_kernel's bitmaps (2048 blocks)
  const bool groupable = sub == 64 && ratio == 1 && nbs <= 2048;
  AttnWs w = ws_common(bh, sub, nbs, nbs, g.Npad, groupable);
  w.ratio = ratio;
  return w;
}

AttnWs cluster_attn_ws_layout(int32_t bh, int32_t sub, int64_t npad_q, int64_t npad_k) {
  AttnWs w = ws_common(bh, sub, (int32_t)(npad_q / sub), (int32_t)(npad_k / sub), npad_k, false);
  w.ratio = 1;
  return w;
}

hipError_t launch_block_sparse_attn(const void* q, const void* k, const void* v, void* out,
                                    int32_t bh, int32_t head_dim, const Geom& g, float scale,
                                    const int32_t* row_ptr, const int32_t* col_idx, void* ws,
                                    bool natural_out, int regroup, bool steps,
                                    hipStream_t stream) {
  if (g.Bk % 32 != 0) return hipErrorInvalidValue;
  if (head_dim != 64 && head_dim != 128) return hipErrorInvalidValue;
  const AttnWs w = attn_ws_layout(bh, g);
  const GeomSched sc{g, w.ratio, w.sub};
  const OutMap om{g, natural_out ? 1 : 0};
  return run_attention(q, k, v, out, bh, head_dim, w, sc, g.Npad, g.Npad, scale, row_ptr, col_idx,
                       ws, om, regroup, steps, stream);
}

hipError_t launch_attn_stage_v(const void* v, int32_t bh, int32_t head_dim, const Geom& g,
                               void* ws, hipStream_t stream) {
  if (g.Bk % 32 != 0) return hipErrorInvalidValue;
  if (head_dim != 64 && head_dim != 128) return hipErrorInvalidValue;
  const AttnWs w = attn_ws_layout(bh, g);
  const int64_t blocks = (int64_t)bh * w.nbs;
  if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
  __bf16* vt = reinterpret_cast<__bf16*>(static_cast<char*>(ws) + w.vt_off);
  const dim3 grid((uint32_t)blocks), blk(kVtThreads);
  // the sub-block size and V^T layout that launch_block_sparse_attn's kernels read
  if (head_dim == 128 && w.sub == 64)
    hipLaunchKernelGGL((stage_v_kernel<128, 64>), grid, blk, 0, stream, (const __bf16*)v, vt, w.nbs, g);
  else if (head_dim == 64 && w.sub == 64)
    hipLaunchKernelGGL((stage_v_kernel<64, 64>), grid, blk, 0, stream, (const __bf16*)v, vt, w.nbs, g);
  else if (head_dim == 128)
    hipLaunchKernelGGL((stage_v_kernel<128, 32>), grid, blk, 0, stream, (const __bf16*)v, vt, w.nbs, g);
  else
    hipLaunchKernelGGL((stage_v_kernel<64, 32>), grid, blk, 0, stream, (const __bf16*)v, vt, w.nbs, g);
  return hipGetLastError();
}

hipError_t launch_cluster_attn(const void* q, const void* k, const void* v, void* out,
                               int32_t bh, int32_t head_dim, int32_t sub, int64_t npad_q,
                               int64_t npad_k, const int32_t* q_start, const int32_t* q_size,
                               int32_t nq, const int32_t* k_start, const int32_t* k_size,
                               int32_t nk, float scale, const int32_t* row_ptr,
                               const int32_t* col_idx, void* ws, hipStream_t stream) {
  if ((sub != 32 && sub != 64) || npad_q % sub || npad_k % sub) return hipErrorInvalidValue;
  if (head_dim != 64 && head_dim != 128) return hipErrorInvalidValue;
  const AttnWs w = cluster_attn_ws_layout(bh, sub, npad_q, npad_k);
  const TableSched sc{q_start, q_size, k_start, k_size, nq, nk, sub};
  const OutMap om{};  // tile (cluster) order
  return run_attention(q, k, v, out, bh, head_dim, w, sc, (int32_t)npad_q, (int32_t)npad_k, scale,
                       row_ptr, col_idx, ws, om, 0, false, stream);
}

}  // namespace svsa
