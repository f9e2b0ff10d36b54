// Internal declarations shared by the library's translation units (host side).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svsa {

// Derived geometry of one call.
struct Geom {
  int32_t T, H, W, tt, th, tw;
  int32_t nT, nH, nW;   // tile grid
  int32_t N, Bk, nb, Npad;
  int32_t pad3d;        // 1: one block per tile (padding inside the sequence)
};

// Valid tokens of block b (the block's first slots).
__host__ __device__ inline int32_t block_valid(const Geom& g, int32_t b) {
  if (!g.pad3d) {
    const int32_t r = g.N - b * g.Bk;
    return r < g.Bk ? r : g.Bk;
  }
  const int32_t a = b / (g.nH * g.nW), c_h = (b / g.nW) % g.nH, c_w = b % g.nW;
  const int32_t sa = g.T - a * g.tt < g.tt ? g.T - a * g.tt : g.tt;
  const int32_t sb = g.H - c_h * g.th < g.th ? g.H - c_h * g.th : g.th;
  const int32_t sc = g.W - c_w * g.tw < g.tw ? g.W - c_w * g.tw : g.tw;
  return sa * sb * sc;
}

// Natural row (t*H*W + h*W + w) of slot `slot` of block `blk` in the tiled
// sequence; the slot must be valid (slot < block_valid(g, blk)).  It inverts
// the tile walk: the slab of tile rows along t (every earlier slab is full),
// then the row of tiles along h inside it (every earlier row is full), then
// the tile along w, then (t, h, w) inside the tile; in the 3D-padded layout
// the block is the tile.
__device__ inline int32_t natural_row(const Geom& g, int32_t blk, int32_t slot) {
  int32_t a, b, c, o;
  if (g.pad3d) {
    a = blk / (g.nH * g.nW);
    b = (blk / g.nW) % g.nH;
    c = blk % g.nW;
    o = slot;
  } else {
    const int32_t p = blk * g.Bk + slot;
    const int32_t slab = g.tt * g.H * g.W;
    a = p / slab;
    int32_t r = p - a * slab;
    const int32_t sa = min(g.tt, g.T - a * g.tt);
    const int32_t row = sa * g.th * g.W;
    b = r / row;
    r -= b * row;
    const int32_t tsz = sa * min(g.th, g.H - b * g.th) * g.tw;
    c = r / tsz;
    o = r - c * tsz;
  }
  const int32_t sb = min(g.th, g.H - b * g.th);
  const int32_t sc = min(g.tw, g.W - c * g.tw);
  const int32_t lt = o / (sb * sc);
  const int32_t rem = o - lt * sb * sc;
  const int32_t lh = rem / sc;
  const int32_t lw = rem - lh * sc;
  return ((a * g.tt + lt) * g.H + b * g.th + lh) * g.W + c * g.tw + lw;
}

// Launchers: enqueue on `stream`, return the launch status.
hipError_t launch_tile_permute(const void* src, void* dst, int elt_bytes, int32_t bh,
                               int32_t head_dim, const Geom& g, bool inverse,
                               hipStream_t stream);
// V^T for the attention kernel straight from natural-order V (into the
// attention workspace laid out by attn_ws_layout).
hipError_t launch_attn_stage_v(const void* v, int32_t bh, int32_t head_dim, const Geom& g,
                               void* ws, hipStream_t stream);
hipError_t launch_tile_permute_pool(const void* src, void* dst, double* means, bool is_bf16,
                                    int32_t bh, int32_t head_dim, const Geom& g,
                                    hipStream_t stream);
hipError_t launch_pool(const void* x, bool is_bf16, double* out, int32_t bh,
                       int32_t head_dim, const Geom& g, hipStream_t stream);

// Block-mask workspace layout (all offsets 256-byte aligned).
struct MaskWs {
  size_t logits_off, bits_off, counts_off, total;
  int32_t words;  // bitmap words per row
};
MaskWs mask_ws_layout(int64_t rows, int32_t nb);
hipError_t launch_block_mask(const double* qbar, const double* kbar, int32_t bh, int32_t heads,
                             int32_t nb, int32_t head_dim, double scale, const float* top_p,
                             const float* keep_frac, int32_t band, int32_t* row_ptr,
                             int32_t* col_idx, void* ws, hipStream_t stream);

// The block mask with its scratch in a file-scope device array (no workspace
// argument): whether the sizes fit, and the launch.
bool block_mask_fits_scratch(int64_t bh, int32_t nb);
hipError_t launch_block_mask_noalloc(const double* qbar, const double* kbar, int32_t bh,
                                     int32_t heads, int32_t nb, int32_t head_dim, double scale,
                                     const float* top_p, const float* keep_frac, int32_t band,
                                     int32_t* row_ptr, int32_t* col_idx, hipStream_t stream);

// Rectangular variant: nq query rows per head against nb key clusters, with
// + ln n_j on every logit of key cluster j when ksizes is given.
hipError_t launch_cluster_mask(const double* qbar, const double* kbar, const int32_t* ksizes,
                               int32_t bh, int32_t heads, int32_t nq, int32_t nb,
                               int32_t head_dim, double scale, const float* top_p,
                               const float* keep_frac, int32_t band, int32_t* row_ptr,
                               int32_t* col_idx, void* ws, hipStream_t stream);

// Row bitmaps (words uint32 per row) + row counts -> CSR (row_ptr, col_idx).
hipError_t launch_csr_from_bits(const uint32_t* bits, const int32_t* counts, int32_t* row_ptr,
                                int32_t* col_idx, int64_t rows, int32_t words,
                                hipStream_t stream);

// Stripe-mask workspace layout and launcher.
constexpr int kStripeMaxHeads = 128;
struct StripeWs {
  size_t tiles_off, ntiles_off, bits_off, counts_off, total;
  int32_t words;
};
StripeWs stripe_ws_layout(int64_t rows, const Geom& g);
hipError_t launch_stripe_mask(const Geom& g, int32_t bh, int32_t heads, const int32_t* params,
                              int32_t band, int32_t* row_ptr, int32_t* col_idx, void* ws,
                              hipStream_t stream);

// Attention workspace layout.
struct AttnWs {
  size_t list_off, count_off, queue_off, meta_off, vt_off, perm_off, total;
  bool groupable;      // query blocks may be regrouped by list (perm_off holds the groups)
  int64_t items;
  int32_t groups;      // query sub-block groups per (b, h)
  int32_t group_size;  // query sub-blocks per group (256 query rows per group)
  int32_t sub;         // sub-block size seen by the attention kernels (64 or 32)
  int32_t ratio;       // sub-blocks per block (Bk / sub)
  int32_t nbs;         // key sub-blocks per head (also the list stride)
  int32_t nbs_q;       // query sub-blocks per head
};
AttnWs attn_ws_layout(int32_t bh, const Geom& g);
AttnWs cluster_attn_ws_layout(int32_t bh, int32_t sub, int64_t npad_q, int64_t npad_k);
hipError_t launch_cluster_attn(const void* q, const void* k, const void* v, void* out,
                               int32_t bh, int32_t head_dim, int32_t sub, int64_t npad_q,
                               int64_t npad_k, const int32_t* q_start, const int32_t* q_size,
                               int32_t nq, const int32_t* k_start, const int32_t* k_size,
                               int32_t nk, float scale, const int32_t* row_ptr,
                               const int32_t* col_idx, void* ws, hipStream_t stream);
hipError_t launch_block_sparse_attn(const void* q, const void* k, const void* v, void* out,
                                    int32_t bh, int32_t head_dim, const Geom& g, float scale,
                                    const int32_t* row_ptr, const int32_t* col_idx, void* ws,
                                    bool natural_out, int regroup, bool steps,
                                    hipStream_t stream);

// Clustering (variable-size blocks).
int64_t cluster_lcap(int32_t N, int32_t C, int32_t align);   // padded layout capacity
struct KmeansWs {
  size_t g_hi_off, g_lo_off, cq_off, start_off, token_off, layout_off, total;
};
size_t layout_ws_bytes(int32_t bh, int32_t N, int32_t C);   // svsa_cluster_layout scratch
KmeansWs kmeans_ws_layout(int32_t bh, int32_t N, int32_t C, int32_t D);
hipError_t launch_kmeans(const void* x, int32_t bh, int32_t N, int32_t D, const double* G,
                         double* cents, int32_t C, int32_t iters, int32_t* labels,
                         int32_t* sizes, void* ws, hipStream_t stream);
hipError_t launch_cluster_metric(const double* cents, const int32_t* sizes, double* G, int32_t bh,
                                 int32_t C, int32_t D, hipStream_t stream);
hipError_t launch_cluster_layout(const int32_t* labels, int32_t bh, int32_t N, int32_t C,
                                 int32_t align, int32_t* start, int32_t* sizes, int32_t* slot,
                                 int32_t* token, void* ws, hipStream_t stream);
hipError_t launch_cluster_means(const void* x, const int32_t* start, const int32_t* sizes,
                                const int32_t* token, double* cents, int32_t bh, int32_t N,
                                int32_t C, int32_t D, int64_t lcap, hipStream_t stream);
hipError_t launch_cluster_permute(const void* src, void* dst, int elt_bytes, int32_t bh,
                                  int32_t N, int32_t D, int32_t C, int64_t lcap,
                                  const int32_t* map, const int32_t* start, bool inverse,
                                  hipStream_t stream);

struct TailWs {
  size_t bits_off, rep_off, move_off, cut_off, counts_off, start_off, sizes_off, slot_off,
      token_off, layout_off, total;
  int32_t words;
};
TailWs tail_ws_layout(int32_t bh, int32_t N, int32_t C, int32_t nk);
hipError_t launch_tail_merge(int32_t* labels, int32_t bh, int32_t N, int32_t C, int32_t nk,
                             int32_t block, int32_t rounds, const int32_t* row_ptr,
                             const int32_t* col_idx, int32_t* row_ptr_out, int32_t* col_idx_out,
                             void* ws, hipStream_t stream);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace svsa
