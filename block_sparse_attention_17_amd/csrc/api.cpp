// C ABI of the block-sparse video attention library: argument checks, geometry,
// workspace sizing and launches on the caller's stream.  Every check runs on
// the host before any work is enqueued; no C++ exception leaves this file.
#include <math.h>
#include <string.h>

#include "svsa.h"
#include "svsa_internal.h"

using svsa::Geom;

namespace {

constexpr int32_t kMaxHeadsMask = 256;
constexpr int32_t kMaxNb = 4096;

bool make_geom(const svsa_geom* in, Geom* g) {
  if (!in) return false;
  if (in->T < 1 || in->H < 1 || in->W < 1 || in->tt < 1 || in->th < 1 || in->tw < 1) return false;
  if (in->pad3d != 0 && in->pad3d != 1) return false;
  const int64_t N = (int64_t)in->T * in->H * in->W;
  const int64_t Bk = (int64_t)in->tt * in->th * in->tw;
  if (N >= (1ll << 30) || Bk >= 65536) return false;
  g->T = in->T; g->H = in->H; g->W = in->W;
  g->tt = in->tt; g->th = in->th; g->tw = in->tw;
  g->pad3d = in->pad3d;
  g->nT = (in->T + in->tt - 1) / in->tt;
  g->nH = (in->H + in->th - 1) / in->th;
  g->nW = (in->W + in->tw - 1) / in->tw;
  g->N = (int32_t)N;
  g->Bk = (int32_t)Bk;
  const int64_t nb = in->pad3d ? (int64_t)g->nT * g->nH * g->nW : (N + Bk - 1) / Bk;
  if (nb >= (1ll << 30)) return false;
  g->nb = (int32_t)nb;
  const int64_t Npad = (int64_t)g->nb * Bk;
  if (Npad >= (1ll << 30)) return false;
  g->Npad = (int32_t)Npad;
  return true;
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

// Alignment the kernels rely on: 16 bytes for bf16 / f32 tensors (16-byte
// vector loads and stores), 8 for float64 arrays, 4 for int32 arrays, 256 for
// workspaces (carved into 256-byte aligned regions).  NULL passes here; the
// NULL checks are separate.
bool al(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int elt_bytes(int32_t dtype) {
  return dtype == SVSA_BF16 ? 2 : dtype == SVSA_F32 ? 4 : 0;
}

int from_hip(hipError_t e) { return e == hipSuccess ? SVSA_OK : SVSA_E_HIP; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + nb && pb < pa + na;
}

}  // namespace

extern "C" {

int svsa_version(void) { return 102; }

// [iCATS] Sec. 4.2 / App. A: per-step top-p from the log-SNR of the noise
// schedule.  With x = (1 - s) x0 + s eps, SNR = ((1 - s) / s)^2 and
// sigmoid(-logSNR) = 1 / (1 + SNR) = s^2 / (s^2 + (1 - s)^2), written here in
// the form that stays finite at s = 0 and s = 1 (the denominator is >= 1/2).
int svsa_snr_top_p(const double* sigmas, int32_t steps, int32_t first_sparse, float p_min,
                   float tau, float* top_p) {
  if (!sigmas || !top_p || steps < 1 || first_sparse < 0 || first_sparse > steps)
    return SVSA_E_INVALID;
  if (!(p_min > 0.0f && p_min <= tau && tau <= 1.0f)) return SVSA_E_INVALID;
  for (int32_t k = 0; k < steps; ++k)
    if (!(sigmas[k] >= 0.0 && sigmas[k] <= 1.0)) return SVSA_E_INVALID;
  auto w = [&](int32_t k) {
    const double s = sigmas[k], r = 1.0 - s;
    return s * s / (s * s + r * r);
  };
  for (int32_t k = 0; k < first_sparse; ++k) top_p[k] = 1.0f;
  if (first_sparse == steps) return SVSA_OK;
  const double w_first = w(first_sparse), w_last = w(steps - 1);
  const double span = w_first - w_last;
  for (int32_t k = first_sparse; k < steps; ++k) {
    double u = span != 0.0 ? (w(k) - w_last) / span : 1.0;
    u = u < 0.0 ? 0.0 : (u > 1.0 ? 1.0 : u);
    top_p[k] = (float)((double)p_min + ((double)tau - (double)p_min) * u);
  }
  return SVSA_OK;
}

// ---------------------------------------------------------------------------
// Variable-size blocks ([iCATS] Sec. 4.1; [SVOO] QK co-clustering).
// ---------------------------------------------------------------------------
namespace {
constexpr int32_t kMaxClusters = 4096;

bool cluster_sizes_ok(int32_t batch, int32_t heads, int32_t n, int32_t C, int32_t D) {
  if (batch < 1 || heads < 1 || n < 1 || C < 1 || C > kMaxClusters) return false;
  const int64_t bh = (int64_t)batch * heads;
  return bh <= 65535 && bh * n < (1ll << 31) && bh * C * (int64_t)D < (1ll << 31);
}
}  // namespace

size_t svsa_kmeans_workspace_bytes(int32_t batch, int32_t heads, int32_t n, int32_t clusters,
                                   int32_t head_dim) {
  if (!cluster_sizes_ok(batch, heads, n, clusters, head_dim) || head_dim < 1) return 0;
  return svsa::kmeans_ws_layout(batch * heads, n, clusters, head_dim).total;
}

int svsa_kmeans(const void* x, int32_t batch, int32_t heads, int32_t n, int32_t head_dim,
                const double* metric, double* centroids, int32_t clusters, int32_t iters,
                int32_t* labels, int32_t* sizes, void* workspace, size_t ws_bytes,
                void* stream) {
  if (!(al(x, 16) && al(metric, 8) && al(centroids, 8) && al(labels, 4) && al(sizes, 4) &&
        al(workspace, 256)))
    return SVSA_E_INVALID;
  if (!x || !centroids || !labels || !sizes || !workspace || iters < 1 || head_dim < 1 ||
      !cluster_sizes_ok(batch, heads, n, clusters, head_dim))
    return SVSA_E_INVALID;
  if (head_dim != 64 && head_dim != 128) return SVSA_E_UNSUPPORTED;
  const int32_t bh = batch * heads;
  if (ws_bytes < svsa::kmeans_ws_layout(bh, n, clusters, head_dim).total) return SVSA_E_WORKSPACE;
  return from_hip(svsa::launch_kmeans(x, bh, n, head_dim, metric, centroids, clusters, iters,
                                      labels, sizes, workspace,
                                      static_cast<hipStream_t>(stream)));
}

size_t svsa_cluster_means_workspace_bytes(int32_t batch, int32_t heads, int32_t n,
                                          int32_t clusters) {
  if (!cluster_sizes_ok(batch, heads, n, clusters, 1)) return 0;
  return svsa::kmeans_ws_layout(batch * heads, n, clusters, 0).total;
}

int svsa_cluster_means(const void* x, const int32_t* labels, int32_t batch, int32_t heads,
                       int32_t n, int32_t head_dim, int32_t clusters, double* centroids,
                       int32_t* sizes, void* workspace, size_t ws_bytes, void* stream) {
  if (!(al(x, 2) && al(labels, 4) && al(centroids, 8) && al(sizes, 4) && al(workspace, 256)))
    return SVSA_E_INVALID;
  if (!x || !labels || !centroids || !sizes || !workspace || head_dim < 1 ||
      !cluster_sizes_ok(batch, heads, n, clusters, head_dim))
    return SVSA_E_INVALID;
  if (head_dim != 64 && head_dim != 128) return SVSA_E_UNSUPPORTED;
  const int32_t bh = batch * heads;
  const svsa::KmeansWs w = svsa::kmeans_ws_layout(bh, n, clusters, 0);
  if (ws_bytes < w.total) return SVSA_E_WORKSPACE;
  char* base = static_cast<char*>(workspace);
  int32_t* start = reinterpret_cast<int32_t*>(base + w.start_off);
  int32_t* token = reinterpret_cast<int32_t*>(base + w.token_off);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = svsa::launch_cluster_layout(labels, bh, n, clusters, 1, start, sizes, nullptr,
                                             token, base + w.layout_off, st);
  if (e == hipSuccess)
    e = svsa::launch_cluster_means(x, start, sizes, token, centroids, bh, n, clusters, head_dim,
                                   n, st);
  return from_hip(e);
}

int svsa_cluster_metric(const double* centroids, const int32_t* sizes, int32_t batch,
                        int32_t heads, int32_t clusters, int32_t head_dim, double* metric,
                        void* stream) {
  if (!(al(centroids, 8) && al(sizes, 4) && al(metric, 8))) return SVSA_E_INVALID;
  if (!centroids || !sizes || !metric || head_dim < 1 ||
      !cluster_sizes_ok(batch, heads, 1, clusters, head_dim))
    return SVSA_E_INVALID;
  if (head_dim % 16 != 0 || head_dim > 256) return SVSA_E_UNSUPPORTED;
  return from_hip(svsa::launch_cluster_metric(centroids, sizes, metric, batch * heads, clusters,
                                              head_dim, static_cast<hipStream_t>(stream)));
}

int64_t svsa_cluster_capacity(int32_t n, int32_t clusters, int32_t align) {
  if (n < 1 || clusters < 1 || clusters > kMaxClusters || align < 1 || align > 1024 ||
      !is_pow2(align))
    return 0;
  return svsa::cluster_lcap(n, clusters, align);
}

size_t svsa_cluster_layout_workspace_bytes(int32_t batch, int32_t heads, int32_t n,
                                           int32_t clusters) {
  if (!cluster_sizes_ok(batch, heads, n, clusters, 1)) return 0;
  return svsa::layout_ws_bytes(batch * heads, n, clusters);
}

int svsa_cluster_layout(const int32_t* labels, int32_t batch, int32_t heads, int32_t n,
                        int32_t clusters, int32_t align, int32_t* start, int32_t* sizes,
                        int32_t* slot, int32_t* token, void* workspace, size_t ws_bytes,
                        void* stream) {
  if (!(al(labels, 4) && al(start, 4) && al(sizes, 4) && al(slot, 4) && al(token, 4) &&
        al(workspace, 256)))
    return SVSA_E_INVALID;
  if (!labels || !start || !sizes || !token || !cluster_sizes_ok(batch, heads, n, clusters, 1))
    return SVSA_E_INVALID;
  const int64_t lcap = svsa_cluster_capacity(n, clusters, align);
  if (lcap == 0) return SVSA_E_INVALID;
  if ((int64_t)batch * heads * lcap >= (1ll << 31)) return SVSA_E_UNSUPPORTED;
  if (!workspace || ws_bytes < svsa::layout_ws_bytes(batch * heads, n, clusters))
    return SVSA_E_WORKSPACE;
  return from_hip(svsa::launch_cluster_layout(labels, batch * heads, n, clusters, align, start,
                                              sizes, slot, token, workspace,
                                              static_cast<hipStream_t>(stream)));
}

int svsa_cluster_permute(const void* src, void* dst, int32_t dtype, int32_t batch, int32_t heads,
                         int32_t n, int32_t head_dim, int32_t clusters, int32_t align,
                         const int32_t* map, const int32_t* start, int32_t inverse,
                         void* stream) {
  if (!(al(src, 16) && al(dst, 16) && al(map, 4) && al(start, 4))) return SVSA_E_INVALID;
  if (!src || !dst || !map || !start || head_dim < 1 ||
      !cluster_sizes_ok(batch, heads, n, clusters, 1))
    return SVSA_E_INVALID;
  const int64_t lcap = svsa_cluster_capacity(n, clusters, align);
  if (lcap == 0) return SVSA_E_INVALID;
  const int eb = elt_bytes(dtype);
  if (!eb) return SVSA_E_UNSUPPORTED;
  const int64_t row_bytes = (int64_t)head_dim * eb;
  if (row_bytes % 16 != 0 || !is_pow2(row_bytes / 16) || row_bytes > 4096)
    return SVSA_E_UNSUPPORTED;
  const int64_t bh = (int64_t)batch * heads;
  const size_t nat = (size_t)bh * n * row_bytes, pad = (size_t)bh * lcap * row_bytes;
  if (overlaps(src, inverse ? pad : nat, dst, inverse ? nat : pad)) return SVSA_E_INVALID;
  return from_hip(svsa::launch_cluster_permute(src, dst, eb, (int32_t)bh, n, head_dim, clusters,
                                               lcap, map, start, inverse != 0,
                                               static_cast<hipStream_t>(stream)));
}

size_t svsa_tail_merge_workspace_bytes(int32_t batch, int32_t heads, int32_t n, int32_t nq,
                                       int32_t nk) {
  if (!cluster_sizes_ok(batch, heads, n, nq, 1) || nk < 1 || nk > kMaxNb) return 0;
  return svsa::tail_ws_layout(batch * heads, n, nq, nk).total;
}

int svsa_tail_merge(int32_t* labels, int32_t batch, int32_t heads, int32_t n, int32_t nq,
                    int32_t nk, int32_t block, int32_t rounds, const int32_t* row_ptr,
                    const int32_t* col_idx, int32_t* row_ptr_out, int32_t* col_idx_out,
                    int64_t col_capacity, void* workspace, size_t ws_bytes, void* stream) {
  if (!(al(labels, 4) && al(row_ptr, 4) && al(col_idx, 4) && al(row_ptr_out, 4) &&
        al(col_idx_out, 4) && al(workspace, 256)))
    return SVSA_E_INVALID;
  if (!labels || !row_ptr || !col_idx || !row_ptr_out || !col_idx_out || block < 1 ||
      rounds < 0 || rounds > 8 || nk < 1 || !cluster_sizes_ok(batch, heads, n, nq, 1))
    return SVSA_E_INVALID;
  if (nk > kMaxNb) return SVSA_E_UNSUPPORTED;
  const int64_t worst = (int64_t)batch * heads * nq * nk;
  if (worst >= 0x7fffffff) return SVSA_E_UNSUPPORTED;
  if (col_capacity < worst) return SVSA_E_CAPACITY;
  if (!workspace || ws_bytes < svsa_tail_merge_workspace_bytes(batch, heads, n, nq, nk))
    return SVSA_E_WORKSPACE;
  return from_hip(svsa::launch_tail_merge(labels, batch * heads, n, nq, nk, block, rounds,
                                          row_ptr, col_idx, row_ptr_out, col_idx_out, workspace,
                                          static_cast<hipStream_t>(stream)));
}

const char* svsa_status_string(int status) {
  switch (status) {
    case SVSA_OK: return "ok";
    case SVSA_E_INVALID: return "invalid argument";
    case SVSA_E_UNSUPPORTED: return "unsupported argument (dtype, head_dim or size limit)";
    case SVSA_E_WORKSPACE: return "workspace too small";
    case SVSA_E_CAPACITY: return "col_idx capacity below the worst case";
    case SVSA_E_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int svsa_tile_permute(const void* src, void* dst, int32_t dtype, int32_t batch, int32_t heads,
                      int32_t head_dim, const svsa_geom* gin, int32_t inverse, void* stream) {
  if (!(al(src, 16) && al(dst, 16))) return SVSA_E_INVALID;
  Geom g;
  if (!src || !dst || batch < 1 || heads < 1 || head_dim < 1 || !make_geom(gin, &g))
    return SVSA_E_INVALID;
  const int eb = elt_bytes(dtype);
  if (!eb) return SVSA_E_UNSUPPORTED;
  const int64_t row_bytes = (int64_t)head_dim * eb;
  if (row_bytes % 16 != 0 || !is_pow2(row_bytes / 16) || row_bytes > 4096)
    return SVSA_E_UNSUPPORTED;
  const int64_t bh = (int64_t)batch * heads;
  if (bh * g.nT * g.nH * g.nW > 0x7fffffff) return SVSA_E_UNSUPPORTED;
  const size_t src_bytes = (size_t)bh * (inverse ? g.Npad : g.N) * row_bytes;
  const size_t dst_bytes = (size_t)bh * (inverse ? g.N : g.Npad) * row_bytes;
  if (overlaps(src, src_bytes, dst, dst_bytes)) return SVSA_E_INVALID;
  return from_hip(svsa::launch_tile_permute(src, dst, eb, (int32_t)bh, head_dim, g, inverse != 0,
                                            static_cast<hipStream_t>(stream)));
}

int svsa_pool(const void* x_tiled, int32_t dtype, double* out, int32_t batch, int32_t heads,
              int32_t head_dim, const svsa_geom* gin, void* stream) {
  if (!(al(x_tiled, 16) && al(out, 8))) return SVSA_E_INVALID;
  Geom g;
  if (!x_tiled || !out || batch < 1 || heads < 1 || head_dim < 1 || !make_geom(gin, &g))
    return SVSA_E_INVALID;
  const int eb = elt_bytes(dtype);
  if (!eb) return SVSA_E_UNSUPPORTED;
  const int64_t row_bytes = (int64_t)head_dim * eb;
  if (row_bytes % 16 != 0 || row_bytes / 16 > 256 || 256 % (row_bytes / 16) != 0 ||
      (256 / (row_bytes / 16)) * head_dim * 8 > 64 * 1024)
    return SVSA_E_UNSUPPORTED;
  const int64_t bh = (int64_t)batch * heads;
  if (bh * g.nb > 0x7fffffff) return SVSA_E_UNSUPPORTED;
  return from_hip(svsa::launch_pool(x_tiled, dtype == SVSA_BF16, out, (int32_t)bh, head_dim, g,
                                    static_cast<hipStream_t>(stream)));
}

int svsa_tile_permute_pool(const void* src, void* dst, double* means, int32_t dtype,
                           int32_t batch, int32_t heads, int32_t head_dim, const svsa_geom* gin,
                           void* stream) {
  if (!(al(src, 16) && al(dst, 16) && al(means, 8))) return SVSA_E_INVALID;
  Geom g;
  if (!src || !dst || !means || batch < 1 || heads < 1 || head_dim < 1 || !make_geom(gin, &g))
    return SVSA_E_INVALID;
  const int eb = elt_bytes(dtype);
  if (!eb) return SVSA_E_UNSUPPORTED;
  const int64_t row_bytes = (int64_t)head_dim * eb;
  if (row_bytes % 16 != 0 || row_bytes / 16 > 256 || 256 % (row_bytes / 16) != 0 ||
      (256 / (row_bytes / 16)) * head_dim * 8 > 64 * 1024)
    return SVSA_E_UNSUPPORTED;
  const int64_t bh = (int64_t)batch * heads;
  if (bh * g.nb > 0x7fffffff) return SVSA_E_UNSUPPORTED;
  const size_t src_bytes = (size_t)bh * g.N * row_bytes;
  const size_t dst_bytes = (size_t)bh * g.Npad * row_bytes;
  const size_t means_bytes = (size_t)bh * g.nb * head_dim * sizeof(double);
  if (overlaps(src, src_bytes, dst, dst_bytes) || overlaps(means, means_bytes, src, src_bytes) ||
      overlaps(means, means_bytes, dst, dst_bytes))
    return SVSA_E_INVALID;
  return from_hip(svsa::launch_tile_permute_pool(src, dst, means, dtype == SVSA_BF16, (int32_t)bh,
                                                 head_dim, g, static_cast<hipStream_t>(stream)));
}

size_t svsa_block_mask_workspace_bytes(int32_t batch, int32_t heads, int32_t nb) {
  if (batch < 1 || heads < 1 || nb < 1) return 0;
  return svsa::mask_ws_layout((int64_t)batch * heads * nb, nb).total;
}

int svsa_block_mask(const double* qbar, const double* kbar, int32_t batch, int32_t heads,
                    int32_t nb, int32_t head_dim, double softmax_scale, const float* top_p,
                    const float* keep_frac, int32_t band_width, int32_t* row_ptr,
                    int32_t* col_idx, int64_t col_capacity, void* workspace, size_t ws_bytes,
                    void* stream) {
  if (!(al(qbar, 8) && al(kbar, 8) && al(row_ptr, 4) && al(col_idx, 4) && al(workspace, 256)))
    return SVSA_E_INVALID;
  if (!qbar || !kbar || !row_ptr || !col_idx || batch < 1 || heads < 1 || nb < 1 ||
      head_dim < 1 || band_width < 1 || !isfinite(softmax_scale))
    return SVSA_E_INVALID;
  if ((top_p == nullptr) == (keep_frac == nullptr)) return SVSA_E_INVALID;
  const float* par = top_p ? top_p : keep_frac;
  for (int32_t h = 0; h < heads && h < kMaxHeadsMask; ++h)
    if (!(par[h] > 0.f && par[h] <= 1.f)) return SVSA_E_INVALID;
  if (heads > kMaxHeadsMask || nb > kMaxNb) return SVSA_E_UNSUPPORTED;
  const int64_t worst = (int64_t)batch * heads * nb * nb;
  if (worst >= 0x7fffffff) return SVSA_E_UNSUPPORTED;
  if (col_capacity < worst) return SVSA_E_CAPACITY;
  if (!workspace || ws_bytes < svsa_block_mask_workspace_bytes(batch, heads, nb))
    return SVSA_E_WORKSPACE;
  return from_hip(svsa::launch_block_mask(qbar, kbar, batch * heads, heads, nb, head_dim,
                                          softmax_scale, top_p, keep_frac, band_width, row_ptr,
                                          col_idx, workspace, static_cast<hipStream_t>(stream)));
}

int svsa_block_mask_noalloc(const double* qbar, const double* kbar, int32_t batch, int32_t heads,
                            int32_t nb, int32_t head_dim, double softmax_scale,
                            const float* top_p, const float* keep_frac, int32_t band_width,
                            int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                            void* stream) {
  if (!(al(qbar, 8) && al(kbar, 8) && al(row_ptr, 4) && al(col_idx, 4))) return SVSA_E_INVALID;
  if (!qbar || !kbar || !row_ptr || !col_idx || batch < 1 || heads < 1 || nb < 1 ||
      head_dim < 1 || band_width < 1 || !isfinite(softmax_scale))
    return SVSA_E_INVALID;
  if ((top_p == nullptr) == (keep_frac == nullptr)) return SVSA_E_INVALID;
  const float* par = top_p ? top_p : keep_frac;
  for (int32_t h = 0; h < heads && h < kMaxHeadsMask; ++h)
    if (!(par[h] > 0.f && par[h] <= 1.f)) return SVSA_E_INVALID;
  if (heads > kMaxHeadsMask || nb > kMaxNb) return SVSA_E_UNSUPPORTED;
  const int64_t worst = (int64_t)batch * heads * nb * nb;
  if (worst >= 0x7fffffff) return SVSA_E_UNSUPPORTED;
  if (col_capacity < worst) return SVSA_E_CAPACITY;
  if (!svsa::block_mask_fits_scratch((int64_t)batch * heads, nb)) return SVSA_E_WORKSPACE;
  return from_hip(svsa::launch_block_mask_noalloc(qbar, kbar, batch * heads, heads, nb, head_dim,
                                                  softmax_scale, top_p, keep_frac, band_width,
                                                  row_ptr, col_idx,
                                                  static_cast<hipStream_t>(stream)));
}

size_t svsa_cluster_mask_workspace_bytes(int32_t batch, int32_t heads, int32_t nq, int32_t nk) {
  if (batch < 1 || heads < 1 || nq < 1 || nk < 1) return 0;
  return svsa::mask_ws_layout((int64_t)batch * heads * nq, nk).total;
}

int svsa_cluster_mask(const double* qbar, const double* kbar, const int32_t* ksizes,
                      int32_t batch, int32_t heads, int32_t nq, int32_t nk, int32_t head_dim,
                      double softmax_scale, const float* top_p, const float* keep_frac,
                      int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                      void* workspace, size_t ws_bytes, void* stream) {
  if (!(al(qbar, 8) && al(kbar, 8) && al(ksizes, 4) && al(row_ptr, 4) && al(col_idx, 4) &&
        al(workspace, 256)))
    return SVSA_E_INVALID;
  if (!qbar || !kbar || !ksizes || !row_ptr || !col_idx || batch < 1 || heads < 1 || nq < 1 ||
      nk < 1 || head_dim < 1 || !isfinite(softmax_scale))
    return SVSA_E_INVALID;
  if ((top_p == nullptr) == (keep_frac == nullptr)) return SVSA_E_INVALID;
  const float* par = top_p ? top_p : keep_frac;
  for (int32_t h = 0; h < heads && h < kMaxHeadsMask; ++h)
    if (!(par[h] > 0.f && par[h] <= 1.f)) return SVSA_E_INVALID;
  if (heads > kMaxHeadsMask || nk > kMaxNb || nq > kMaxNb) return SVSA_E_UNSUPPORTED;
  const int64_t worst = (int64_t)batch * heads * nq * nk;
  if (worst >= 0x7fffffff) return SVSA_E_UNSUPPORTED;
  if (col_capacity < worst) return SVSA_E_CAPACITY;
  if (!workspace || ws_bytes < svsa_cluster_mask_workspace_bytes(batch, heads, nq, nk))
    return SVSA_E_WORKSPACE;
  return from_hip(svsa::launch_cluster_mask(qbar, kbar, ksizes, batch * heads, heads, nq, nk,
                                            head_dim, softmax_scale, top_p, keep_frac, 0,
                                            row_ptr, col_idx, workspace,
                                            static_cast<hipStream_t>(stream)));
}

size_t svsa_stripe_mask_workspace_bytes(int32_t batch, int32_t heads, const svsa_geom* gin) {
  Geom g;
  if (batch < 1 || heads < 1 || !make_geom(gin, &g)) return 0;
  return svsa::stripe_ws_layout((int64_t)batch * heads * g.nb, g).total;
}

int svsa_stripe_mask(const svsa_geom* gin, int32_t batch, int32_t heads, const int32_t* params,
                     int32_t band_width, int32_t* row_ptr, int32_t* col_idx,
                     int64_t col_capacity, void* workspace, size_t ws_bytes, void* stream) {
  if (!(al(row_ptr, 4) && al(col_idx, 4) && al(workspace, 256))) return SVSA_E_INVALID;
  Geom g;
  if (!params || !row_ptr || !col_idx || batch < 1 || heads < 1 || band_width < 0 ||
      !make_geom(gin, &g))
    return SVSA_E_INVALID;
  for (int32_t h = 0; h < heads && h < svsa::kStripeMaxHeads; ++h)
    if (params[h * 6 + 0] < 1 || params[h * 6 + 3] < 1) return SVSA_E_INVALID;
  if (heads > svsa::kStripeMaxHeads || g.nb > kMaxNb || g.Bk > 1024) return SVSA_E_UNSUPPORTED;
  const int64_t worst = (int64_t)batch * heads * g.nb * g.nb;
  if (worst >= 0x7fffffff) return SVSA_E_UNSUPPORTED;
  if (col_capacity < worst) return SVSA_E_CAPACITY;
  if (!workspace || ws_bytes < svsa_stripe_mask_workspace_bytes(batch, heads, gin))
    return SVSA_E_WORKSPACE;
  return from_hip(svsa::launch_stripe_mask(g, batch * heads, heads, params, band_width, row_ptr,
                                           col_idx, workspace, static_cast<hipStream_t>(stream)));
}

size_t svsa_attn_workspace_bytes(int32_t batch, int32_t heads, const svsa_geom* gin) {
  Geom g;
  if (batch < 1 || heads < 1 || !make_geom(gin, &g)) return 0;
  if (g.Bk % 32 != 0) return 0;
  return svsa::attn_ws_layout(batch * heads, g).total;
}

namespace {
int attn_impl(const void* q, const void* k, const void* v, void* out, int32_t batch,
              int32_t heads, int32_t head_dim, const svsa_geom* gin, float softmax_scale,
              const int32_t* row_ptr, const int32_t* col_idx, int32_t flags, void* workspace,
              size_t ws_bytes, void* stream) {
  if (flags & ~(SVSA_ATTN_OUT_NATURAL | SVSA_ATTN_POSITIONAL_GROUPS | SVSA_ATTN_GROUPS_BY_LIST |
                SVSA_ATTN_STEP_PAIRS))
    return SVSA_E_INVALID;
  if ((flags & SVSA_ATTN_POSITIONAL_GROUPS) && (flags & SVSA_ATTN_GROUPS_BY_LIST))
    return SVSA_E_INVALID;
  const bool natural = (flags & SVSA_ATTN_OUT_NATURAL) != 0;
  const bool steps = (flags & SVSA_ATTN_STEP_PAIRS) != 0;
  const int regroup = (flags & SVSA_ATTN_POSITIONAL_GROUPS) ? 0
                      : (flags & SVSA_ATTN_GROUPS_BY_LIST) ? 2 : 1;
  if (!(al(q, 16) && al(k, 16) && al(v, 16) && al(out, 16) && al(row_ptr, 4) && al(col_idx, 4) &&
        al(workspace, 256)))
    return SVSA_E_INVALID;
  Geom g;
  // v == NULL: V^T was staged into the workspace by svsa_attn_stage_v
  if (!q || !k || !out || !row_ptr || !col_idx || batch < 1 || heads < 1 ||
      head_dim < 1 || !make_geom(gin, &g) || !isfinite(softmax_scale))
    return SVSA_E_INVALID;
  if (head_dim != 64 && head_dim != 128) return SVSA_E_UNSUPPORTED;
  if (g.Bk % 32 != 0 || g.nb > kMaxNb) return SVSA_E_UNSUPPORTED;
  const int32_t sub = g.Bk % 64 == 0 ? 64 : 32;
  // sub-blocks seen by the kernels
  const int64_t nbs = g.pad3d ? (int64_t)g.nb * (g.Bk / sub) : ((int64_t)g.N + sub - 1) / sub;
  if (nbs > kMaxNb) return SVSA_E_UNSUPPORTED;
  if ((int64_t)g.Npad * head_dim * 2 >= (1ll << 31)) return SVSA_E_UNSUPPORTED;
  const int64_t bh = (int64_t)batch * heads;
  if (bh * nbs * nbs >= 0x7fffffff) return SVSA_E_UNSUPPORTED;
  const size_t tbytes = (size_t)bh * g.Npad * head_dim * 2;
  const size_t obytes = natural ? (size_t)bh * g.N * head_dim * 2 : tbytes;
  if (overlaps(out, obytes, q, tbytes) || overlaps(out, obytes, k, tbytes) ||
      (v && overlaps(out, obytes, v, tbytes)))
    return SVSA_E_INVALID;
  if (!workspace || ws_bytes < svsa_attn_workspace_bytes(batch, heads, gin))
    return SVSA_E_WORKSPACE;
  if (overlaps(out, obytes, workspace, ws_bytes)) return SVSA_E_INVALID;
  return from_hip(svsa::launch_block_sparse_attn(q, k, v, out, (int32_t)bh, head_dim, g,
                                                 softmax_scale, row_ptr, col_idx, workspace,
                                                 natural, regroup, steps,
                                                 static_cast<hipStream_t>(stream)));
}
}  // namespace

int svsa_block_sparse_attn(const void* q, const void* k, const void* v, void* out, int32_t batch,
                           int32_t heads, int32_t head_dim, const svsa_geom* g,
                           float softmax_scale, const int32_t* row_ptr, const int32_t* col_idx,
                           void* workspace, size_t ws_bytes, void* stream) {
  return attn_impl(q, k, v, out, batch, heads, head_dim, g, softmax_scale, row_ptr, col_idx, 0,
                   workspace, ws_bytes, stream);
}

int svsa_block_sparse_attn_ex(const void* q, const void* k, const void* v, void* out,
                              int32_t batch, int32_t heads, int32_t head_dim, const svsa_geom* g,
                              float softmax_scale, const int32_t* row_ptr,
                              const int32_t* col_idx, int32_t flags, void* workspace,
                              size_t ws_bytes, void* stream) {
  return attn_impl(q, k, v, out, batch, heads, head_dim, g, softmax_scale, row_ptr, col_idx,
                   flags, workspace, ws_bytes, stream);
}

int svsa_attn_stage_v(const void* v, int32_t batch, int32_t heads, int32_t head_dim,
                      const svsa_geom* gin, void* workspace, size_t ws_bytes, void* stream) {
  if (!(al(v, 16) && al(workspace, 256))) return SVSA_E_INVALID;
  Geom g;
  if (!v || batch < 1 || heads < 1 || head_dim < 1 || !make_geom(gin, &g))
    return SVSA_E_INVALID;
  if (head_dim != 64 && head_dim != 128) return SVSA_E_UNSUPPORTED;
  if (g.Bk % 32 != 0 || g.nb > kMaxNb) return SVSA_E_UNSUPPORTED;
  const int32_t sub = g.Bk % 64 == 0 ? 64 : 32;
  const int64_t nbs = g.pad3d ? (int64_t)g.nb * (g.Bk / sub) : ((int64_t)g.N + sub - 1) / sub;
  if (nbs > kMaxNb) return SVSA_E_UNSUPPORTED;
  if ((int64_t)g.Npad * head_dim * 2 >= (1ll << 31)) return SVSA_E_UNSUPPORTED;
  const int64_t bh = (int64_t)batch * heads;
  if (bh * nbs * nbs >= 0x7fffffff) return SVSA_E_UNSUPPORTED;
  if (!workspace || ws_bytes < svsa_attn_workspace_bytes(batch, heads, gin))
    return SVSA_E_WORKSPACE;
  if (overlaps(v, (size_t)bh * g.N * head_dim * 2, workspace, ws_bytes)) return SVSA_E_INVALID;
  return from_hip(svsa::launch_attn_stage_v(v, (int32_t)bh, head_dim, g, workspace,
                                            static_cast<hipStream_t>(stream)));
}

size_t svsa_cluster_attn_workspace_bytes(int32_t batch, int32_t heads, int32_t n_q, int32_t nq,
                                         int32_t n_k, int32_t nk, int32_t align) {
  if (batch < 1 || heads < 1 || (align != 32 && align != 64)) return 0;
  const int64_t cap_q = svsa_cluster_capacity(n_q, nq, align);
  const int64_t cap_k = svsa_cluster_capacity(n_k, nk, align);
  if (cap_q == 0 || cap_k == 0) return 0;
  return svsa::cluster_attn_ws_layout(batch * heads, align, cap_q, cap_k).total;
}

int svsa_cluster_attn(const void* q, const void* k, const void* v, void* out, int32_t batch,
                      int32_t heads, int32_t head_dim, int32_t n_q, int32_t nq,
                      const int32_t* q_start, const int32_t* q_size, int32_t n_k, int32_t nk,
                      const int32_t* k_start, const int32_t* k_size, int32_t align,
                      float softmax_scale, const int32_t* row_ptr, const int32_t* col_idx,
                      void* workspace, size_t ws_bytes, void* stream) {
  if (!(al(q, 16) && al(k, 16) && al(v, 16) && al(out, 16) && al(q_start, 4) && al(q_size, 4) &&
        al(k_start, 4) && al(k_size, 4) && al(row_ptr, 4) && al(col_idx, 4) && al(workspace, 256)))
    return SVSA_E_INVALID;
  if (!q || !k || !v || !out || !q_start || !q_size || !k_start || !k_size || !row_ptr ||
      !col_idx || batch < 1 || heads < 1 || head_dim < 1 || !isfinite(softmax_scale))
    return SVSA_E_INVALID;
  if (align != 32 && align != 64) return SVSA_E_INVALID;
  const int64_t cap_q = svsa_cluster_capacity(n_q, nq, align);
  const int64_t cap_k = svsa_cluster_capacity(n_k, nk, align);
  if (cap_q == 0 || cap_k == 0) return SVSA_E_INVALID;
  if (head_dim != 64 && head_dim != 128) return SVSA_E_UNSUPPORTED;
  const int64_t bh = (int64_t)batch * heads;
  // key sub-blocks fit the 13-bit index of the schedule entries; one head's
  // rows fit a 32-bit buffer range
  if (cap_k / align > 8192 || cap_q * head_dim * 2 >= (1ll << 31) ||
      cap_k * head_dim * 2 >= (1ll << 31) || bh > 65535)
    return SVSA_E_UNSUPPORTED;
  const int64_t groups = (cap_q / align + 256 / align - 1) / (256 / align);
  if (bh * groups * (cap_k / align) >= 0x7fffffff || bh * nq * nk >= 0x7fffffff)
    return SVSA_E_UNSUPPORTED;
  const size_t qbytes = (size_t)bh * cap_q * head_dim * 2;
  const size_t kbytes = (size_t)bh * cap_k * head_dim * 2;
  if (overlaps(out, qbytes, q, qbytes) || overlaps(out, qbytes, k, kbytes) ||
      overlaps(out, qbytes, v, kbytes))
    return SVSA_E_INVALID;
  if (!workspace ||
      ws_bytes < svsa_cluster_attn_workspace_bytes(batch, heads, n_q, nq, n_k, nk, align))
    return SVSA_E_WORKSPACE;
  return from_hip(svsa::launch_cluster_attn(q, k, v, out, (int32_t)bh, head_dim, align, cap_q,
                                            cap_k, q_start, q_size, nq, k_start, k_size, nk,
                                            softmax_scale, row_ptr, col_idx, workspace,
                                            static_cast<hipStream_t>(stream)));
}

}  // extern "C"
