"""The whole block-sparse attention path as one reusable object.

Holds the device buffers of one problem shape (allocated once through torch)
and chains the four C entry points: tile reorder of Q, K, V -> block means of
Q and K -> top-p (or fixed-fraction) block mask -> block-sparse attention ->
inverse reorder of the output.  No arithmetic happens here.
"""
from math import sqrt

import torch

from . import binding as B


class BlockSparseAttention:
    def __init__(self, batch, heads, head_dim, geom, device="cuda"):
        self.batch, self.heads, self.head_dim, self.geom = batch, heads, head_dim, geom
        g = geom
        dev = torch.device(device)
        bf = dict(dtype=torch.bfloat16, device=dev)
        shp_t = (batch, heads, g.N_pad, head_dim)
        self.qt = torch.empty(shp_t, **bf)
        self.kt = torch.empty(shp_t, **bf)
        self.ot = torch.empty(shp_t, **bf)   # V goes straight into attn_ws (no tiled copy)
        self.out = torch.empty((batch, heads, g.N, head_dim), **bf)
        self.qbar = torch.empty((batch, heads, g.nb, head_dim), dtype=torch.float64, device=dev)
        self.kbar = torch.empty_like(self.qbar)
        rows = batch * heads * g.nb
        self.row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
        self.col_idx = torch.empty(rows * g.nb, dtype=torch.int32, device=dev)
        self.mask_ws = torch.empty(B.svsa_block_mask_workspace_bytes(batch, heads, g.nb),
                                   dtype=torch.uint8, device=dev)
        self.attn_ws = torch.empty(B.svsa_attn_workspace_bytes(batch, heads, g),
                                   dtype=torch.uint8, device=dev)

    def permute_in(self, q, k, v, stream=None):
        """Tile reorder of Q and K with their block means (qbar / kbar) in the same
        pass; V is reordered straight into the attention workspace's V^T."""
        B.svsa_tile_permute_pool(q, self.qt, self.qbar, self.geom, stream=stream)
        B.svsa_tile_permute_pool(k, self.kt, self.kbar, self.geom, stream=stream)
        B.svsa_attn_stage_v(v, self.attn_ws, self.geom, stream=stream)

    def build_mask(self, top_p=None, keep_frac=None, band_width=1, stream=None):
        """Block mask from the block means that permute_in wrote."""
        B.svsa_block_mask(self.qbar, self.kbar, 1.0 / sqrt(self.head_dim), self.row_ptr,
                          self.col_idx, self.mask_ws, top_p=top_p, keep_frac=keep_frac,
                          band_width=band_width, stream=stream)

    def build_stripe_mask(self, params, band_width=0, stream=None):
        """CSR of the PSA stripe mask (params: [heads, 6], tile units) into
        row_ptr / col_idx; the stripe workspace is allocated on first use."""
        if getattr(self, "stripe_ws", None) is None:
            self.stripe_ws = torch.empty(
                B.svsa_stripe_mask_workspace_bytes(self.batch, self.heads, self.geom),
                dtype=torch.uint8, device=self.row_ptr.device)
        B.svsa_stripe_mask(self.geom, self.batch, params, self.row_ptr, self.col_idx,
                           self.stripe_ws, band_width=band_width, stream=stream)

    def attend(self, scale=None, stream=None, row_ptr=None, col_idx=None, natural_out=False,
               groups="auto", step_pairs=False):
        """Attention over the CSR lists into ot (tile order), or straight into out
        (natural order, natural_out=True: the kernel does the inverse reorder).
        groups: "auto" (query blocks grouped by their lists when the work is
        large enough), "list" (always when the blocks allow it) or "positional".
        step_pairs: walk each union list in steps of one or two key blocks with
        disjoint keepers (SVSA_ATTN_STEP_PAIRS; pays on fixed-fraction masks)."""
        scale = 1.0 / sqrt(self.head_dim) if scale is None else scale
        gflag = {"auto": 0, "list": B.SVSA_ATTN_GROUPS_BY_LIST,
                 "positional": B.SVSA_ATTN_POSITIONAL_GROUPS}[groups]
        flags = ((B.SVSA_ATTN_OUT_NATURAL if natural_out else 0) | gflag
                 | (B.SVSA_ATTN_STEP_PAIRS if step_pairs else 0))
        B.svsa_block_sparse_attn_ex(self.qt, self.kt, None, self.out if natural_out else self.ot,
                                    self.geom, scale,
                                    self.row_ptr if row_ptr is None else row_ptr,
                                    self.col_idx if col_idx is None else col_idx,
                                    self.attn_ws, flags=flags, stream=stream)
        return self.out if natural_out else self.ot

    def permute_out(self, stream=None):
        B.svsa_tile_permute(self.ot, self.out, self.geom, inverse=True, stream=stream)
        return self.out

    def __call__(self, q, k, v, top_p=None, keep_frac=None, band_width=1, stream=None):
        """One pass of the whole path; returns the natural-order bf16 output.
        Fixed-fraction masks (keep_frac) run with step pairs."""
        self.permute_in(q, k, v, stream)
        self.build_mask(top_p, keep_frac, band_width, stream)
        return self.attend(stream=stream, natural_out=True, step_pairs=keep_frac is not None)


class ClusteredAttention:
    """Attention over variable-size blocks from query / key clustering
    ([iCATS] Sec. 4.1; [SVOO] QK co-clustering), chaining the cluster entry
    points: query k-means under the key clusters' metric (plain feature space
    on the first call) -> key k-means under the updated query clusters'
    metric -> cluster mask -> optional tail merging of the query clusters
    ([iCATS] Sec. 4.3) -> padded cluster layouts -> permuted Q, K, V ->
    cluster attention -> token order.  Centroids persist between calls (warm
    start across denoising steps); initial centroids are the caller's."""

    def __init__(self, batch, heads, head_dim, n, q_clusters, k_clusters, align=32,
                 q_iters=2, k_iters=2, tail_merge=False, tail_rounds=2, device="cuda"):
        # align: cluster padding granularity, 32 or 64 tokens.  Clusters of a
        # few dozen to a few hundred tokens waste less at 32, and the attention
        # kernel then streams two 32-token entries per 64-key tile.
        self.batch, self.heads, self.head_dim, self.n = batch, heads, head_dim, n
        self.nq, self.nk, self.align = q_clusters, k_clusters, align
        self.q_iters, self.k_iters = q_iters, k_iters
        dev = torch.device(device)
        f64 = dict(dtype=torch.float64, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        bf = dict(dtype=torch.bfloat16, device=dev)
        bh = (batch, heads)
        self.qcent = torch.empty(bh + (q_clusters, head_dim), **f64)
        self.kcent = torch.empty(bh + (k_clusters, head_dim), **f64)
        self.metric = torch.empty(bh + (head_dim, head_dim), **f64)
        self.qlab = torch.empty(bh + (n,), **i32)
        self.klab = torch.empty(bh + (n,), **i32)
        self.qsize = torch.zeros(bh + (q_clusters,), **i32)
        self.ksize = torch.zeros(bh + (k_clusters,), **i32)
        self.cap_q = B.svsa_cluster_capacity(n, q_clusters, align)
        self.cap_k = B.svsa_cluster_capacity(n, k_clusters, align)
        self.q_start = torch.empty(bh + (q_clusters + 1,), **i32)
        self.k_start = torch.empty(bh + (k_clusters + 1,), **i32)
        self.q_slot = torch.empty(bh + (n,), **i32)
        self.k_slot = torch.empty(bh + (n,), **i32)
        self.q_token = torch.empty(bh + (self.cap_q,), **i32)
        self.k_token = torch.empty(bh + (self.cap_k,), **i32)
        self.qp = torch.empty(bh + (self.cap_q, head_dim), **bf)
        self.kp = torch.empty(bh + (self.cap_k, head_dim), **bf)
        self.vp = torch.empty(bh + (self.cap_k, head_dim), **bf)
        self.op = torch.empty(bh + (self.cap_q, head_dim), **bf)
        self.out = torch.empty(bh + (n, head_dim), **bf)
        rows = batch * heads * q_clusters
        self.row_ptr = torch.empty(rows + 1, **i32)
        self.col_idx = torch.empty(rows * k_clusters, **i32)
        km = max(B.svsa_kmeans_workspace_bytes(batch, heads, n, q_clusters, head_dim),
                 B.svsa_kmeans_workspace_bytes(batch, heads, n, k_clusters, head_dim))
        self.km_ws = torch.empty(km, dtype=torch.uint8, device=dev)
        self.layout_ws = torch.empty(
            max(B.svsa_cluster_layout_workspace_bytes(batch, heads, n, q_clusters),
                B.svsa_cluster_layout_workspace_bytes(batch, heads, n, k_clusters)),
            dtype=torch.uint8, device=dev)
        self.mask_ws = torch.empty(
            B.svsa_cluster_mask_workspace_bytes(batch, heads, q_clusters, k_clusters),
            dtype=torch.uint8, device=dev)
        self.attn_ws = torch.empty(
            B.svsa_cluster_attn_workspace_bytes(batch, heads, n, q_clusters, n, k_clusters, align),
            dtype=torch.uint8, device=dev)
        self.tail_merge, self.tail_rounds = tail_merge, tail_rounds
        if tail_merge:
            self.row_ptr_m = torch.empty_like(self.row_ptr)
            self.col_idx_m = torch.empty_like(self.col_idx)
            self.tail_ws = torch.empty(
                B.svsa_tail_merge_workspace_bytes(batch, heads, n, q_clusters, k_clusters),
                dtype=torch.uint8, device=dev)
        self.warm = False

    def set_centroids(self, qcent, kcent):
        """Initial centroids (float64 [B, Hh, C, D]); the next call clusters the
        queries in plain feature space."""
        self.qcent.copy_(qcent)
        self.kcent.copy_(kcent)
        self.warm = False

    def cluster(self, q, k, stream=None):
        if self.warm:
            B.svsa_cluster_metric(self.kcent, self.ksize, self.metric, stream=stream)
        B.svsa_kmeans(q, self.qcent, self.qlab, self.qsize, self.km_ws, self.q_iters,
                      metric=self.metric if self.warm else None, stream=stream)
        B.svsa_cluster_metric(self.qcent, self.qsize, self.metric, stream=stream)
        B.svsa_kmeans(k, self.kcent, self.klab, self.ksize, self.km_ws, self.k_iters,
                      metric=self.metric, stream=stream)
        self.warm = True

    def layout(self, q, k, v, stream=None):
        a = self.align
        B.svsa_cluster_layout(self.qlab, self.nq, a, self.q_start, self.qsize, self.q_slot,
                              self.q_token, self.layout_ws, stream=stream)
        B.svsa_cluster_layout(self.klab, self.nk, a, self.k_start, self.ksize, self.k_slot,
                              self.k_token, self.layout_ws, stream=stream)
        B.svsa_cluster_permute(q, self.qp, self.n, self.nq, a, self.q_token, self.q_start,
                               stream=stream)
        B.svsa_cluster_permute(k, self.kp, self.n, self.nk, a, self.k_token, self.k_start,
                               stream=stream)
        B.svsa_cluster_permute(v, self.vp, self.n, self.nk, a, self.k_token, self.k_start,
                               stream=stream)

    def build_mask(self, top_p=None, keep_frac=None, stream=None):
        B.svsa_cluster_mask(self.qcent, self.kcent, self.ksize, 1.0 / sqrt(self.head_dim),
                            self.row_ptr, self.col_idx, self.mask_ws, top_p=top_p,
                            keep_frac=keep_frac, stream=stream)

    def merge_tails(self, stream=None):
        """[iCATS] Sec. 4.3 tail merging of the query clusters (labels in place;
        the merged mask goes to row_ptr_m / col_idx_m)."""
        B.svsa_tail_merge(self.qlab, self.nq, self.nk, self.align, self.row_ptr, self.col_idx,
                          self.row_ptr_m, self.col_idx_m, self.tail_ws, rounds=self.tail_rounds,
                          stream=stream)

    def attend(self, row_ptr=None, col_idx=None, stream=None):
        if row_ptr is None:
            row_ptr, col_idx = ((self.row_ptr_m, self.col_idx_m) if self.tail_merge
                                else (self.row_ptr, self.col_idx))
        B.svsa_cluster_attn(self.qp, self.kp, self.vp, self.op, self.n, self.q_start, self.qsize,
                            self.n, self.k_start, self.ksize, self.align,
                            1.0 / sqrt(self.head_dim), row_ptr, col_idx, self.attn_ws,
                            stream=stream)

    def permute_out(self, stream=None):
        B.svsa_cluster_permute(self.op, self.out, self.n, self.nq, self.align, self.q_slot,
                               self.q_start, inverse=True, stream=stream)
        return self.out

    def __call__(self, q, k, v, top_p=None, keep_frac=None, stream=None):
        self.cluster(q, k, stream)
        self.build_mask(top_p, keep_frac, stream)
        if self.tail_merge:
            self.merge_tails(stream)
        self.layout(q, k, v, stream)
        self.attend(stream=stream)
        return self.permute_out(stream)
