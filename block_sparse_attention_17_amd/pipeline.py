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
        self.vt = torch.empty(shp_t, **bf)
        self.ot = torch.empty(shp_t, **bf)
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
        B.svsa_tile_permute(q, self.qt, self.geom, stream=stream)
        B.svsa_tile_permute(k, self.kt, self.geom, stream=stream)
        B.svsa_tile_permute(v, self.vt, self.geom, stream=stream)

    def build_mask(self, top_p=None, keep_frac=None, band_width=1, stream=None):
        B.svsa_pool(self.qt, self.qbar, self.geom, stream=stream)
        B.svsa_pool(self.kt, self.kbar, self.geom, stream=stream)
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

    def attend(self, scale=None, stream=None, row_ptr=None, col_idx=None):
        scale = 1.0 / sqrt(self.head_dim) if scale is None else scale
        B.svsa_block_sparse_attn(self.qt, self.kt, self.vt, self.ot, self.geom, scale,
                                 self.row_ptr if row_ptr is None else row_ptr,
                                 self.col_idx if col_idx is None else col_idx,
                                 self.attn_ws, stream=stream)

    def permute_out(self, stream=None):
        B.svsa_tile_permute(self.ot, self.out, self.geom, inverse=True, stream=stream)
        return self.out

    def __call__(self, q, k, v, top_p=None, keep_frac=None, band_width=1, stream=None):
        """One pass of the whole path; returns the natural-order bf16 output."""
        self.permute_in(q, k, v, stream)
        self.build_mask(top_p, keep_frac, band_width, stream)
        self.attend(stream=stream)
        return self.permute_out(stream)
