"""MI355X (gfx950) block-sparse video attention: top-p block masks over 3D tiles.

Python face of ``libsvsa.so`` (HIP kernels behind a C ABI, ``include/svsa.h``).
Importing fails loudly when the library has not been built.
"""
from .binding import (svsa_cluster_attn, svsa_cluster_attn_workspace_bytes,
                      svsa_cluster_capacity, svsa_cluster_layout,
                      svsa_cluster_layout_workspace_bytes, svsa_cluster_mask,
                      svsa_cluster_means, svsa_cluster_means_workspace_bytes,
                      svsa_cluster_mask_workspace_bytes, svsa_cluster_metric, svsa_cluster_permute,
                      svsa_kmeans, svsa_kmeans_workspace_bytes, svsa_tail_merge,
                      svsa_tail_merge_workspace_bytes)
from .binding import (EXPORTED, Geometry, SvsaError, SVSA_BF16, SVSA_F32, library, library_path,
                      status_string, svsa_attn_workspace_bytes, svsa_block_mask,
                      svsa_block_mask_workspace_bytes, svsa_block_mask_noalloc,
                      svsa_block_sparse_attn, svsa_pool,
                      svsa_snr_top_p, svsa_status_string, svsa_stripe_mask,
                      svsa_stripe_mask_workspace_bytes, svsa_tile_permute, svsa_tile_permute_pool,
                      svsa_attn_stage_v, svsa_block_sparse_attn_ex,
                      SVSA_ATTN_OUT_NATURAL, SVSA_ATTN_POSITIONAL_GROUPS,
                      SVSA_ATTN_GROUPS_BY_LIST, SVSA_ATTN_STEP_PAIRS, svsa_version)
from .pipeline import BlockSparseAttention, ClusteredAttention

__all__ = ["EXPORTED", "Geometry", "SvsaError", "SVSA_BF16", "SVSA_F32", "library",
           "library_path", "status_string", "svsa_attn_workspace_bytes", "svsa_block_mask",
           "svsa_block_mask_workspace_bytes", "svsa_block_mask_noalloc", "svsa_block_sparse_attn",
           "svsa_pool",
           "svsa_snr_top_p", "svsa_status_string", "svsa_stripe_mask",
           "svsa_stripe_mask_workspace_bytes", "svsa_tile_permute", "svsa_tile_permute_pool",
           "svsa_attn_stage_v", "svsa_block_sparse_attn_ex", "SVSA_ATTN_OUT_NATURAL",
           "SVSA_ATTN_POSITIONAL_GROUPS", "SVSA_ATTN_GROUPS_BY_LIST", "SVSA_ATTN_STEP_PAIRS",
           "svsa_version",
           "BlockSparseAttention", "ClusteredAttention", "svsa_cluster_attn",
           "svsa_cluster_attn_workspace_bytes", "svsa_cluster_capacity", "svsa_cluster_layout",
           "svsa_cluster_mask", "svsa_cluster_mask_workspace_bytes", "svsa_cluster_metric",
           "svsa_cluster_permute", "svsa_kmeans", "svsa_kmeans_workspace_bytes",
           "svsa_cluster_means", "svsa_cluster_means_workspace_bytes",
           "svsa_cluster_layout_workspace_bytes", "svsa_tail_merge",
           "svsa_tail_merge_workspace_bytes"]
