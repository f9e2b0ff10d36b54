"""The five workload shapes of the block-sparse video attention path.

Grids and head shapes follow the pages: the Wan2.1 / HunyuanVideo latent
grids 21x45x80 and 33x45x80 are the DiT shapes given in the PSA paper
(Parameterized Stripe Attention for Efficient Video Generation), App. C.2
"Initialization of Mask Candidates", and heads x head_dim (40x128 for Wan2.1-14B, 24x128
for HunyuanVideo) are the ones that reproduce the dense TFLOP column of PSA
Table 2 (4*N^2*D*heads).  The tiny and small cases are CPU-checkable shapes; small_b2 is the small shape
with batch 2.  The *_pad3d / *_psa3d cases use PSA's 3D padding (one block per
tile, padding inside the sequence; PSA App. C.2).
"""
from dataclasses import dataclass, field
from math import ceil


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int          # enters every seed, so configs never share draws
    batch: int
    heads: int
    head_dim: int
    grid: tuple          # (T, H, W) latent grid
    tile: tuple          # (tt, th, tw) tile shape; block = one tile volume
    src_dtype: str       # "fp32" (tiny case) or "bf16"
    top_p: tuple         # top-p values run on this config (first = default)
    band: int = 1        # diagonal band width w: keep |i-j| <= w-1
    pe_scale: str = "fixed"      # "fixed" (1.5) or "uniform" (U[0.5, 3.0] per head)
    pe_freq: str = "unit"        # "unit" or "per_head" (2^U[-2,0] per head)
    fixed_mode: bool = False     # also run the per-head keep-fraction mode
    pad3d: bool = False          # one block per tile, padding inside the sequence

    @property
    def N(self):
        T, H, W = self.grid
        return T * H * W

    @property
    def Bk(self):
        tt, th, tw = self.tile
        return tt * th * tw

    @property
    def nb(self):
        if self.pad3d:
            return ceil(self.grid[0] / self.tile[0]) * ceil(self.grid[1] / self.tile[1]) * \
                ceil(self.grid[2] / self.tile[2])
        return ceil(self.N / self.Bk)

    @property
    def N_pad(self):
        return self.nb * self.Bk


CONFIGS = {
    "tiny": Config("tiny", 1, 1, 1, 64, (4, 8, 8), (2, 4, 4), "fp32", (0.9,)),
    "small": Config("small", 2, 1, 8, 64, (8, 16, 16), (4, 4, 4), "bf16", (0.9,),
                    pe_freq="per_head"),
    "wan480": Config("wan480", 3, 1, 40, 128, (21, 30, 52), (4, 4, 4), "bf16", (0.9,),
                     pe_scale="uniform"),
    "wan720": Config("wan720", 4, 1, 40, 128, (21, 45, 80), (4, 4, 4), "bf16",
                     (0.9, 0.8, 0.95), pe_scale="uniform"),
    "hv720": Config("hv720", 5, 1, 24, 128, (33, 45, 80), (4, 4, 4), "bf16", (0.9,),
                    pe_scale="uniform", fixed_mode=True),
    # the Wan2.1-720p shape with PSA's PSABlock shape 3x8x16 (384 tokens) as the
    # tile ([PSA] App. C.2), tail padding only: 197 blocks of 384
    "wan720_psa": Config("wan720_psa", 7, 1, 40, 128, (21, 45, 80), (3, 8, 16), "bf16", (0.9,),
                         pe_scale="uniform"),
    # the same with PSA's 3D padding (the grid padded to 21x48x80, one block per
    # PSABlock: 7 x 6 x 5 = 210 blocks of 384 slots)
    "wan720_psa3d": Config("wan720_psa3d", 8, 1, 40, 128, (21, 45, 80), (3, 8, 16), "bf16",
                           (0.9,), pe_scale="uniform", pad3d=True),
    # a small 3D-padded case with partial tiles on every axis
    "small_pad3d": Config("small_pad3d", 9, 1, 4, 64, (5, 7, 9), (2, 4, 4), "bf16", (0.9,),
                          pad3d=True),
    # 3D padding with 128-slot blocks (two 64-token sub-blocks; edge tiles hold
    # as few as 4 tokens, so whole sub-blocks are padding)
    "tiny_pad3d": Config("tiny_pad3d", 10, 1, 2, 128, (3, 9, 20), (2, 4, 16), "bf16", (0.9,),
                         pad3d=True),
    # the largest block count the attention and mask entry points accept: 4096
    # blocks of 64 tokens (262,144 tokens, one head)
    "maxnb": Config("maxnb", 11, 1, 1, 64, (16, 64, 256), (4, 4, 4), "bf16", (0.9,)),
    # more (batch, head) pairs than the work queues place by measured work
    # (2100 > 2048): a tiny grid, batch 2100, one head
    "manybh": Config("manybh", 12, 2100, 1, 64, (4, 8, 8), (4, 4, 4), "bf16", (0.9,)),
    # 700 (batch, head) pairs of two query groups each: the work queues cut each
    # pair into fewer runs (2048 / 700 = 2) so that all 1,400 runs are placed by work
    "midbh": Config("midbh", 13, 700, 1, 64, (4, 8, 16), (4, 4, 4), "bf16", (0.9,)),
    # two independent samples of the small shape in one call (batch > 1)
    "small_b2": Config("small_b2", 6, 2, 8, 64, (8, 16, 16), (4, 4, 4), "bf16", (0.9,),
                       pe_freq="per_head"),
}


def get_config(name):
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown config {name!r}; known: {sorted(CONFIGS)}") from None
