"""Plain, slow, fp64 CPU oracle of the block-sparse video attention path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the HIP library (no kernels, headers, helpers or tables); the only
thing both sides use is the seeded input generator ``svsa_synth``.

Every stage reads the *same* bf16 (or fp32) values as the GPU, widened
exactly to float64, and computes in float64 with NumPy.  Sources (web pages;
cited by title and section):

* [PSA]   "Parameterized Stripe Attention for Efficient Video Generation".
* [iCATS] "iCATS: Fast Video Generation via Interaction-Aware Sparse Attention
          and Timestep-Adaptive Sparsity" (paper summary page).
* [SPADE] "SPADE: An Input-Adaptive Sparse Attention Engine for Fast Video
          Diffusion Models Inference" (abstract page).
* [SVOO]  "Attention Sparsity is Input-Stable: Training-Free Sparse Attention
          for Video Generation via Offline Sparsity Profiling and Online QK
          Co-Clustering" (metadata page with harvested function names).

Readings taken where the pages are silent (each is pinned by a test):

* Blocks are consecutive Bk-token chunks of the tile-ordered sequence, Bk =
  tile volume, nb = ceil(N / Bk); only the tail of the sequence is padded.
  Partial edge tiles stay in place (tile grid walked row-major).
* A block summary is the mean over the block's valid tokens only.
* Block scores are a row softmax of pooled logits scaled by 1/sqrt(D) over
  all nb key blocks; no size weighting.
* Top-p keeps the shortest prefix of the score-descending order (ties: lower
  key index first) whose cumulative mass reaches p (>=); p >= 1 keeps all.
  The diagonal band |i - j| <= w - 1 is added afterwards and is not counted
  toward the mass.  Fixed mode keeps ceil(f_h * nb) blocks instead.
* Attention excludes padded keys (their logits are -inf) and leaves padded
  query rows unspecified (they are not compared).
* Stripe masks ([PSA] Alg. 1) are evaluated at tile granularity: a tile has
  coordinates (t', s') = (tile's t index, h index * nW + w index) in the tile
  grid (nT, nH, nW), the six parameters are in tile units (as PSA's search
  ranges are in PSABlock units), a stride <= 0 stands for infinity, and a
  query block keeps a key block when some tile of the first attends to some
  tile of the second.  The diagonal band of the top-p path can be added.
* 3D padding ([PSA] Sec. 4.1 / App. C.2: the latent grid is padded so that
  every PSABlock is full): every tile is its own block of Bk slots, nb =
  nT*nH*nW; its valid tokens fill the first slots (row-major (t, h, w) order)
  and the remaining slots are padding, excluded like the tail padding.  The
  order of tokens inside a block does not change any block-level quantity.
* Variable-size blocks from query / key clustering ([iCATS] Sec. 3.1, 4.1;
  [SVOO] "online bidirectional QK co-clustering"; the pages give the idea,
  not the algorithm).  Reading: replacing a query q by its centroid mu moves
  its logit against a key k by (q - mu).k, so the summed squared change over
  the keys is the quadratic form (q - mu)^T G (q - mu) with G = sum_k k k^T,
  approximated from the key clusters as G = sum_j n_j kappa_j kappa_j^T (and
  symmetrically for keys with the query clusters).  Clustering is Lloyd's
  k-means under that fixed metric: each iteration assigns every token to the
  centroid of least quadratic-form distance (ties: lowest index) and moves
  every non-empty centroid to the mean of its members (an empty one stays).
  G = I is plain feature-space k-means (the first sparse step).  Initial
  centroids and iteration counts are inputs.  Clusters are laid out one after
  another, each starting on a multiple of the alignment, members in natural
  order, padding zero.  Cluster scores are the row softmax over key clusters
  of scale * mu_i . kappa_j + ln n_j (the mass of n_j keys that all equal
  kappa_j; empty key clusters get none); top-p / fixed fraction as for
  blocks, no band.  A query token attends to every token of its cluster's
  kept key clusters.
* Tail merging ([iCATS] Sec. 4.3, App. E.1) of the query clusters of one
  head, given their kept key-cluster sets and the block size b: (1) clusters
  with identical kept sets merge into the lowest such index; (2) two rounds:
  every non-empty cluster with a tail (size mod b > 0) finds its nearest
  other such cluster by Jaccard similarity of the kept sets (ties: lowest
  index); mutually nearest pairs whose tails fit one block move the smaller
  tail (equal tails: the higher index's) -- the donor's last members in token
  order -- to the other cluster, whose kept set becomes the union.  Emptied
  clusters keep their index and occupy no rows.
* SNR-guided top-p ([iCATS] Sec. 4.2, App. A): the pages give the schedule's
  shape and its two parameters (pmin, tau) but no formula.  Reading: with the
  flow-matching noise level s (x = (1 - s) x0 + s eps), logSNR = 2 ln((1-s)/s)
  and w = sigmoid(-logSNR); steps before the first sparse one are dense
  (p = 1); later steps interpolate linearly in w from tau (first sparse step)
  to pmin (last step).  The formula itself is parity unpinned (the pins fix
  this reading, not the pages' unprinted formula).

parity pins: see tests/test_oracle_*.py; every public function is pinned.
"""
from math import ceil, sqrt

import numpy as np

__all__ = [
    "num_blocks", "tile_order", "permute_fwd", "permute_inv", "block_valid_counts",
    "pool", "block_logits", "block_scores", "select_row", "block_mask",
    "attention", "attention_rows", "dense_attention", "kept_flops", "widen",
    "psa_attends", "block_tiles", "stripe_row", "stripe_mask", "block_layout", "snr_top_p",
    "cluster_means", "quad_distances", "kmeans_assign", "kmeans", "cluster_metric",
    "cluster_layout", "cluster_permute", "cluster_unpermute", "cluster_scores", "cluster_mask",
    "cluster_attention_rows", "tail_merge",
]


def widen(x):
    """bf16 bit patterns (uint16) or float32 values -> float64, exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def num_blocks(N, Bk):
    """nb = ceil(N / Bk): the tail block holds the remainder."""
    return -(-N // Bk)


# --------------------------------------------------------------------------
# Stage 1: tile order.  [PSA] Sec. 3.2 "Efficient and Flexible Kernel": Q, K, V
# are reorganised from the (T, H, W) layout into a block-centric arrangement
# (T', H', W', b_t, b_h, b_w) so that every block is contiguous in memory.
# The natural index is i = t*H*W + h*W + w ([PSA] App. D, Prop. 1).  [SVOO]
# names the forward / inverse pair "token_reorder_to_frame_major" /
# "to_token_major".
# --------------------------------------------------------------------------
def tile_order(grid, tile):
    """pi: int64 [N]; pi[j] = natural index of the j-th token in tile order.

    Tiles are visited row-major over the tile grid (ceil(T/tt), ceil(H/th),
    ceil(W/tw)); tokens inside a tile row-major in (t, h, w).  Edge tiles are
    partial and keep their place.  Built as a lexicographic sort of the
    (tile coordinates, in-tile coordinates) key of every token.
    """
    T, H, W = grid
    tt, th, tw = tile
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    t, h, w = t.ravel(), h.ravel(), w.ravel()
    natural = (t * H + h) * W + w
    # np.lexsort sorts by the last key first.
    order = np.lexsort((w % tw, h % th, t % tt, w // tw, h // th, t // tt))
    return natural[order].astype(np.int64)


def permute_fwd(x, grid, tile, pad3d=False):
    """X'[..., j, :] = X[..., slot(j), :] for every valid slot j; padding slots
    are zero (see block_layout).

    x: [B, Hh, N, D] in natural order (any float dtype or bf16 bits).
    Returns float64 [B, Hh, nb*Bk, D].
    """
    xf = widen(x)
    B, Hh, N, D = xf.shape
    slots, _ = block_layout(grid, tile, pad3d)
    valid = slots >= 0
    assert int(valid.sum()) == N
    out = np.zeros((B, Hh, slots.size, D))
    out[:, :, valid, :] = xf[:, :, slots[valid], :]
    return out


def permute_inv(xp, grid, tile, pad3d=False):
    """O[..., slot(j), :] = O'[..., j, :] for every valid slot j (padding dropped)."""
    xf = widen(xp)
    N = int(np.prod(grid))
    slots, _ = block_layout(grid, tile, pad3d)
    valid = slots >= 0
    out = np.empty(xf.shape[:2] + (N, xf.shape[3]))
    out[:, :, slots[valid], :] = xf[:, :, valid, :]
    return out


def block_layout(grid, tile, pad3d=False):
    """(slots, counts): slots int64 [nb*Bk] = natural index of the token in each
    tiled slot or -1 for padding; counts int64 [nb] = valid tokens of each
    block (always the first slots of the block).

    pad3d=False: the tile order of tile_order(), cut into consecutive Bk-token
    blocks, padding only at the tail.  pad3d=True: one block per tile (tiles
    row-major over the tile grid), the tile's tokens first, padding after."""
    T, H, W = grid
    tt, th, tw = tile
    N, Bk = T * H * W, tt * th * tw
    if not pad3d:
        nb = num_blocks(N, Bk)
        slots = np.full(nb * Bk, -1, dtype=np.int64)
        slots[:N] = tile_order(grid, tile)
        return slots, block_valid_counts(N, Bk)
    nT, nH, nW = -(-T // tt), -(-H // th), -(-W // tw)
    nb = nT * nH * nW
    slots = np.full(nb * Bk, -1, dtype=np.int64)
    counts = np.zeros(nb, dtype=np.int64)
    for a in range(nT):
        for b in range(nH):
            for c in range(nW):
                k = (a * nH + b) * nW + c
                t, h, w = np.meshgrid(np.arange(a * tt, min((a + 1) * tt, T)),
                                      np.arange(b * th, min((b + 1) * th, H)),
                                      np.arange(c * tw, min((c + 1) * tw, W)), indexing="ij")
                nat = ((t * H + h) * W + w).ravel()
                slots[k * Bk: k * Bk + nat.size] = nat
                counts[k] = nat.size
    return slots, counts


def block_valid_counts(N, Bk):
    """n_i: number of real (non-padding) tokens in each block."""
    nb = num_blocks(N, Bk)
    n = np.full(nb, Bk, dtype=np.int64)
    n[-1] = N - (nb - 1) * Bk
    return n


# --------------------------------------------------------------------------
# Stage 2: block summaries.  [SPADE] abstract: dynamic masks are expressed as
# a "Summarizer" followed by an "Estimator"; [iCATS] Sec. 4: region
# importance is scored at the level of token groups.  Reading: the summary of
# a block is the arithmetic mean of its valid tokens.
# --------------------------------------------------------------------------
def pool(xp, N, Bk, counts=None):
    """Xbar_i = (1/n_i) * sum of the valid rows of block i.  -> [B, Hh, nb, D].

    counts: valid tokens per block (the first rows of each block); default the
    tail-padded layout's."""
    xf = widen(xp)
    B, Hh, Np, D = xf.shape
    if counts is None:
        counts = block_valid_counts(N, Bk)
    nb = len(counts)
    assert Np == nb * Bk
    out = np.empty((B, Hh, nb, D))
    for i in range(nb):
        rows = xf[:, :, i * Bk: i * Bk + counts[i], :]
        out[:, :, i, :] = rows.sum(axis=2) / counts[i]
    return out


# --------------------------------------------------------------------------
# Stage 3a: block-to-block importance, softmax(Qbar Kbar^T / sqrt(d)), one row
# per query block ([SPADE] "Estimator"; [iCATS] Sec. 4 cluster-level scores).
# --------------------------------------------------------------------------
def block_logits(qbar, kbar, scale):
    """L[b, h, i, j] = scale * <Qbar_i, Kbar_j>  (float64)."""
    return np.matmul(qbar, np.swapaxes(kbar, -1, -2)) * scale


def block_scores(qbar, kbar, scale):
    """S[b, h, i, :] = exp(L - max L) / sum exp(L - max L) over all nb blocks."""
    L = block_logits(qbar, kbar, scale)
    e = np.exp(L - L.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


# --------------------------------------------------------------------------
# Stage 3b: selection.  [iCATS] abstract and Sec. 3.2: a fixed top-p rule keeps
# the most important key regions until their cumulative importance reaches p.
# The band width follows the width convention of [PSA] Alg. 1 (a distance d
# is inside a band of width w when d <= w - 1).  The fixed-fraction mode is
# the per-layer intrinsic pruning level of [SVOO] (abstract).
# --------------------------------------------------------------------------
def select_row(s_row, i, band, top_p=None, keep_frac=None):
    """Kept key blocks of query block i, ascending.

    s_row: float64 [nb] block scores of the row.  Exactly one of top_p /
    keep_frac is given (both float32 values, widened exactly).
    """
    nb = s_row.shape[0]
    # score-descending, ties by ascending key index (stable sort of -s)
    order = np.argsort(-s_row, kind="stable")
    if keep_frac is not None:
        k = int(ceil(float(np.float32(keep_frac)) * nb))
        k = min(max(k, 1), nb)
    else:
        p = float(np.float32(top_p))
        if p >= 1.0:
            k = nb
        else:
            csum = np.cumsum(s_row[order])       # csum[r] = mass of the top r+1
            # smallest k >= 1 whose top-k mass reaches p
            reached = np.nonzero(csum >= p)[0]
            k = int(reached[0]) + 1 if reached.size else nb
    kept = np.zeros(nb, dtype=bool)
    kept[order[:k]] = True
    j = np.arange(nb)
    kept |= np.abs(j - i) <= band - 1
    return np.nonzero(kept)[0].astype(np.int32)


def block_mask(S, band, top_p=None, keep_frac=None):
    """CSR of kept blocks over rows r = (b*Hh + h)*nb + i.

    S: [B, Hh, nb, nb] block scores; top_p / keep_frac: per-head arrays (one is
    None).  Returns (row_ptr int64 [B*Hh*nb+1], col_idx int32 [nnz]).
    """
    B, Hh, nb, _ = S.shape
    counts, cols = [], []
    for b in range(B):
        for h in range(Hh):
            for i in range(nb):
                if keep_frac is not None:
                    c = select_row(S[b, h, i], i, band, keep_frac=keep_frac[h])
                else:
                    c = select_row(S[b, h, i], i, band, top_p=top_p[h])
                cols.append(c)
                counts.append(c.size)
    row_ptr = np.zeros(len(counts) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.concatenate(cols).astype(np.int32) if cols else np.zeros(0, np.int32)
    return row_ptr, col_idx


# --------------------------------------------------------------------------
# Stage 4: block-sparse attention over the kept blocks.  [PSA] App. B, Alg. 2:
# per query block, S = Q K^T over each listed KV block, invalid (padded)
# positions set to -inf, safe softmax, P V accumulated into the output.
# The oracle evaluates the same quantity directly: one softmax over the union
# of the kept blocks' valid keys (what the blockwise accumulation equals).
# --------------------------------------------------------------------------
def attention_rows(qp, kp, vp, b, h, i, cols, N, Bk, scale, counts=None):
    """Output rows of query block i of (b, h) as float64 [n_i, D].

    qp, kp, vp: tiled [B, Hh, nb*Bk, D] arrays (bf16 bits or float).
    cols: kept key blocks of this row.  counts: valid tokens per block (a
    prefix of each block); default the tail-padded layout's.
    """
    if counts is None:
        counts = block_valid_counts(N, Bk)
    nb = len(counts)
    n_i = int(counts[i])
    q = widen(qp[b, h, i * Bk: i * Bk + n_i])
    keys = np.concatenate([np.arange(j * Bk, j * Bk + int(counts[j])) for j in cols])
    assert all(0 <= j < nb for j in cols)
    k = widen(kp[b, h, keys])
    v = widen(vp[b, h, keys])
    logits = (q @ k.T) * scale
    wgt = np.exp(logits - logits.max(axis=1, keepdims=True))
    wgt /= wgt.sum(axis=1, keepdims=True)
    return wgt @ v


def attention(qp, kp, vp, row_ptr, col_idx, N, Bk, scale, rows=None, counts=None):
    """O' (tiled, float64 [B, Hh, nb*Bk, D]) for the listed query blocks.

    rows: optional iterable of (b, h, i); default all.  Rows not computed and
    padded query rows are NaN.
    """
    B, Hh, Np, D = qp.shape
    if counts is None:
        counts = block_valid_counts(N, Bk)
    nb = len(counts)
    out = np.full((B, Hh, Np, D), np.nan)
    if rows is None:
        rows = [(b, h, i) for b in range(B) for h in range(Hh) for i in range(nb)]
    for (b, h, i) in rows:
        r = (b * Hh + h) * nb + i
        cols = col_idx[row_ptr[r]: row_ptr[r + 1]]
        n_i = int(counts[i])
        out[b, h, i * Bk: i * Bk + n_i] = attention_rows(qp, kp, vp, b, h, i, cols, N, Bk, scale,
                                                         counts)
    return out


def dense_attention(q, k, v, scale):
    """softmax(Q K^T * scale) V over all N keys, natural order, float64."""
    qf, kf, vf = widen(q), widen(k), widen(v)
    logits = np.matmul(qf, np.swapaxes(kf, -1, -2)) * scale
    wgt = np.exp(logits - logits.max(axis=-1, keepdims=True))
    wgt /= wgt.sum(axis=-1, keepdims=True)
    return np.matmul(wgt, vf)


def kept_flops(row_ptr, col_idx, N, Bk, D, nrows_per_head=None, counts=None):
    """Algorithmic FLOPs of block-sparse attention: 4*D*sum_(i,j kept) n_i*n_j.

    This is the accounting of [PSA] Table 2, whose dense rows equal 4*N^2*D*heads.
    """
    n = block_valid_counts(N, Bk) if counts is None else np.asarray(counts)
    nb = len(n)
    total = 0
    nrows = len(row_ptr) - 1
    for r in range(nrows):
        i = r % nb
        cols = col_idx[row_ptr[r]: row_ptr[r + 1]]
        total += int(n[i]) * int(n[cols].sum())
    return 4 * D * total


# --------------------------------------------------------------------------
# Stripe masks.  [PSA] Sec. 3.2 "Unified Representation": six integers
# M(Tw, To, Ts, Sw, So, Ss) give the width, offset and stride of the
# inter-frame and intra-frame diagonal bands; [PSA] Alg. 1 ("PSA Mask
# Definition") decides whether position i attends to position j from
# (t, s) = (i div (H*W), i mod (H*W)); masking is applied per PSABlock.
# Reading: positions are tiles of the tile grid, so H*W becomes nH*nW; an
# infinite stride (here any value <= 0) reduces that axis to one band.
# --------------------------------------------------------------------------
def _band_cond(delta, width, offset, stride):
    d = np.abs(delta - offset)
    if stride > 0:
        d = d % stride
    return d <= width - 1


def psa_attends(ti, si, tj, sj, params):
    """[PSA] Alg. 1 on tile coordinates: inter-frame condition on the frame
    (tile-slab) distance, then intra-frame condition on the in-frame distance.
    Arrays broadcast; params = (Tw, To, Ts, Sw, So, Ss)."""
    Tw, To, Ts, Sw, So, Ss = (int(x) for x in params)
    inter = _band_cond(np.asarray(tj) - np.asarray(ti), Tw, To, Ts)
    intra = _band_cond(np.asarray(sj) - np.asarray(si), Sw, So, Ss)
    return inter & intra


def block_tiles(grid, tile, pad3d=False):
    """For every block, the distinct tiles its valid tokens belong to, as a
    list of (t', s') int64 arrays (s' = h' * nW + w')."""
    T, H, W = grid
    tt, th, tw = tile
    nH, nW = -(-H // th), -(-W // tw)
    if pad3d:   # one block per tile
        nT = -(-T // tt)
        return [(np.array([k // (nH * nW)]), np.array([k % (nH * nW)])) for k in range(nT * nH * nW)]
    N = T * H * W
    Bk = tt * th * tw
    nb = num_blocks(N, Bk)
    pi = tile_order(grid, tile)
    t, rem = np.divmod(pi, H * W)
    h, w = np.divmod(rem, W)
    tp, sp = t // tt, (h // th) * nW + (w // tw)
    out = []
    for b in range(nb):
        sl = slice(b * Bk, min((b + 1) * Bk, N))
        pairs = np.unique(np.stack([tp[sl], sp[sl]], axis=1), axis=0)
        out.append((pairs[:, 0], pairs[:, 1]))
    return out


def stripe_row(tiles, i, params, band):
    """Kept key blocks of query block i (ascending): some tile of block i
    attends to some tile of block j under [PSA] Alg. 1, or |i - j| <= band-1."""
    nb = len(tiles)
    ti, si = tiles[i]
    kept = np.zeros(nb, dtype=bool)
    for j in range(nb):
        tj, sj = tiles[j]
        kept[j] = bool(np.any(psa_attends(ti[:, None], si[:, None], tj[None, :], sj[None, :],
                                          params)))
    kept |= np.abs(np.arange(nb) - i) <= band - 1
    return np.nonzero(kept)[0].astype(np.int32)


def stripe_mask(grid, tile, params, band, batch=1, rows=None, pad3d=False):
    """CSR over rows r = (b*Hh + h)*nb + i with the stripe mask of head h
    (params: [Hh, 6]).  rows: optional list of (b, h, i) to evaluate; then the
    result is a dict {(b, h, i): cols} instead of a CSR."""
    tiles = block_tiles(grid, tile, pad3d)
    nb = len(tiles)
    params = np.asarray(params, dtype=np.int64)
    Hh = params.shape[0]
    if rows is not None:
        return {(b, h, i): stripe_row(tiles, i, params[h], band) for (b, h, i) in rows}
    counts, cols = [], []
    for b in range(batch):
        for h in range(Hh):
            for i in range(nb):
                c = stripe_row(tiles, i, params[h], band)
                cols.append(c)
                counts.append(c.size)
    row_ptr = np.zeros(len(counts) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.concatenate(cols).astype(np.int32) if cols else np.zeros(0, np.int32)
    return row_ptr, col_idx


# --------------------------------------------------------------------------
# SNR-guided sparsity.  [iCATS] Sec. 4.2 and App. A: top-p changes over the
# denoising steps as a smooth function of the log signal-to-noise ratio of
# the noise schedule -- dense before the first sparse step, lowered through
# the middle of denoising, nearly flat early and late; pmin and tau per model
# in App. B.  Reading (the formula is not on the pages): w = sigmoid(-logSNR),
# linear in w between tau at the first sparse step and pmin at the last.
# --------------------------------------------------------------------------
def snr_top_p(sigmas, first_sparse, p_min, tau):
    """float64 [steps] top-p per denoising step.

    sigmas: flow-matching noise levels s_k in [0, 1] (x = (1 - s) x0 + s eps).
    Steps k < first_sparse are dense (1.0)."""
    s = np.asarray(sigmas, dtype=np.float64)
    steps = s.size
    with np.errstate(divide="ignore"):
        log_snr = 2.0 * (np.log(1.0 - s) - np.log(s))       # -inf at s = 1, +inf at s = 0
    w = 1.0 / (1.0 + np.exp(log_snr))                       # sigmoid(-logSNR)
    p = np.ones(steps)
    if first_sparse >= steps:
        return p
    w_first, w_last = w[first_sparse], w[steps - 1]
    for k in range(first_sparse, steps):
        u = 1.0 if w_first == w_last else (w[k] - w_last) / (w_first - w_last)
        p[k] = p_min + (tau - p_min) * min(1.0, max(0.0, u))
    return p


# --------------------------------------------------------------------------
# Variable-size blocks: query / key clustering.  [iCATS] Sec. 3.1 and 4.1:
# clustering should minimise the error of the query-key interactions, which
# is written as a quadratic form in the feature space so that the full
# interaction matrix is never built; query clusters start in plain feature
# space and later use the key clusters' metric, and the query clusters in
# turn guide the key clustering.  [SVOO]: online bidirectional QK
# co-clustering into blocks.  The steps below are this module's reading.
# --------------------------------------------------------------------------
def cluster_means(x, labels, C):
    """(means float64 [B, Hh, C, D], sizes int64 [B, Hh, C]): the mean of each
    cluster's member tokens (NaN rows for empty clusters)."""
    xf = widen(x)
    B, Hh, N, D = xf.shape
    lab = np.asarray(labels)
    means = np.full((B, Hh, C, D), np.nan)
    sizes = np.zeros((B, Hh, C), np.int64)
    for b in range(B):
        for h in range(Hh):
            for c in range(C):
                members = xf[b, h, lab[b, h] == c]
                sizes[b, h, c] = members.shape[0]
                if members.shape[0]:
                    means[b, h, c] = members.sum(axis=0) / members.shape[0]
    return means, sizes


def quad_distances(x, cents, G=None):
    """float64 [N, C]: (x_n - c)^T G (x_n - c) for one head (G = I if None).

    x: [N, D] tokens, cents: [C, D]."""
    xf = widen(x)
    c = np.asarray(cents, dtype=np.float64)
    diff = xf[:, None, :] - c[None, :, :]                 # [N, C, D]
    if G is None:
        return np.einsum("ncd,ncd->nc", diff, diff)
    return np.einsum("ncd,de,nce->nc", diff, np.asarray(G, np.float64), diff)


def kmeans_assign(x, cents, G=None):
    """int32 [N]: index of the centroid of least quadratic-form distance
    (lowest index among equal distances)."""
    return np.argmin(quad_distances(x, cents, G), axis=1).astype(np.int32)


def kmeans(x, cents0, iters, G=None):
    """Lloyd iterations for one head: assign, then move every non-empty
    centroid to its members' mean.  Returns (centroids float64 [C, D], sizes
    int64 [C], labels int32 [N] of the last assignment); the centroids are the
    means of those labels (empty clusters keep their previous centroid)."""
    xf = widen(x)
    c = np.array(cents0, dtype=np.float64)
    C = c.shape[0]
    labels = np.zeros(xf.shape[0], np.int32)
    sizes = np.zeros(C, np.int64)
    for _ in range(iters):
        labels = kmeans_assign(xf, c, G)
        m, sz = cluster_means(xf[None, None], labels[None, None], C)
        sizes = sz[0, 0]
        keep = sizes > 0
        c[keep] = m[0, 0, keep]
    return c, sizes, labels


def cluster_metric(cents, sizes):
    """G = sum_c n_c c c^T (float64 [D, D]) for one head: the quadratic form
    that the clusters of one side induce on the other side's tokens."""
    c = np.asarray(cents, dtype=np.float64)
    n = np.asarray(sizes, dtype=np.float64)
    return (c * n[:, None]).T @ c


def cluster_layout(labels, C, align):
    """Padded layout of one head's clusters.

    Returns (start int64 [C+1], slot int64 [N], token int64 [start[C]]):
    cluster c owns slots start[c] .. start[c] + n_c - 1 (its members in
    ascending natural index), start[0] = 0 and start[c+1] = start[c] +
    align * ceil(n_c / align); slot[t] = the slot of token t; token[s] = the
    token in slot s or -1 for padding."""
    lab = np.asarray(labels)
    sizes = np.bincount(lab, minlength=C)[:C]
    start = np.zeros(C + 1, np.int64)
    start[1:] = np.cumsum(-(-sizes // align) * align)
    slot = np.empty(lab.size, np.int64)
    token = np.full(int(start[C]), -1, np.int64)
    for c in range(C):
        members = np.nonzero(lab == c)[0]            # ascending natural index
        slot[members] = start[c] + np.arange(members.size)
        token[start[c]: start[c] + members.size] = members
    return start, slot, token


def cluster_permute(x, token):
    """X'[s] = X[token[s]] (zero for padding slots) for one head [N, D] -> [L, D]."""
    xf = widen(x)
    out = np.zeros((token.size, xf.shape[1]))
    ok = token >= 0
    out[ok] = xf[token[ok]]
    return out


def cluster_unpermute(xp, slot):
    """O[t] = O'[slot[t]] for one head."""
    return widen(xp)[np.asarray(slot)]


def cluster_scores(qbar, kbar, ksizes, scale):
    """float64 [nq, nk] for one head: row softmax over the key clusters of
    scale * qbar_i . kbar_j + ln n_j; empty key clusters score 0."""
    n = np.asarray(ksizes)
    # an empty key cluster has no tokens (its centroid may be undefined): no mass
    kb = np.where((n > 0)[:, None], np.asarray(kbar, np.float64), 0.0)
    L = (np.asarray(qbar, np.float64) @ kb.T) * scale
    L = np.where(n > 0, L + np.log(np.maximum(n, 1).astype(np.float64))[None, :], -np.inf)
    w = np.exp(L - L.max(axis=1, keepdims=True))
    return w / w.sum(axis=1, keepdims=True)


def cluster_mask(S, top_p=None, keep_frac=None):
    """CSR over rows r = (b*Hh + h)*nq + i of kept key clusters (no band).

    S: [B, Hh, nq, nk] cluster scores; top_p / keep_frac per head."""
    B, Hh, nq, nk = S.shape
    counts, cols = [], []
    for b in range(B):
        for h in range(Hh):
            for i in range(nq):
                if keep_frac is not None:
                    c = select_row(S[b, h, i], i, 0, keep_frac=keep_frac[h])
                else:
                    c = select_row(S[b, h, i], i, 0, top_p=top_p[h])
                cols.append(c)
                counts.append(c.size)
    row_ptr = np.zeros(len(counts) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.concatenate(cols).astype(np.int32) if cols else np.zeros(0, np.int32)
    return row_ptr, col_idx


def cluster_attention_rows(q, k, v, qlab, klab, i, cols, scale):
    """Attention of the query tokens of cluster i (one head, natural order)
    over every key token of the listed key clusters: (tokens int64, float64
    [m_i, D]).  q, k, v: [N, D]; qlab, klab: [N] cluster labels."""
    toks = np.nonzero(np.asarray(qlab) == i)[0]
    keys = np.nonzero(np.isin(np.asarray(klab), np.asarray(cols)))[0]
    if toks.size == 0:
        return toks, np.zeros((0, widen(q).shape[1]))
    qf, kf, vf = widen(q)[toks], widen(k)[keys], widen(v)[keys]
    logits = (qf @ kf.T) * scale
    wgt = np.exp(logits - logits.max(axis=1, keepdims=True))
    wgt /= wgt.sum(axis=1, keepdims=True)
    return toks, wgt @ vf


# --------------------------------------------------------------------------
# Tail merging.  [iCATS] Sec. 4.3 and App. E.1: query clusters that attend to
# the same key clusters merge without changing the attention pattern; then,
# over two rounds, tail tokens move between mutually closest clusters whose
# tails fit one block, the receiving cluster taking the union of both masks.
# The similarity, the choice of donor and of its tail tokens are this
# module's reading (see the header).
# --------------------------------------------------------------------------
def tail_merge(labels, kept, block, rounds=2):
    """One head.  labels: int [N] query cluster of each token; kept: bool
    [C, nk] kept key clusters of each query cluster; block: tokens per query
    block.  Returns (labels int32 [N], kept bool [C, nk], sizes int64 [C])."""
    lab = np.array(labels, dtype=np.int64)
    R = np.array(kept, dtype=bool)
    C = R.shape[0]
    sizes = np.bincount(lab, minlength=C)[:C]
    rep = np.arange(C)
    for i in range(C):
        if sizes[i] == 0:
            continue
        for j in range(i):
            if sizes[j] > 0 and np.array_equal(R[j], R[i]):
                rep[i] = j
                break
    lab = rep[lab]
    for _ in range(rounds):
        sizes = np.bincount(lab, minlength=C)[:C]
        tail = sizes % block
        part = [i for i in range(C) if sizes[i] > 0 and tail[i] > 0]
        nearest = {}
        for i in part:
            best, bi, bu = -1, 0, 1
            for j in part:
                if j == i:
                    continue
                inter = int(np.sum(R[i] & R[j]))
                uni = max(int(np.sum(R[i] | R[j])), 1)
                if best < 0 or inter * bu > bi * uni:      # strictly more similar
                    best, bi, bu = j, inter, uni
            if best >= 0:
                nearest[i] = best
        moves = []
        for i in part:
            j = nearest.get(i, -1)
            if j > i and nearest.get(j, -1) == i and tail[i] + tail[j] <= block:
                donor, recv = (i, j) if tail[i] < tail[j] else (j, i)
                moves.append((donor, recv))
        for donor, recv in moves:
            members = np.nonzero(lab == donor)[0]
            lab[members[members.size - tail[donor]:]] = recv
            R[recv] |= R[donor]
    sizes = np.bincount(lab, minlength=C)[:C]
    return lab.astype(np.int32), R, sizes
