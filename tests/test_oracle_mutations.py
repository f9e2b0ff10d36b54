"""Each pin must catch a plausible mistake: plant one in the oracle (on the CPU,
via monkeypatch) and check that the corresponding pin test fails."""
import numpy as np
import pytest

from oracle import svsa_oracle as orc
import tests.test_oracle_attention as ta
import tests.test_oracle_permute as tp
import tests.test_oracle_select as ts
import tests.test_oracle_stripe as tst
import tests.test_oracle_pad3d as tpd
import tests.test_oracle_snr as tsnr
import tests.test_oracle_cluster as tcl
import tests.test_oracle_tail as ttl

_SNR = orc.snr_top_p   # the unmutated schedule, for mutations built on top of it
_MEANS = orc.cluster_means
_ASSIGN = orc.kmeans_assign
_LAYOUT = orc.cluster_layout
_ROWS = orc.cluster_attention_rows


def _scores_no_scale(qbar, kbar, scale):
    L = np.matmul(qbar, np.swapaxes(kbar, -1, -2))
    e = np.exp(L - L.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _scores_transposed(qbar, kbar, scale):
    L = np.matmul(kbar, np.swapaxes(qbar, -1, -2)) * scale
    e = np.exp(L - L.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _pool_divide_by_bk(xp, N, Bk):
    xf = orc.widen(xp)
    B, Hh, Np, D = xf.shape
    return xf.reshape(B, Hh, Np // Bk, Bk, D).sum(axis=3) / Bk


def _tile_order_swapped(grid, tile):
    T, H, W = grid
    tt, th, tw = tile
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    t, h, w = t.ravel(), h.ravel(), w.ravel()
    order = np.lexsort((h % th, w % tw, t % tt, w // tw, h // th, t // tt))
    return ((t * H + h) * W + w)[order]


_orig_select = orc.select_row


def _select_band_off_by_one(s_row, i, band, top_p=None, keep_frac=None):
    return _orig_select(s_row, i, band + 1, top_p=top_p, keep_frac=keep_frac)


def _select_strict(s_row, i, band, top_p=None, keep_frac=None):
    if top_p is None:
        return _orig_select(s_row, i, band, keep_frac=keep_frac)
    order = np.argsort(-s_row, kind="stable")
    csum = np.cumsum(s_row[order])
    k = int(np.nonzero(csum > float(np.float32(top_p)))[0][0]) + 1 if np.any(
        csum > float(np.float32(top_p))) else s_row.size
    kept = np.zeros(s_row.size, bool)
    kept[order[:k]] = True
    kept |= np.abs(np.arange(s_row.size) - i) <= band - 1
    return np.nonzero(kept)[0]



def _select_fixed_variant(count):
    """Fixed-fraction selection with another block count rule."""
    def select(s_row, i, band, top_p=None, keep_frac=None):
        if keep_frac is None:
            return _orig_select(s_row, i, band, top_p=top_p)
        nb = s_row.size
        k = min(max(count(np.float32(keep_frac), nb), 1), nb)
        kept = np.zeros(nb, bool)
        kept[np.argsort(-s_row, kind="stable")[:k]] = True
        kept |= np.abs(np.arange(nb) - i) <= band - 1
        return np.nonzero(kept)[0]
    select.__name__ = f"_select_fixed_{count.__name__}"
    return select


def float32_product(f, nb):
    return int(np.ceil(np.float32(f) * np.float32(nb)))


def nearest(f, nb):
    return int(round(float(f) * nb))

def _attention_rows_with_pads(qp, kp, vp, b, h, i, cols, N, Bk, scale, counts=None):
    n_i = min(Bk, N - i * Bk)
    q = orc.widen(qp[b, h, i * Bk: i * Bk + n_i])
    keys = np.concatenate([np.arange(j * Bk, (j + 1) * Bk) for j in cols])
    k, v = orc.widen(kp[b, h, keys]), orc.widen(vp[b, h, keys])
    lg = q @ k.T * scale
    w = np.exp(lg - lg.max(1, keepdims=True))
    return (w / w.sum(1, keepdims=True)) @ v


def _attention_rows_v_is_k(qp, kp, vp, b, h, i, cols, N, Bk, scale, counts=None):
    return _orig_rows(qp, kp, kp, b, h, i, cols, N, Bk, scale, counts)



def _attention_rows_no_scale(qp, kp, vp, b, h, i, cols, N, Bk, scale, counts=None):
    return _orig_rows(qp, kp, vp, b, h, i, cols, N, Bk, 1.0, counts)

_orig_rows = orc.attention_rows


_orig_pool = orc.pool


def _pool_ignores_counts(xp, N, Bk, counts=None):
    xf = orc.widen(xp)
    nb = xf.shape[2] // Bk
    return xf.reshape(xf.shape[0], xf.shape[1], nb, Bk, xf.shape[3]).mean(axis=3)


def _rows_ignore_counts(qp, kp, vp, b, h, i, cols, N, Bk, scale, counts=None):
    q = orc.widen(qp[b, h, i * Bk: i * Bk + int(counts[i])])
    keys = np.concatenate([np.arange(j * Bk, (j + 1) * Bk) for j in cols])
    lg = q @ orc.widen(kp[b, h, keys]).T * scale
    w = np.exp(lg - lg.max(1, keepdims=True))
    return (w / w.sum(1, keepdims=True)) @ orc.widen(vp[b, h, keys])


_orig_layout = orc.block_layout


def _layout_pads_in_place(grid, tile, pad3d=False):
    if not pad3d:
        return _orig_layout(grid, tile, pad3d)
    T, H, W = grid
    tt, th, tw = tile
    nT, nH, nW = -(-T // tt), -(-H // th), -(-W // tw)
    Bk = tt * th * tw
    slots = np.full(nT * nH * nW * Bk, -1, dtype=np.int64)
    counts = np.zeros(nT * nH * nW, dtype=np.int64)
    for a in range(nT):
        for b in range(nH):
            for c in range(nW):
                k = (a * nH + b) * nW + c
                for x in range(Bk):   # slot x <-> in-tile (t, h, w), padding where off-grid
                    t, h, w = a * tt + x // (th * tw), b * th + (x // tw) % th, c * tw + x % tw
                    if t < T and h < H and w < W:
                        slots[k * Bk + x] = (t * H + h) * W + w
                        counts[k] += 1
    return slots, counts


_orig_band = orc._band_cond


def _band_wider(delta, width, offset, stride):
    return _orig_band(delta, width + 1, offset, stride)


def _band_no_stride(delta, width, offset, stride):
    return _orig_band(delta, width, offset, 0)


def _attends_reversed(ti, si, tj, sj, params):
    Tw, To, Ts, Sw, So, Ss = (int(x) for x in params)
    return (orc._band_cond(np.asarray(ti) - np.asarray(tj), Tw, To, Ts)
            & orc._band_cond(np.asarray(si) - np.asarray(sj), Sw, So, Ss))


def _block_tiles_nh(grid, tile, pad3d=False):
    T, H, W = grid
    tt, th, tw = tile
    nH = -(-H // th)
    N = T * H * W
    Bk = tt * th * tw
    pi = orc.tile_order(grid, tile)
    t, rem = np.divmod(pi, H * W)
    h, w = np.divmod(rem, W)
    tp, sp = t // tt, (h // th) * nH + (w // tw)
    out = []
    for b in range(-(-N // Bk)):
        sl = slice(b * Bk, min((b + 1) * Bk, N))
        pairs = np.unique(np.stack([tp[sl], sp[sl]], axis=1), axis=0)
        out.append((pairs[:, 0], pairs[:, 1]))
    return out

def _snr_linear_in_log_snr(sigmas, first_sparse, p_min, tau):
    # interpolates in logSNR itself instead of sigmoid(-logSNR)
    s = np.asarray(sigmas, float)
    with np.errstate(divide="ignore"):
        lam = 2.0 * (np.log(1.0 - s) - np.log(s))
    p = np.ones(s.size)
    for k in range(first_sparse, s.size):
        u = (lam[k] - lam[-1]) / (lam[first_sparse] - lam[-1])
        p[k] = p_min + (tau - p_min) * min(1.0, max(0.0, u))
    return p


def _snr_unsquared(sigmas, first_sparse, p_min, tau):
    # SNR = (1 - s) / s (amplitude ratio) instead of its square: w = s
    s = np.asarray(sigmas, float)
    p = np.ones(s.size)
    for k in range(first_sparse, s.size):
        u = 1.0 if s[first_sparse] == s[-1] else (s[k] - s[-1]) / (s[first_sparse] - s[-1])
        p[k] = p_min + (tau - p_min) * min(1.0, max(0.0, u))
    return p


def _snr_no_warmup(sigmas, first_sparse, p_min, tau):
    return _SNR(sigmas, 0, p_min, tau)


def _kmeans_empty_becomes_nan(x, cents0, iters, G=None):
    xf = orc.widen(x)
    c = np.array(cents0, dtype=np.float64)
    labels = np.zeros(xf.shape[0], np.int32)
    sizes = np.zeros(c.shape[0], np.int64)
    for _ in range(iters):
        labels = _ASSIGN(xf, c, G)
        m, sz = _MEANS(xf[None, None], labels[None, None], c.shape[0])
        c, sizes = m[0, 0], sz[0, 0]
    return c, sizes, labels


def _quad_ignores_metric(x, cents, G=None):
    diff = orc.widen(x)[:, None, :] - np.asarray(cents, np.float64)[None]
    return np.einsum("ncd,ncd->nc", diff, diff)


def _scores_without_size(qbar, kbar, ksizes, scale):
    L = (np.asarray(qbar, np.float64) @ np.asarray(kbar, np.float64).T) * scale
    w = np.exp(L - L.max(axis=1, keepdims=True))
    return w / w.sum(axis=1, keepdims=True)


def _layout_unpadded(labels, C, align):
    return _LAYOUT(labels, C, 1)


def _metric_without_sizes(cents, sizes):
    c = np.asarray(cents, np.float64)
    return c.T @ c


def _cluster_rows_query_labels(q, k, v, qlab, klab, i, cols, scale):
    return _ROWS(q, k, v, qlab, qlab, i, cols, scale)


def _tail_variant(one_sided=False, big_donor=False, no_union=False, head=False):
    def fn(labels, kept, block, rounds=2):
        lab = np.array(labels, dtype=np.int64)
        R = np.array(kept, dtype=bool)
        C = R.shape[0]
        sizes = np.bincount(lab, minlength=C)[:C]
        rep = np.arange(C)
        for i in range(C):
            for j in range(i):
                if sizes[i] > 0 and sizes[j] > 0 and np.array_equal(R[j], R[i]):
                    rep[i] = j
                    break
        lab = rep[lab]
        for _ in range(rounds):
            sizes = np.bincount(lab, minlength=C)[:C]
            tail = sizes % block
            part = [i for i in range(C) if sizes[i] > 0 and tail[i] > 0]
            near = {}
            for i in part:
                cand = [(-(np.sum(R[i] & R[j]) / max(np.sum(R[i] | R[j]), 1)), j)
                        for j in part if j != i]
                if cand:
                    near[i] = min(cand)[1]
            moves, used = [], set()
            for i in part:
                j = near.get(i, -1)
                ok = j >= 0 and (one_sided or (j > i and near.get(j, -1) == i))
                if ok and i not in used and j not in used and tail[i] + tail[j] <= block:
                    small = (i, j) if tail[i] < tail[j] else (j, i)
                    moves.append(small[::-1] if big_donor else small)
                    used |= {i, j}
            for donor, recv in moves:
                members = np.nonzero(lab == donor)[0]
                take = members[:tail[donor]] if head else members[members.size - tail[donor]:]
                lab[take] = recv
                if not no_union:
                    R[recv] |= R[donor]
        return lab.astype(np.int32), R, np.bincount(lab, minlength=C)[:C]
    return fn


MUTATIONS = [
    ("block_scores", _scores_no_scale, ts.test_scores_closed_form_one_channel, ()),
    ("block_scores", _scores_transposed, ts.test_scores_closed_form_one_channel, ()),
    ("pool", _pool_divide_by_bk, tp.test_pool_tail_uses_valid_count_and_constant_stays_constant, ()),
    ("tile_order", _tile_order_swapped, tp.test_tile_order_worked_example, ("golden",)),
    ("select_row", _select_band_off_by_one, ts.test_band_width, ()),
    ("select_row", _select_strict, ts.test_topp_reaching_p_exactly_is_inclusive, ()),
    ("select_row", _select_fixed_variant(float32_product),
     ts.test_fixed_fraction_count_uses_the_float32_fraction, ()),
    ("select_row", _select_fixed_variant(nearest),
     ts.test_fixed_fraction_count_uses_the_float32_fraction, ()),
    ("attention_rows", _attention_rows_with_pads, ta.test_padded_keys_are_excluded, ()),
    ("attention_rows", _attention_rows_with_pads,
     ta.test_sparse_row_closed_form_two_kept_blocks_with_a_tail, ()),
    ("attention_rows", _attention_rows_no_scale,
     ta.test_sparse_row_closed_form_two_kept_blocks_with_a_tail, ()),
    ("attention_rows", _attention_rows_v_is_k, ta.test_all_blocks_kept_equals_dense_sdpa,
     ("grid_tile",)),
    ("_band_cond", _band_wider, tst.test_stripe_svg_special_case_is_a_plain_window, ()),
    ("_band_cond", _band_no_stride, tst.test_stripe_stride_repeats_the_band, ()),
    ("psa_attends", _attends_reversed, tst.test_stripe_offset_direction, ()),
    ("block_tiles", _block_tiles_nh, tst.test_stripe_hand_worked_examples, ("golden",)),
    ("pool", _pool_ignores_counts, tpd.test_pad3d_pool_is_the_mean_of_each_tile, ()),
    ("attention_rows", _rows_ignore_counts, tpd.test_pad3d_full_attention_equals_dense, ()),
    ("block_layout", _layout_pads_in_place, tpd.test_pad3d_hand_worked_layouts, ("golden",)),
    ("snr_top_p", _snr_linear_in_log_snr, tsnr.test_snr_hand_worked_schedules, ("golden",)),
    ("snr_top_p", _snr_unsquared, tsnr.test_snr_hand_worked_schedules, ("golden",)),
    ("snr_top_p", _snr_no_warmup, tsnr.test_snr_hand_worked_schedules, ("golden",)),
    ("kmeans", _kmeans_empty_becomes_nan, tcl.test_kmeans_euclidean_equals_scipy, (1, 3)),
    ("quad_distances", _quad_ignores_metric, tcl.test_quad_distances_equal_squared_mahalanobis,
     ()),
    ("cluster_scores", _scores_without_size, tcl.test_cluster_scores_weight_by_size, ()),
    ("cluster_layout", _layout_unpadded, tcl.test_cluster_layout_hand_worked, ("golden",)),
    ("cluster_metric", _metric_without_sizes, tcl.test_cluster_metric_is_the_interaction_error,
     ()),
    ("cluster_attention_rows", _cluster_rows_query_labels,
     tcl.test_cluster_attention_all_kept_equals_dense_sdpa, ()),
    ("tail_merge", _tail_variant(one_sided=True), ttl.test_tail_merge_hand_worked, ("golden",)),
    ("tail_merge", _tail_variant(big_donor=True), ttl.test_tail_merge_hand_worked, ("golden",)),
    ("tail_merge", _tail_variant(no_union=True), ttl.test_tail_merge_invariants, ()),
    ("tail_merge", _tail_variant(head=True), ttl.test_tail_merge_hand_worked, ("golden",)),
]


@pytest.mark.parametrize("name,fn,pin,args", MUTATIONS,
                         ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_pin_catches_planted_mistake(monkeypatch, golden_dir, name, fn, pin, args):
    monkeypatch.setattr(orc, name, fn)
    call = []
    for a in args:
        call.append(golden_dir if a == "golden" else a)
    if args == ("grid_tile",):
        call = [(4, 8, 8), (2, 4, 4)]
    with pytest.raises(AssertionError):
        pin(*call)
