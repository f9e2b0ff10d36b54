"""GPU parity of every stage against the fp64 oracle, through the C ABI.

Run on an MI355X:  python -u -m pytest tests -m gpu -x -v --timeout 120 --timeout-method thread
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import svsa_oracle as orc  # noqa: E402
from svsa_synth import get_config  # noqa: E402

from tests import gpu_cases as gc  # noqa: E402

pytestmark = pytest.mark.gpu

ALL = ["tiny", "small", "wan480", "wan720", "hv720", "wan720_psa", "small_pad3d", "tiny_pad3d",
       "wan720_psa3d"]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ---------------------------------------------------------------- stage 1
@pytest.mark.parametrize("name", ALL)
def test_permute_bit_exact(name):
    run, orun = gc.gpu_run(name), gc.oracle_run(name)
    for tag, g, o in (("q", run.qt_bits, orun.qt_bits), ("k", run.kt_bits, orun.kt_bits),
                      ("v", run.vt_bits, orun.vt_bits)):
        assert np.array_equal(g, o), f"{name}: permuted {tag} differs"


@pytest.mark.parametrize("name", ["small", "wan720", "small_pad3d", "wan720_psa3d"])
def test_inverse_permute_round_trip(name):
    import block_sparse_attention_17_amd as m
    run = gc.gpu_run(name)
    back = torch.empty_like(run.q_dev)
    m.svsa_tile_permute(run.bsa.qt, back, run.geom, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), run.q_dev.view(torch.int16))


@pytest.mark.parametrize("name", ["wan720", "wan720_psa3d"])
def test_natural_output_full_size(name):
    """Full size, in the launch configuration bench.py times (V staged into the
    attention workspace, top-p 0.9): the natural-order output of
    svsa_block_sparse_attn_ex equals the inverse reorder of the tile-order
    output bitwise on every token."""
    import block_sparse_attention_17_amd as m
    run = gc.gpu_run(name)
    run.mask(top_p=np.full(run.cfg.heads, 0.9, np.float32), band=run.cfg.band)
    tile_out = run.bsa.attend()
    nat = run.bsa.attend(natural_out=True)
    back = torch.empty_like(nat)
    m.svsa_tile_permute(tile_out, back, run.geom, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), nat.view(torch.int16))


@pytest.mark.parametrize("grid,tile,D", [((3, 5, 6), (2, 2, 4), 64), ((5, 7, 3), (4, 4, 4), 128),
                                         ((21, 30, 52), (4, 4, 4), 64), ((1, 1, 1), (2, 2, 2), 64),
                                         ((4, 6, 9), (2, 4, 4), 64), ((3, 1, 5), (2, 4, 4), 128)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("pad3d", [False, True])
def test_permute_partial_tiles_and_f32(grid, tile, D, dtype, pad3d):
    import block_sparse_attention_17_amd as m
    G = m.Geometry(*grid, *tile, pad3d=pad3d)
    rng = np.random.default_rng(7)
    N = G.N
    if dtype == "f32":
        x = rng.standard_normal((2, 3, N, D)).astype(np.float32)
        xd = torch.from_numpy(x).cuda()
    else:
        x = rng.integers(0, 0x7F7F, size=(2, 3, N, D), dtype=np.uint16)
        xd = gc.bits_to_dev(x)
    out = torch.full((2, 3, G.N_pad, D), 7, dtype=xd.dtype, device="cuda")
    m.svsa_tile_permute(xd, out, G)
    ref = orc.permute_fwd(x, grid, tile, pad3d)
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, ref)
    back = torch.empty_like(xd)
    m.svsa_tile_permute(out, back, G, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(back.cpu(), xd.cpu())


# ---------------------------------------------------------------- stage 2
@pytest.mark.parametrize("name", ALL)
def test_pool_bit_exact(name):
    run, orun = gc.gpu_run(name), gc.oracle_run(name)
    assert np.array_equal(run.qbar, orun.qbar), f"{name}: Qbar differs"
    assert np.array_equal(run.kbar, orun.kbar), f"{name}: Kbar differs"


def test_pool_f32_partial_tail():
    import block_sparse_attention_17_amd as m
    G = m.Geometry(3, 5, 6, 2, 2, 4)   # N = 90, Bk = 16, tail block of 10
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 2, G.N, 64)).astype(np.float32)
    xt = torch.empty((1, 2, G.N_pad, 64), dtype=torch.float32, device="cuda")
    m.svsa_tile_permute(torch.from_numpy(x).cuda(), xt, G)
    out = torch.empty((1, 2, G.nb, 64), dtype=torch.float64, device="cuda")
    m.svsa_pool(xt, out, G)
    ref = orc.pool(orc.permute_fwd(x, (3, 5, 6), (2, 2, 4)), G.N, G.Bk)
    np.testing.assert_allclose(out.cpu().numpy(), ref, rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("grid,tile,D", [((3, 5, 6), (2, 2, 4), 64), ((5, 7, 3), (4, 4, 4), 128),
                                         ((21, 30, 52), (4, 4, 4), 128), ((1, 1, 1), (2, 2, 2), 64),
                                         ((9, 21, 35), (3, 8, 16), 128),
                                         ((5, 20, 40), (4, 16, 32), 64)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("pad3d", [False, True])
def test_fused_permute_pool(grid, tile, D, dtype, pad3d):
    """svsa_tile_permute_pool equals svsa_tile_permute followed by svsa_pool
    bitwise, and the oracle's reorder and block means (exactly for bf16
    inputs, to 1e-15 for float32 ones).  Partial tiles on every axis, blocks
    straddling partial tiles (packed layout), padding-only block slots (3D
    padding), and a 2048-token block (more rows than one pass of the kernel's
    row map holds)."""
    import block_sparse_attention_17_amd as m
    G = m.Geometry(*grid, *tile, pad3d=pad3d)
    gc.log(f"fused permute+pool grid {grid} tile {tile} D={D} {dtype} pad3d={pad3d}")
    rng = np.random.default_rng(11)
    x = torch.from_numpy(rng.standard_normal((2, 3, G.N, D)).astype(np.float32)).cuda()
    if dtype == "bf16":
        x = x.to(torch.bfloat16)
    x64 = x.float().cpu().numpy().astype(np.float64)
    fused = torch.full((2, 3, G.N_pad, D), 7, dtype=x.dtype, device="cuda")
    means = torch.full((2, 3, G.nb, D), 7.0, dtype=torch.float64, device="cuda")
    m.svsa_tile_permute_pool(x, fused, means, G)
    two = torch.full_like(fused, 5)
    means2 = torch.full_like(means, 5.0)
    m.svsa_tile_permute(x, two, G)
    m.svsa_pool(two, means2, G)
    torch.cuda.synchronize()
    assert torch.equal(fused.cpu(), two.cpu())
    assert torch.equal(means.cpu(), means2.cpu())
    ref_t = orc.permute_fwd(x64, grid, tile, pad3d)
    assert np.array_equal(fused.float().cpu().numpy().astype(np.float64), ref_t)
    _, counts = orc.block_layout(grid, tile, pad3d)
    ref_m = orc.pool(ref_t, G.N, G.Bk, counts)
    if dtype == "bf16":
        assert np.array_equal(means.cpu().numpy(), ref_m)
    else:
        np.testing.assert_allclose(means.cpu().numpy(), ref_m, rtol=1e-15, atol=1e-15)


# ---------------------------------------------------------------- stage 3
MASK_CASES = [("tiny", 0.9, None), ("small", 0.9, None), ("wan480", 0.9, None),
              ("wan720", 0.9, None), ("wan720", 0.8, None), ("wan720", 0.95, None),
              ("hv720", 0.9, None), ("hv720", None, "keep"), ("small_b2", 0.9, None),
              ("wan720_psa", 0.9, None), ("small_pad3d", 0.9, None), ("tiny_pad3d", 0.9, None),
              ("wan720_psa3d", 0.9, None), ("maxnb", 0.9, None)]


@pytest.mark.parametrize("name,p,mode", MASK_CASES)
def test_block_mask_matches_oracle(name, p, mode):
    cfg = get_config(name)
    run, orun = gc.gpu_run(name), gc.oracle_run(name)
    heads = cfg.heads
    top_p = None if mode else np.full(heads, p, np.float32)
    keep = run.inp.keep_frac if mode else None
    g_rp, g_ci = run.mask(top_p=top_p, keep_frac=keep, band=cfg.band)
    o_rp, o_ci = orun.mask(top_p=top_p, keep_frac=keep, band=cfg.band)
    assert g_rp.shape == o_rp.shape
    tol, bad = gc.mask_mismatch(cfg, orun.S, g_rp, g_ci, o_rp, o_ci, top_p=top_p,
                                keep_frac=keep, band=cfg.band)
    gc.log(f"{name} p={p} mode={mode}: {len(tol)} tolerated rows, {len(bad)} failing, "
           f"kept fraction {o_rp[-1] / (cfg.batch * heads * cfg.nb ** 2):.4f}")
    assert not bad, f"rows {bad[:10]} differ beyond the threshold tolerance"
    # every GPU row ascending and unique
    for r in range(0, len(g_rp) - 1, max(1, (len(g_rp) - 1) // 997)):
        row = g_ci[g_rp[r]: g_rp[r + 1]]
        assert np.all(np.diff(row) > 0)


def test_block_mask_band_and_limits():
    cfg = get_config("small")
    run, orun = gc.gpu_run("small"), gc.oracle_run("small")
    for kw in (dict(top_p=np.full(cfg.heads, 1.0, np.float32)),
               dict(top_p=np.full(cfg.heads, 1e-6, np.float32)),
               dict(keep_frac=np.full(cfg.heads, 1.0, np.float32)),
               dict(top_p=np.linspace(0.3, 0.99, cfg.heads).astype(np.float32))):
        for band in (1, 3):
            g_rp, g_ci = run.mask(band=band, **kw)
            o_rp, o_ci = orun.mask(band=band, **kw)
            tol, bad = gc.mask_mismatch(cfg, orun.S, g_rp, g_ci, o_rp, o_ci, band=band, **kw)
            assert not bad


@pytest.mark.parametrize("nb", [200, 300])
def test_block_mask_equal_and_few_distinct_scores(nb):
    """Crafted block summaries whose rows hold exactly equal scores (no radix
    pass; the tie rule alone decides), two or three distinct values (long
    common key prefixes, ties at the boundary), scores that underflow to zero,
    many ties at row-dependent scales, and rows whose probabilities past the
    first ten blocks are subnormal (the normalisation's plain-division path,
    and a fixed-fraction boundary among subnormal keys): the lists equal the
    oracle's up to the near-threshold rule, in top-p and fixed-fraction modes."""
    import types
    import torch
    from block_sparse_attention_17_amd import binding as B
    H, D = 6, 16
    scale = 1.0 / np.sqrt(D)
    j = np.arange(nb)
    logit = np.zeros((H, nb))
    logit[1] = np.where(j % 3 == 0, 2.0, 0.0)
    logit[2] = np.where(j % 5 == 0, 3.0, np.where(j % 7 == 0, 1.5, 0.0))
    logit[3] = np.where(j < 40, 0.0, -1000.0)          # exp underflows to 0.0
    logit[4] = np.round(np.random.default_rng(11).normal(size=nb) * 2) / 2
    logit[5] = np.where(j < 10, 0.0, -712.0 - 30.0 * j / nb)   # e^-712 .. e^-742: subnormal
    qbar = np.zeros((1, H, nb, D))
    kbar = np.zeros((1, H, nb, D))
    qbar[0, :, :, 0] = 1.0 / scale
    qbar[0, 4, :, 0] *= 1 + (j % 3)                   # row-dependent scale, same ties
    kbar[0, :, :, 0] = logit
    S = orc.block_scores(qbar, kbar, scale)
    dq, dk = torch.from_numpy(qbar).cuda(), torch.from_numpy(kbar).cuda()
    rows = H * nb
    rp_d = torch.empty(rows + 1, dtype=torch.int32, device="cuda")
    ci_d = torch.empty(rows * nb, dtype=torch.int32, device="cuda")
    ws = torch.empty(B.svsa_block_mask_workspace_bytes(1, H, nb), dtype=torch.uint8,
                     device="cuda")
    cfg = types.SimpleNamespace(nb=nb, heads=H)
    settings = [dict(top_p=np.full(H, p, np.float32)) for p in (1e-6, 0.5, 0.9, 0.999)]
    settings += [dict(keep_frac=np.full(H, f, np.float32)) for f in (0.1, 0.5)]
    for kw in settings:
        for band in (1, 2):
            B.svsa_block_mask(dq, dk, scale, rp_d, ci_d, ws, band_width=band, **kw)
            torch.cuda.synchronize()
            g_rp = rp_d.cpu().numpy().astype(np.int64)
            g_ci = ci_d[: int(g_rp[-1])].cpu().numpy()
            o_rp, o_ci = orc.block_mask(S, band, **kw)
            tol, bad = gc.mask_mismatch(cfg, S, g_rp, g_ci, o_rp, o_ci, band=band, **kw)
            gc.log(f"crafted nb={nb} {list(kw)[0]}={float(list(kw.values())[0][0])} "
                   f"band={band}: {len(tol)} tolerated, {len(bad)} failing")
            assert not bad, f"rows {bad[:10]} differ beyond the threshold tolerance"
            for r in range(rows):
                row = g_ci[g_rp[r]: g_rp[r + 1]]
                assert row.size >= 1 and np.all(np.diff(row) > 0)


def test_block_mask_over_snr_schedule():
    """Per-step top-p from svsa_snr_top_p ([iCATS] Sec. 4.2 reading) drives the
    mask: every step's CSR equals the oracle's mask at the oracle's schedule."""
    import block_sparse_attention_17_amd as m
    from svsa_synth import flow_sigmas
    cfg = get_config("small")
    run, orun = gc.gpu_run("small"), gc.oracle_run("small")
    sig = flow_sigmas(8, 5.0)
    sched = m.svsa_snr_top_p(sig, 2, 0.7, 0.999)
    ref = orc.snr_top_p(sig, 2, float(np.float32(0.7)), float(np.float32(0.999)))
    np.testing.assert_allclose(sched, ref, rtol=2 ** -23, atol=0)
    kept = []
    for p_k in sched:
        tp = np.full(cfg.heads, p_k, np.float32)
        g_rp, g_ci = run.mask(top_p=tp, band=cfg.band)
        o_rp, o_ci = orun.mask(top_p=tp, band=cfg.band)
        tol, bad = gc.mask_mismatch(cfg, orun.S, g_rp, g_ci, o_rp, o_ci, top_p=tp, band=cfg.band)
        assert not bad
        kept.append(int(g_rp[-1]))
    gc.log(f"small SNR schedule: top-p {np.round(sched, 4).tolist()} kept blocks {kept}")
    assert all(a >= b for a, b in zip(kept, kept[1:]))     # top-p never rises


# ---------------------------------------------------------------- stage 4
_ATTN_BASE = [("tiny", None), ("small", None), ("wan480", 6), ("wan720", 3), ("hv720", 2),
              ("small_b2", None), ("small_pad3d", None), ("tiny_pad3d", None), ("maxnb", 12)]
# every top-p each config sweeps (Wan-720p: 0.8, 0.9 and 0.95)
ATTN_CASES = [(name, per_head, p) for name, per_head in _ATTN_BASE for p in get_config(name).top_p]


@pytest.mark.parametrize("name,per_head,p", ATTN_CASES)
def test_attention_matches_oracle(name, per_head, p):
    cfg = get_config(name)
    run, orun = gc.gpu_run(name), gc.oracle_run(name)
    o_rp, o_ci = orun.mask(top_p=np.full(cfg.heads, p, np.float32), band=cfg.band)
    out_bits = run.attention(o_rp, o_ci)
    if per_head is None:
        rows = [(b, h, i) for b in range(cfg.batch) for h in range(cfg.heads) for i in range(cfg.nb)]
    else:
        rows = gc.sample_rows(cfg, o_rp, per_head)
    ref = orun.attention_blocks(o_rp, o_ci, rows)
    max_abs, rel = gc.attn_errors(out_bits, ref, cfg)
    gc.log(f"{name} p={p}: {len(rows)} q-blocks, max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2


@pytest.mark.parametrize("name,mode,which", [("wan720", 0.8, "heaviest"),
                                             ("wan720", 0.95, "heaviest"),
                                             ("hv720", 0.9, "heaviest"),
                                             ("hv720", "fixed", "median")])
def test_attention_whole_head(name, mode, which):
    """Full size, every query block of one whole head against the oracle with
    the oracle's mask: the heaviest head (most kept blocks) at the swept top-p
    values not covered whole elsewhere, and a median head in the fixed-fraction
    mode."""
    cfg = get_config(name)
    run, orun = gc.gpu_run(name), gc.oracle_run(name)
    if mode == "fixed":
        o_rp, o_ci = orun.mask(keep_frac=run.inp.keep_frac, band=cfg.band)
    else:
        o_rp, o_ci = orun.mask(top_p=np.full(cfg.heads, mode, np.float32), band=cfg.band)
    out_bits = run.attention(o_rp, o_ci)
    kept = np.diff(o_rp).reshape(cfg.heads, cfg.nb).sum(1)
    order = np.argsort(kept, kind="stable")
    h = int(order[-1]) if which == "heaviest" else int(order[len(order) // 2])
    rows = [(0, h, i) for i in range(cfg.nb)]
    gc.log(f"{name} {mode}: oracle attention of head {h} ({kept[h]} kept blocks)")
    max_abs, rel = gc.attn_errors(out_bits, orun.attention_blocks(o_rp, o_ci, rows), cfg)
    gc.log(f"{name} {mode} head {h} ({kept[h] / cfg.nb ** 2:.3f} kept), all {cfg.nb} q-blocks: "
           f"max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2


def test_more_pairs_than_the_queues_balance():
    """2100 (batch, head) pairs (beyond the 2048 the work queues place by
    measured work): mask equal to the oracle's, attention on sampled pairs."""
    cfg = get_config("manybh")
    run, orun = gc.gpu_run("manybh"), gc.oracle_run("manybh")
    tp = np.full(cfg.heads, 0.9, np.float32)
    g_rp, g_ci = run.mask(top_p=tp, band=cfg.band)
    o_rp, o_ci = orun.mask(top_p=tp, band=cfg.band)
    assert np.array_equal(g_rp, o_rp) and np.array_equal(g_ci, o_ci)
    out_bits = run.attention(o_rp, o_ci)
    rows = [(b, 0, i) for b in (0, 1, 777, 2047, 2048, 2099) for i in range(cfg.nb)]
    max_abs, rel = gc.attn_errors(out_bits, orun.attention_blocks(o_rp, o_ci, rows), cfg)
    gc.log(f"manybh: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2


def test_pairs_cut_into_fewer_runs():
    """700 (batch, head) pairs of 8 blocks (two query groups each): each pair's
    groups go to the work queues as two runs of one group.  Mask equal to the
    oracle's, attention on the first, a middle and the last pairs."""
    cfg = get_config("midbh")
    run, orun = gc.gpu_run("midbh"), gc.oracle_run("midbh")
    assert cfg.batch * cfg.heads == 700 and cfg.nb == 8
    tp = np.full(cfg.heads, 0.9, np.float32)
    g_rp, g_ci = run.mask(top_p=tp, band=cfg.band)
    o_rp, o_ci = orun.mask(top_p=tp, band=cfg.band)
    assert np.array_equal(g_rp, o_rp) and np.array_equal(g_ci, o_ci)
    out_bits = run.attention(o_rp, o_ci)
    rows = [(b, 0, i) for b in (0, 1, 350, 511, 512, 699) for i in range(cfg.nb)]
    max_abs, rel = gc.attn_errors(out_bits, orun.attention_blocks(o_rp, o_ci, rows), cfg)
    gc.log(f"midbh: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2


def test_attention_whole_heads_wan720():
    """Full Wan-720p size, top-p 0.9: every query block of four whole heads
    (the heaviest, the lightest and two median heads by kept blocks)."""
    cfg = get_config("wan720")
    run, orun = gc.gpu_run("wan720"), gc.oracle_run("wan720")
    o_rp, o_ci = orun.mask(top_p=np.full(cfg.heads, 0.9, np.float32), band=cfg.band)
    out_bits = run.attention(o_rp, o_ci)
    kept = np.diff(o_rp).reshape(cfg.heads, cfg.nb).sum(1)
    order = np.argsort(kept, kind="stable")
    heads = sorted({int(order[-1]), int(order[0]), int(order[len(order) // 2]),
                    int(order[len(order) // 2 - 1])})
    for h in heads:
        rows = [(0, h, i) for i in range(cfg.nb)]
        max_abs, rel = gc.attn_errors(out_bits, orun.attention_blocks(o_rp, o_ci, rows), cfg)
        gc.log(f"wan720 head {h} ({kept[h]} kept blocks), all {cfg.nb} q-blocks: "
               f"max_abs={max_abs:.3e} rel_l2={rel:.3e}")
        assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2


def test_attention_psa_block_shape_wan720():
    """384-token blocks (PSA's 3x8x16 PSABlock shape): the attention kernel runs
    them as six 64-token sub-blocks; rows of five heads, incl. the tail block."""
    cfg = get_config("wan720_psa")
    run, orun = gc.gpu_run("wan720_psa"), gc.oracle_run("wan720_psa")
    o_rp, o_ci = orun.mask(top_p=np.full(cfg.heads, 0.9, np.float32), band=cfg.band)
    out_bits = run.attention(o_rp, o_ci)
    rows = gc.sample_rows(cfg, o_rp, 1, seed=9, heads=[0, 7, 13, 21, 33])
    max_abs, rel = gc.attn_errors(out_bits, orun.attention_blocks(o_rp, o_ci, rows), cfg)
    gc.log(f"wan720_psa: {len(rows)} q-blocks, max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2


def test_attention_psa_3d_padding_wan720():
    """PSA's 3D-padded layout at full size: 210 blocks of 384 slots, the last
    tile row holding 3x5x16 = 240 tokens (sub-blocks 4 and 5 padding only);
    sampled rows include the padded tiles' rows."""
    cfg = get_config("wan720_psa3d")
    run, orun = gc.gpu_run("wan720_psa3d"), gc.oracle_run("wan720_psa3d")
    o_rp, o_ci = orun.mask(top_p=np.full(cfg.heads, 0.9, np.float32), band=cfg.band)
    out_bits = run.attention(o_rp, o_ci)
    rows = gc.sample_rows(cfg, o_rp, 1, seed=4, heads=[0, 11, 26, 39])
    rows += [(0, 5, i) for i in (25, 29, 209)]    # tiles of the padded last tile row
    max_abs, rel = gc.attn_errors(out_bits, orun.attention_blocks(o_rp, o_ci, rows), cfg)
    gc.log(f"wan720_psa3d: {len(rows)} q-blocks, max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2


def test_whole_path_pad3d_equals_dense_attention():
    """3D-padded layout, every block kept: the whole path (permute, pool, mask,
    attention, inverse permute) equals dense attention in natural order."""
    cfg = get_config("tiny_pad3d")
    run = gc.gpu_run("tiny_pad3d")
    out = run.bsa(run.q_dev, run.k_dev, run.v_dev, top_p=np.ones(cfg.heads, np.float32))
    torch.cuda.synchronize()
    got = orc.widen(gc.dev_to_bits(out))
    ref = orc.dense_attention(run.inp.q, run.inp.k, run.inp.v, 1 / np.sqrt(cfg.head_dim))
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert np.abs(got - ref).max() <= gc.MAX_ABS and rel <= gc.REL_L2


def test_attention_fixed_mode_hv720():
    cfg = get_config("hv720")
    run, orun = gc.gpu_run("hv720"), gc.oracle_run("hv720")
    keep = run.inp.keep_frac
    o_rp, o_ci = orun.mask(keep_frac=keep, band=cfg.band)
    out_bits = run.attention(o_rp, o_ci)
    rows = gc.sample_rows(cfg, o_rp, 2, seed=5)
    max_abs, rel = gc.attn_errors(out_bits, orun.attention_blocks(o_rp, o_ci, rows), cfg)
    gc.log(f"hv720 fixed: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2


def test_dense_path_equals_dense_attention():
    """Every block kept (p = 1) through the whole path = dense softmax attention."""
    import block_sparse_attention_17_amd as m
    cfg = get_config("small")
    run = gc.gpu_run("small")
    out = run.bsa(run.q_dev, run.k_dev, run.v_dev, top_p=np.ones(cfg.heads, np.float32))
    torch.cuda.synchronize()
    got = orc.widen(gc.dev_to_bits(out))
    inp = run.inp
    ref = orc.dense_attention(inp.q, inp.k, inp.v, 1 / np.sqrt(cfg.head_dim))
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert err.max() <= gc.MAX_ABS and rel <= gc.REL_L2
    assert run.bsa.row_ptr[-1].item() == cfg.heads * cfg.nb * cfg.nb


def test_whole_path_bitwise_deterministic():
    cfg = get_config("wan480")
    run = gc.gpu_run("wan480")
    outs = []
    for _ in range(2):
        o = run.bsa(run.q_dev, run.k_dev, run.v_dev, top_p=np.full(cfg.heads, 0.9, np.float32))
        torch.cuda.synchronize()
        outs.append(o.clone())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


@pytest.mark.parametrize("step_pairs", [False, True])
def test_attention_edge_cases_custom_csr(step_pairs):
    """Empty row -> zeros (also a whole 4-block query group with nothing to
    do); out-of-range columns ignored; one block per row is local attention.
    Both list walks (entries, and step pairs)."""
    import block_sparse_attention_17_amd as m
    cfg = get_config("small")
    run, orun = gc.gpu_run("small"), gc.oracle_run("small")
    nb, H = cfg.nb, cfg.heads
    rows_cols = []
    for h in range(H):
        for i in range(nb):
            if (h, i) == (0, 5) or (h == 2 and 8 <= i < 12):
                rows_cols.append([])                      # empty (head 2: a whole group)
            elif (h, i) == (1, 7):
                rows_cols.append([-3, 2, 7, nb + 4])      # out-of-range ignored
            else:
                rows_cols.append([i])                     # diagonal only
    rp = np.zeros(H * nb + 1, np.int64)
    rp[1:] = np.cumsum([len(c) for c in rows_cols])
    ci = np.array([c for cs in rows_cols for c in cs], np.int32)
    out_bits = run.attention(rp, ci, step_pairs=step_pairs)
    zero_blk = orc.widen(out_bits[0, 0, 5 * 64: 6 * 64])
    assert np.all(zero_blk == 0)
    assert np.all(orc.widen(out_bits[0, 2, 8 * 64: 12 * 64]) == 0)
    clean = [[c for c in cs if 0 <= c < nb] for cs in rows_cols]
    rp2 = np.zeros_like(rp)
    rp2[1:] = np.cumsum([len(c) for c in clean])
    ci2 = np.array([c for cs in clean for c in cs], np.int32)
    rows = [(0, h, i) for h in range(H) for i in range(nb)
            if (h, i) != (0, 5) and not (h == 2 and 8 <= i < 12)]
    ref = orun.attention_blocks(rp2, ci2, rows)
    max_abs, rel = gc.attn_errors(out_bits, ref, cfg)
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2


@pytest.mark.parametrize("step_pairs", [False, True])
def test_empty_groups_with_stale_workspace(step_pairs):
    """Work items whose union list is empty stream nothing and write zeros,
    whatever the attention workspace held: every workspace byte is 0xFF before
    V is staged.  Cases: a whole 4-block query group of empty rows, and PSA's
    3D-padded 3x8x16 tiles on a 9x21x35 grid, whose last tile row holds sub-blocks
    of padding only (their groups keep nothing).  Both list walks."""
    import block_sparse_attention_17_amd as m
    # (a) a whole query group of empty rows
    cfg = get_config("small")
    run, orun = gc.gpu_run("small"), gc.oracle_run("small")
    nb, H = cfg.nb, cfg.heads
    cols = [[] if (h == 3 and 4 <= i < 8) or (h == 0 and i < 4) else
            sorted({i, (i * 7 + h) % nb, (i + 5) % nb}) for h in range(H) for i in range(nb)]
    rp = np.zeros(H * nb + 1, np.int64)
    rp[1:] = np.cumsum([len(c) for c in cols])
    ci = np.array([c for cs in cols for c in cs], np.int32)
    run.bsa.attn_ws.fill_(0xFF)
    m.svsa_attn_stage_v(run.v_dev, run.bsa.attn_ws, run.geom)
    out_bits = run.attention(rp, ci, step_pairs=step_pairs)
    assert np.all(orc.widen(out_bits[0, 3, 4 * 64: 8 * 64]) == 0)
    assert np.all(orc.widen(out_bits[0, 0, : 4 * 64]) == 0)
    rows = [(0, h, i) for h in range(H) for i in range(nb) if cols[h * nb + i]]
    max_abs, rel = gc.attn_errors(out_bits, orun.attention_blocks(rp, ci, rows), cfg)
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2
    # (b) 3D-padded tiles with padding-only sub-blocks, every valid row
    grid, tile, D, Hh = (9, 21, 35), (3, 8, 16), 128, 2
    G = m.Geometry(*grid, *tile, pad3d=True)
    rng = np.random.default_rng(61)
    from svsa_synth import f32_to_bf16_bits
    bits = [f32_to_bf16_bits(rng.standard_normal((1, Hh, G.N, D)).astype(np.float32))
            for _ in range(3)]
    nat = [gc.bits_to_dev(b) for b in bits]
    tiled = [torch.empty((1, Hh, G.N_pad, D), dtype=torch.bfloat16, device="cuda")
             for _ in range(2)]
    for x, t in zip(nat, tiled):
        m.svsa_tile_permute(x, t, G)
    lists = [sorted(set(rng.choice(G.nb, size=int(rng.integers(1, G.nb + 1)),
                                   replace=False).tolist()) | {i})
             for _ in range(Hh) for i in range(G.nb)]
    rp = np.zeros(Hh * G.nb + 1, np.int64)
    rp[1:] = np.cumsum([len(c) for c in lists])
    ci = np.array([c for cs in lists for c in cs], np.int32)
    rp_d = torch.from_numpy(rp.astype(np.int32)).cuda()
    ci_d = torch.from_numpy(ci).cuda()
    ws = torch.full((m.svsa_attn_workspace_bytes(1, Hh, G),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    m.svsa_attn_stage_v(nat[2], ws, G)
    out = torch.full((1, Hh, G.N, D), 7.0, dtype=torch.bfloat16, device="cuda")
    m.svsa_block_sparse_attn_ex(tiled[0], tiled[1], None, out, G, 1 / np.sqrt(D), rp_d, ci_d, ws,
                                flags=m.SVSA_ATTN_OUT_NATURAL
                                | (m.SVSA_ATTN_STEP_PAIRS if step_pairs else 0))
    torch.cuda.synchronize()
    got = orc.widen(gc.dev_to_bits(out))
    slots, counts = orc.block_layout(grid, tile, True)
    assert (counts % 64 != 0).any() and (counts <= G.Bk - 64).any()   # padding-only sub-blocks
    qt, kt, vt = (orc.permute_fwd(b, grid, tile, True) for b in bits)
    ref_t = orc.attention(qt, kt, vt, rp, ci, G.N, G.Bk, 1 / np.sqrt(D), counts=counts)
    ref = orc.permute_inv(ref_t, grid, tile, True)
    max_abs = float(np.abs(got - ref).max())
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    gc.log(f"stale workspace, 3D-padded 3x8x16: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2


@pytest.mark.parametrize("D", [128, 64])
def test_attention_large_logit_range(D):
    """Rows whose later kept key block scores ~80 nats above the blocks they
    keep first: the online softmax has to move its running offset by far more
    than its lazy threshold and rescale what it accumulated; the result still
    matches the oracle.  Other rows of the same call keep ordinary logits."""
    import block_sparse_attention_17_amd as m
    from svsa_synth import f32_to_bf16_bits
    G = m.Geometry(4, 8, 16, 4, 4, 4)            # 512 tokens, 8 blocks of 64
    H, nb = 2, G.nb
    rng = np.random.default_rng(71)
    q = rng.standard_normal((1, H, G.N_pad, D)).astype(np.float32)
    k = rng.standard_normal((1, H, G.N_pad, D)).astype(np.float32)
    v = rng.standard_normal((1, H, G.N_pad, D)).astype(np.float32)
    u = np.zeros(D, np.float32)
    u[3] = 1.0
    q[0, 0, :128] = 30.0 * u + 0.01 * q[0, 0, :128]     # query blocks 0, 1 of head 0
    k[0, 0, 5 * 64: 6 * 64] = 30.0 * u                    # key block 5 of head 0
    bits = [f32_to_bf16_bits(x) for x in (q, k, v)]
    lists = [sorted({i, 5, (i + 3) % nb}) for _ in range(H) for i in range(nb)]
    rp = np.zeros(H * nb + 1, np.int64)
    rp[1:] = np.cumsum([len(c) for c in lists])
    ci = np.array([c for cs in lists for c in cs], np.int32)
    dev = [gc.bits_to_dev(b) for b in bits]
    out = torch.empty_like(dev[0])
    ws = torch.empty(m.svsa_attn_workspace_bytes(1, H, G), dtype=torch.uint8, device="cuda")
    m.svsa_block_sparse_attn(dev[0], dev[1], dev[2], out, G, 1 / np.sqrt(D),
                             torch.from_numpy(rp.astype(np.int32)).cuda(),
                             torch.from_numpy(ci).cuda(), ws)
    torch.cuda.synchronize()
    got = orc.widen(gc.dev_to_bits(out))
    ref = orc.attention(bits[0], bits[1], bits[2], rp, ci, G.N, G.Bk, 1 / np.sqrt(D))
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    gc.log(f"large logit range D={D}: max_abs={err.max():.3e} rel_l2={rel:.3e}")
    assert np.all(np.isfinite(got))
    assert err.max() <= gc.MAX_ABS and rel <= gc.REL_L2


@pytest.mark.parametrize("grid,tile,D,pad3d", [((5, 9, 14), (4, 4, 4), 128, False),
                                               ((5, 9, 14), (4, 4, 4), 64, True),
                                               ((7, 20, 35), (3, 4, 8), 128, False),
                                               ((7, 20, 35), (3, 4, 8), 64, True),
                                               ((9, 21, 35), (3, 8, 16), 128, False),
                                               ((9, 21, 35), (3, 8, 16), 128, True)])
def test_staged_v_equals_tiled_v(grid, tile, D, pad3d):
    """svsa_attn_stage_v from natural-order V, then svsa_block_sparse_attn with
    v = NULL, gives the output of svsa_block_sparse_attn on svsa_tile_permute's
    tiled V bitwise (64- and 32-token sub-blocks, partial tiles, both layouts,
    random kept sets); a second call on the same workspace gives it again, and
    the natural-order output (SVSA_ATTN_OUT_NATURAL) equals the inverse reorder
    of the tile-order one."""
    import block_sparse_attention_17_amd as m
    G = m.Geometry(*grid, *tile, pad3d=pad3d)
    H, nb = 2, G.nb
    gc.log(f"staged V: grid {grid} tile {tile} D={D} pad3d={pad3d}, {nb} blocks")
    rng = np.random.default_rng(59)
    nat = [torch.from_numpy(rng.standard_normal((1, H, G.N, D)).astype(np.float32)).cuda()
           .to(torch.bfloat16) for _ in range(3)]
    tiled = [torch.empty((1, H, G.N_pad, D), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    for x, t in zip(nat, tiled):
        m.svsa_tile_permute(x, t, G)
    lists = [sorted(set(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False).tolist())
                    | {i}) for _ in range(H) for i in range(nb)]
    rp = np.zeros(H * nb + 1, np.int32)
    rp[1:] = np.cumsum([len(c) for c in lists])
    rp_d = torch.from_numpy(rp).cuda()
    ci_d = torch.from_numpy(np.array([c for cs in lists for c in cs], np.int32)).cuda()
    wsb = m.svsa_attn_workspace_bytes(1, H, G)
    ws1 = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    ws2 = torch.full((wsb,), 0x5A, dtype=torch.uint8, device="cuda")
    ref = torch.empty_like(tiled[0])
    got = torch.full_like(tiled[0], 3.0)
    got2 = torch.full_like(tiled[0], 5.0)
    m.svsa_block_sparse_attn(tiled[0], tiled[1], tiled[2], ref, G, 1 / np.sqrt(D), rp_d, ci_d, ws1)
    m.svsa_attn_stage_v(nat[2], ws2, G)
    m.svsa_block_sparse_attn(tiled[0], tiled[1], None, got, G, 1 / np.sqrt(D), rp_d, ci_d, ws2)
    m.svsa_block_sparse_attn(tiled[0], tiled[1], None, got2, G, 1 / np.sqrt(D), rp_d, ci_d, ws2)
    nat_out = torch.full((1, H, G.N, D), 7.0, dtype=torch.bfloat16, device="cuda")
    m.svsa_block_sparse_attn_ex(tiled[0], tiled[1], None, nat_out, G, 1 / np.sqrt(D), rp_d, ci_d,
                                ws2, flags=m.SVSA_ATTN_OUT_NATURAL)
    ref_nat = torch.empty_like(nat_out)
    m.svsa_tile_permute(ref, ref_nat, G, inverse=True)
    torch.cuda.synchronize()
    # natural-order output from the kernel = inverse reorder of the tile-order output
    assert torch.equal(ref_nat.view(torch.int16).cpu(), nat_out.view(torch.int16).cpu())
    # padding slots of the output are unspecified (the packed layout's tail past
    # the last sub-block is not written at all): compare the valid rows
    slots, _ = orc.block_layout(grid, tile, pad3d)
    valid = torch.from_numpy(slots >= 0)
    r = ref.view(torch.int16).cpu()[:, :, valid]
    assert torch.equal(r, got.view(torch.int16).cpu()[:, :, valid])
    assert torch.equal(r, got2.view(torch.int16).cpu()[:, :, valid])


@pytest.mark.parametrize("pad3d", [False, True])
def test_attention_96_token_blocks_d128(pad3d):
    """Blocks of 96 tokens (three 32-token sub-blocks: the kernel streams the
    schedule two entries per 64-key tile, so tiles straddle blocks) at head_dim
    128, packed (partial tail block) and 3D-padded (partial tiles, sub-blocks
    of padding only): every valid row against the oracle on random kept sets."""
    import block_sparse_attention_17_amd as m
    from svsa_synth.gen import f32_to_bf16_bits
    grid, tile, H, D = (5, 7, 10), (3, 4, 8), 3, 128
    N, Bk = grid[0] * grid[1] * grid[2], tile[0] * tile[1] * tile[2]
    slots, counts = orc.block_layout(grid, tile, pad3d)
    nb = len(counts)
    rng = np.random.default_rng(41 + int(pad3d))
    nat = {n: f32_to_bf16_bits(rng.standard_normal((1, H, N, D)).astype(np.float32))
           for n in "qkv"}
    valid = slots >= 0
    tiled = {}
    for n in "qkv":
        t = np.zeros((1, H, nb * Bk, D), np.uint16)
        t[:, :, valid] = nat[n][:, :, slots[valid]]
        tiled[n] = t
    lists = []
    for h in range(H):
        for i in range(nb):
            keep = set(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False).tolist())
            lists.append(sorted(keep | {i}))
    rp = np.zeros(H * nb + 1, np.int64)
    rp[1:] = np.cumsum([len(c) for c in lists])
    ci = np.array([c for cs in lists for c in cs], np.int32)
    geom = m.Geometry(*grid, *tile, pad3d=pad3d)
    out = torch.empty((1, H, nb * Bk, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(m.svsa_attn_workspace_bytes(1, H, geom), dtype=torch.uint8, device="cuda")
    gc.log(f"96-token blocks, D 128, pad3d={pad3d}: {nb} blocks, {int(rp[-1])} kept pairs")
    m.svsa_block_sparse_attn(*(gc.bits_to_dev(tiled[n]) for n in "qkv"), out, geom,
                             1 / np.sqrt(D), torch.from_numpy(rp.astype(np.int32)).cuda(),
                             torch.from_numpy(ci).cuda(), ws)
    torch.cuda.synchronize()
    got = gc.dev_to_bits(out)
    ref = orc.attention(tiled["q"], tiled["k"], tiled["v"], rp, ci, N, Bk, 1 / np.sqrt(D),
                        counts=counts)
    g_all, r_all = [], []
    for h in range(H):
        for i in range(nb):
            rows = slice(i * Bk, i * Bk + int(counts[i]))
            g_all.append(orc.widen(got[0, h, rows]).ravel())
            r_all.append(ref[0, h, rows].ravel())
    g, r = np.concatenate(g_all), np.concatenate(r_all)
    max_abs = float(np.max(np.abs(g - r)))
    rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
    gc.log(f"  max_abs {max_abs:.3e} rel_l2 {rel:.3e}")
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2


_SWEEP_TILES = [(2, 4, 4), (1, 4, 8), (2, 2, 8), (4, 4, 4), (3, 4, 8), (2, 4, 8), (1, 8, 8),
                (2, 8, 8), (3, 8, 16)]


def _sweep_case(seed):
    """Seeded small geometry: a tile whose volume is a multiple of 32, a grid
    with partial tiles on most axes, either layout, head_dim 64 or 128."""
    rng = np.random.default_rng(1000 + seed)
    tile = _SWEEP_TILES[seed % len(_SWEEP_TILES)]
    while True:
        grid = tuple(int(rng.integers(t, 3 * t + 4)) for t in tile)
        if grid[0] * grid[1] * grid[2] <= 6000:
            break
    return dict(grid=grid, tile=tile, pad3d=bool(rng.integers(0, 2)),
                D=int(rng.choice([64, 128])), top_p=float(rng.uniform(0.5, 0.97)),
                band=int(rng.integers(1, 3)), rng=rng)


@pytest.mark.parametrize("seed", range(10))
def test_whole_path_random_small_geometries(seed):
    """The whole path on seeded small geometries: tile permute and block means
    bit-exact, the mask against the oracle's (near-threshold rule), attention
    with the oracle's mask on every valid row, inverse permute back to the
    natural order."""
    import types
    import block_sparse_attention_17_amd as m
    from svsa_synth.gen import f32_to_bf16_bits
    c = _sweep_case(seed)
    grid, tile, pad3d, D, rng = c["grid"], c["tile"], c["pad3d"], c["D"], c["rng"]
    H = 2
    geom = m.Geometry(*grid, *tile, pad3d=pad3d)
    N, Bk, nb = geom.N, geom.Bk, geom.nb
    gc.log(f"sweep {seed}: grid {grid} tile {tile} pad3d={pad3d} D={D} nb={nb} "
           f"top_p={c['top_p']:.3f} band={c['band']}")
    nat = {n: f32_to_bf16_bits(rng.standard_normal((1, H, N, D)).astype(np.float32))
           for n in "qkv"}
    _, counts = orc.block_layout(grid, tile, pad3d)
    tiled_o = {n: orc.permute_fwd(nat[n], grid, tile, pad3d) for n in "qkv"}
    dev = {n: gc.bits_to_dev(nat[n]) for n in "qkv"}
    tiled = {n: torch.empty((1, H, geom.N_pad, D), dtype=torch.bfloat16, device="cuda")
             for n in "qkv"}
    for n in "qkv":
        m.svsa_tile_permute(dev[n], tiled[n], geom)
    bars = {n: torch.empty((1, H, nb, D), dtype=torch.float64, device="cuda") for n in "qk"}
    for n in "qk":
        m.svsa_pool(tiled[n], bars[n], geom)
    torch.cuda.synchronize()
    for n in "qkv":
        assert np.array_equal(orc.widen(gc.dev_to_bits(tiled[n])), tiled_o[n]), f"tiled {n} differs"
    qbar_o = orc.pool(tiled_o["q"], N, Bk, counts)
    kbar_o = orc.pool(tiled_o["k"], N, Bk, counts)
    assert np.array_equal(bars["q"].cpu().numpy(), qbar_o)
    assert np.array_equal(bars["k"].cpu().numpy(), kbar_o)
    scale = 1 / np.sqrt(D)
    tp = np.full(H, c["top_p"], np.float32)
    S = orc.block_scores(qbar_o, kbar_o, scale)
    o_rp, o_ci = orc.block_mask(S, c["band"], top_p=tp)
    rp_d = torch.empty(H * nb + 1, dtype=torch.int32, device="cuda")
    ci_d = torch.empty(H * nb * nb, dtype=torch.int32, device="cuda")
    mws = torch.empty(m.svsa_block_mask_workspace_bytes(1, H, nb), dtype=torch.uint8,
                      device="cuda")
    m.svsa_block_mask(bars["q"], bars["k"], scale, rp_d, ci_d, mws, top_p=tp,
                      band_width=c["band"])
    torch.cuda.synchronize()
    g_rp = rp_d.cpu().numpy().astype(np.int64)
    g_ci = ci_d[: int(g_rp[-1])].cpu().numpy()
    tol, bad = gc.mask_mismatch(types.SimpleNamespace(nb=nb, heads=H), S, g_rp, g_ci, o_rp,
                                o_ci, top_p=tp, band=c["band"])
    assert not bad, f"mask rows {bad[:5]} differ beyond the threshold tolerance"
    out_t = torch.empty((1, H, geom.N_pad, D), dtype=torch.bfloat16, device="cuda")
    aws = torch.empty(m.svsa_attn_workspace_bytes(1, H, geom), dtype=torch.uint8, device="cuda")
    m.svsa_block_sparse_attn(tiled["q"], tiled["k"], tiled["v"], out_t, geom, scale,
                             torch.from_numpy(o_rp.astype(np.int32)).cuda(),
                             torch.from_numpy(o_ci).cuda(), aws)
    out_n = torch.empty((1, H, N, D), dtype=torch.bfloat16, device="cuda")
    m.svsa_tile_permute(out_t, out_n, geom, inverse=True)
    torch.cuda.synchronize()
    ref_t = orc.attention(tiled_o["q"], tiled_o["k"], tiled_o["v"], o_rp, o_ci, N, Bk, scale,
                          counts=counts)
    got_t = gc.dev_to_bits(out_t)
    valid = np.concatenate([np.arange(i * Bk, i * Bk + int(counts[i])) for i in range(nb)])
    g = orc.widen(got_t[:, :, valid])
    r = ref_t[:, :, valid]
    max_abs = float(np.max(np.abs(g - r)))
    rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
    gc.log(f"  {len(tol)} tolerated mask rows; attention max_abs {max_abs:.2e} rel_l2 {rel:.2e}")
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2
    assert np.array_equal(orc.widen(gc.dev_to_bits(out_n)), orc.permute_inv(got_t, grid, tile, pad3d))


def test_tail_keys_masked_wan720():
    """The 16-token tail block of the Wan-720p shape: padded keys are excluded."""
    cfg = get_config("wan720")
    run, orun = gc.gpu_run("wan720"), gc.oracle_run("wan720")
    nb, H = cfg.nb, cfg.heads
    # every row of heads 0..1 keeps {0, nb-1}: the tail block is always involved
    rp_l, ci_l = [0], []
    for h in range(H):
        for i in range(nb):
            cols = sorted({0, i, nb - 1}) if h < 2 else [i]
            ci_l += cols
            rp_l.append(len(ci_l))
    rp = np.array(rp_l, np.int64)
    ci = np.array(ci_l, np.int32)
    out_bits = run.attention(rp, ci)
    rows = [(0, h, i) for h in (0, 1) for i in (0, 1, 500, nb - 2, nb - 1)]
    max_abs, rel = gc.attn_errors(out_bits, orun.attention_blocks(rp, ci, rows), cfg)
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2


def test_regrouped_query_blocks_cover_every_row():
    """Query blocks regrouped by their lists (SVSA_ATTN_GROUPS_BY_LIST: the shape
    is below the size where the default regroups; 64-token blocks, 270 per head: two
    windows of the grouping, a last group with two empty slots).  Each row keeps
    one of five seeded key-block templates plus its diagonal, so rows with equal
    lists lie far apart and the groups are not consecutive.  The output is
    prefilled with NaN: every valid row must be written and match the oracle; the
    positional grouping (SVSA_ATTN_POSITIONAL_GROUPS) agrees to rounding but not
    bitwise (the regrouped path ran), and a repeated call is bitwise the same."""
    import block_sparse_attention_17_amd as m
    from svsa_synth import f32_to_bf16_bits
    G = m.Geometry(10, 36, 48, 4, 4, 4)          # 17280 tokens, 270 blocks of 64
    H, D, nb = 2, 128, G.nb
    assert nb == 270 and nb % 4 == 2
    rng = np.random.default_rng(83)
    q, k, v = (rng.standard_normal((1, H, G.N_pad, D)).astype(np.float32) for _ in range(3))
    bits = [f32_to_bf16_bits(x) for x in (q, k, v)]
    templates = [sorted(rng.choice(nb, size=24, replace=False).tolist()) for _ in range(5)]
    which = rng.integers(0, 5, size=(H, nb))
    lists = [sorted(set(templates[which[h, i]]) | {i}) for h in range(H) for i in range(nb)]
    rp = np.zeros(H * nb + 1, np.int64)
    rp[1:] = np.cumsum([len(c) for c in lists])
    ci = np.array([c for cs in lists for c in cs], np.int32)
    dev = [gc.bits_to_dev(b) for b in bits]
    rpd = torch.from_numpy(rp.astype(np.int32)).cuda()
    cid = torch.from_numpy(ci).cuda()
    ws = torch.empty(m.svsa_attn_workspace_bytes(1, H, G), dtype=torch.uint8, device="cuda")

    def run(flags, c=cid):
        out = torch.full_like(dev[0], float("nan"))
        m.svsa_block_sparse_attn_ex(dev[0], dev[1], dev[2], out, G, 1 / np.sqrt(D), rpd, c, ws,
                                    flags=flags)
        torch.cuda.synchronize()
        return gc.dev_to_bits(out)

    gc.log("regrouped attention: 2 heads x 270 blocks")
    grouped, again = run(m.SVSA_ATTN_GROUPS_BY_LIST), run(m.SVSA_ATTN_GROUPS_BY_LIST)
    positional = run(m.SVSA_ATTN_POSITIONAL_GROUPS)
    assert np.array_equal(grouped, again)
    # the grouping reads the lists in 16-byte vectors from aligned addresses:
    # col_idx 4, 8 and 12 bytes past a 16-byte boundary (neighbours hold
    # out-of-range values) gives the same output bitwise
    for shift in (1, 2, 3):
        big = torch.full((ci.size + 4,), -7, dtype=torch.int32, device="cuda")
        big[shift: shift + ci.size] = cid
        view = big[shift: shift + ci.size]
        assert view.data_ptr() % 16 == 4 * shift
        assert np.array_equal(run(m.SVSA_ATTN_GROUPS_BY_LIST, view), grouped), shift
    ref = orc.attention(bits[0], bits[1], bits[2], rp, ci, G.N, G.Bk, 1 / np.sqrt(D))
    for name, o in (("regrouped", grouped), ("positional", positional)):
        got = orc.widen(o[:, :, :G.N])
        assert np.all(np.isfinite(got)), name
        err = got - ref[:, :, :G.N]
        max_abs = float(np.abs(err).max())
        rel = float(np.linalg.norm(err) / np.linalg.norm(ref[:, :, :G.N]))
        gc.log(f"{name}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
        assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2, name
    assert not np.array_equal(grouped[:, :, :G.N], positional[:, :, :G.N])


def test_all_kept_lists_keep_positional_groups():
    """Every row keeps every key block (the dense launch): the regrouping keeps
    the positional groups, and the output matches both the oracle and the call
    with SVSA_ATTN_POSITIONAL_GROUPS bitwise."""
    import block_sparse_attention_17_amd as m
    from svsa_synth import f32_to_bf16_bits
    G = m.Geometry(6, 12, 20, 4, 4, 4)           # 1440 tokens, 23 blocks (partial tail)
    H, D, nb = 2, 128, G.nb
    rng = np.random.default_rng(89)
    bits = [f32_to_bf16_bits(rng.standard_normal((1, H, G.N_pad, D)).astype(np.float32))
            for _ in range(3)]
    lists = [list(range(nb)) for _ in range(H * nb)]
    rp = np.zeros(H * nb + 1, np.int64)
    rp[1:] = np.cumsum([len(c) for c in lists])
    ci = np.array([c for cs in lists for c in cs], np.int32)
    dev = [gc.bits_to_dev(b) for b in bits]
    rpd = torch.from_numpy(rp.astype(np.int32)).cuda()
    cid = torch.from_numpy(ci).cuda()
    ws = torch.empty(m.svsa_attn_workspace_bytes(1, H, G), dtype=torch.uint8, device="cuda")
    outs = []
    for flags in (m.SVSA_ATTN_GROUPS_BY_LIST, m.SVSA_ATTN_POSITIONAL_GROUPS, 0):
        out = torch.full_like(dev[0], float("nan"))
        m.svsa_block_sparse_attn_ex(dev[0], dev[1], dev[2], out, G, 1 / np.sqrt(D), rpd, cid, ws,
                                    flags=flags)
        torch.cuda.synchronize()
        outs.append(gc.dev_to_bits(out)[:, :, :G.N])
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    ref = orc.attention(bits[0], bits[1], bits[2], rp, ci, G.N, G.Bk, 1 / np.sqrt(D))[:, :, :G.N]
    got = orc.widen(outs[0])
    err = got - ref
    assert np.abs(err).max() <= gc.MAX_ABS
    assert np.linalg.norm(err) / np.linalg.norm(ref) <= gc.REL_L2
