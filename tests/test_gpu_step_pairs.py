"""GPU parity of the step-pair list walk (SVSA_ATTN_STEP_PAIRS) against the
fp64 oracle, through the C ABI.

With step pairs the four query blocks of a workgroup walk their union list in
steps of one or two key blocks, two when the sets of blocks keeping them are
disjoint; every query block must still see exactly its own kept key blocks, so
the output is the oracle's attention on the oracle's lists ([PSA] App. B,
Alg. 2, per query block) within the same tolerances as the default walk.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import svsa_oracle as orc  # noqa: E402
from svsa_synth import get_config  # noqa: E402

from tests import gpu_cases as gc  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _csr(lists):
    rp = np.zeros(len(lists) + 1, np.int64)
    rp[1:] = np.cumsum([len(c) for c in lists])
    ci = np.array([c for cs in lists for c in cs], np.int32)
    return rp, ci


def _crafted_lists(nb, heads, seed):
    """Per head a keep pattern over groups of four consecutive query blocks
    (m = i % 4 the block's place in its group) that leaves many union entries
    kept by only some of the four: disjoint single keepers (1 + 1 pairs), two
    keepers (2 + 2), three keepers next to singles (3 + 1), seeded random
    subsets at several densities, and every block kept (no pair).  The
    diagonal block is always kept."""
    rng = np.random.default_rng(seed)
    dens = [0.15, 0.35, 0.6, 1.0]
    lists = []
    for h in range(heads):
        for i in range(nb):
            m = i % 4
            if h == 0:
                cols = [j for j in range(nb) if (j + m) % 4 == 0]
            elif h == 1:
                cols = [j for j in range(nb) if (j // 2 + m // 2) % 2 == 0]
            elif h == 2:
                cols = [j for j in range(nb) if j % 4 != m]
            elif h == 3:
                cols = [j for j in range(nb) if (j % 4 != m if j < nb // 2 else (j + m) % 4 == 0)]
            else:
                p = dens[(h - 4) % len(dens)]
                cols = np.nonzero(rng.random(nb) < p)[0].tolist()
            lists.append(sorted(set(cols) | {i}))
    return lists


def test_step_pairs_crafted_keep_patterns():
    """Every (head, query block) of the small config on crafted lists whose
    union entries pair in every way the pairing rules allow: equal to the
    oracle; and to the default walk within float32 summation order."""
    cfg = get_config("small")
    run, orun = gc.gpu_run("small"), gc.oracle_run("small")
    rp, ci = _csr(_crafted_lists(cfg.nb, cfg.heads, seed=91))
    got = run.attention(rp, ci, step_pairs=True)
    rows = [(0, h, i) for h in range(cfg.heads) for i in range(cfg.nb)]
    max_abs, rel = gc.attn_errors(got, orun.attention_blocks(rp, ci, rows), cfg)
    gc.log(f"step pairs, crafted patterns: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2
    base = run.attention(rp, ci, step_pairs=False)
    diff = np.abs(orc.widen(got) - orc.widen(base))
    assert float(diff.max()) <= 2e-2


STEP_CASES = [("small", None, 0.9), ("small_b2", None, 0.9), ("small_pad3d", None, 0.9),
              ("tiny_pad3d", None, 0.9), ("wan480", 6, 0.9), ("wan720", 3, 0.9),
              ("hv720", 2, "fixed"), ("maxnb", 12, 0.9)]


@pytest.mark.parametrize("name,per_head,mode", STEP_CASES)
def test_step_pairs_match_oracle(name, per_head, mode):
    """The oracle's own masks (top-p, or the fixed-fraction mode the pipeline
    runs with step pairs): every query block of the small configs, seeded
    samples of every head at full size."""
    cfg = get_config(name)
    run, orun = gc.gpu_run(name), gc.oracle_run(name)
    if mode == "fixed":
        o_rp, o_ci = orun.mask(keep_frac=run.inp.keep_frac, band=cfg.band)
    else:
        o_rp, o_ci = orun.mask(top_p=np.full(cfg.heads, mode, np.float32), band=cfg.band)
    out_bits = run.attention(o_rp, o_ci, step_pairs=True)
    if per_head is None:
        rows = [(b, h, i) for b in range(cfg.batch) for h in range(cfg.heads) for i in range(cfg.nb)]
    else:
        rows = gc.sample_rows(cfg, o_rp, per_head)
    max_abs, rel = gc.attn_errors(out_bits, orun.attention_blocks(o_rp, o_ci, rows), cfg)
    gc.log(f"step pairs {name} {mode}: {len(rows)} q-blocks, max_abs={max_abs:.3e} "
           f"rel_l2={rel:.3e}")
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2


def test_step_pairs_whole_head_hv720_fixed():
    """HunyuanVideo-720p fixed-fraction mode, every query block of the heaviest
    head (most kept blocks) with step pairs."""
    cfg = get_config("hv720")
    run, orun = gc.gpu_run("hv720"), gc.oracle_run("hv720")
    o_rp, o_ci = orun.mask(keep_frac=run.inp.keep_frac, band=cfg.band)
    out_bits = run.attention(o_rp, o_ci, step_pairs=True)
    kept = np.diff(o_rp).reshape(cfg.heads, cfg.nb).sum(1)
    h = int(np.argmax(kept))
    rows = [(0, h, i) for i in range(cfg.nb)]
    max_abs, rel = gc.attn_errors(out_bits, orun.attention_blocks(o_rp, o_ci, rows), cfg)
    gc.log(f"step pairs hv720 fixed head {h}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2


def test_step_pairs_whole_path_reproducible():
    """The whole path in fixed-fraction mode (which runs with step pairs) is
    bitwise reproducible, and agrees with the default walk on the same lists
    to float32 summation order."""
    cfg = get_config("wan480")
    run = gc.gpu_run("wan480")
    kf = np.linspace(0.1, 0.5, cfg.heads).astype(np.float32)
    outs = []
    for _ in range(2):
        o = run.bsa(run.q_dev, run.k_dev, run.v_dev, keep_frac=kf)
        torch.cuda.synchronize()
        outs.append(o.clone())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    base = run.bsa.attend(natural_out=True, step_pairs=False).clone()
    torch.cuda.synchronize()
    diff = (outs[0].float() - base.float()).abs().max().item()
    gc.log(f"wan480 fixed fraction: step pairs vs entries max |diff| {diff:.3e}")
    assert diff <= 2e-2
