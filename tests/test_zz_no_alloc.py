"""svsa_block_mask_noalloc (the block mask with the library's own device
scratch: no workspace argument, no allocation) against svsa_block_mask on the
same block summaries: the CSR lists must be identical (integer work:
bit-exact).  Consecutive calls share the device scratch, so the calls run one
after the other with different sizes: Wan-720p (logits in 8 chunks of 5
heads), then the smaller 8-head case, then HV-720p in fixed-fraction mode (12
chunks of 2 heads)."""
from math import sqrt

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from tests import gpu_cases as gc  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _noalloc(run, top_p=None, keep_frac=None):
    import block_sparse_attention_17_amd as m
    cfg = run.cfg
    rows = cfg.batch * cfg.heads * cfg.nb
    rp = torch.full((rows + 1,), -1, dtype=torch.int32, device="cuda")
    ci = torch.full((rows * cfg.nb,), -1, dtype=torch.int32, device="cuda")
    gc.log(f"{cfg.name}: svsa_block_mask_noalloc top_p={top_p is not None}")
    m.svsa_block_mask_noalloc(run.bsa.qbar, run.bsa.kbar, 1 / sqrt(cfg.head_dim), rp, ci,
                              top_p=top_p, keep_frac=keep_frac, band_width=cfg.band)
    torch.cuda.synchronize()
    rph = rp.cpu().numpy().astype(np.int64)
    return rph, ci[: int(rph[-1])].cpu().numpy()


def test_noalloc_mask_equals_workspace_mask():
    cases = [("wan720", 0.9, False), ("small", 0.9, False), ("hv720", None, True)]
    for name, p, fixed in cases:
        run = gc.gpu_run(name)
        cfg = run.cfg
        tp = None if fixed else np.full(cfg.heads, p, np.float32)
        kf = run.inp.keep_frac if fixed else None
        g_rp, g_ci = _noalloc(run, top_p=tp, keep_frac=kf)
        w_rp, w_ci = run.mask(top_p=tp, keep_frac=kf, band=cfg.band)
        assert np.array_equal(g_rp, w_rp), name
        assert np.array_equal(g_ci, w_ci), name
        gc.log(f"{name}: no-alloc lists identical ({int(g_rp[-1])} kept blocks)")
