"""Rules for comparing GPU results with the fp64 oracle (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module; the HIP library never does.

* Index lists (the top-p / fixed-fraction block mask, [iCATS] Sec. 3.2): equal,
  except where a difference can only come from rounding at the selection
  threshold -- a block outside the diagonal band whose score lies within 1e-4
  (relative) of the row's threshold score, or a one-block boundary shift where
  the oracle's cumulative mass is within 1e-4 of p.
* Attention output (bf16 against float64): max |err| <= 2e-2 and relative L2
  error <= 5e-3 over the valid output rows.
"""
import numpy as np

from .svsa_oracle import select_row, widen

MAX_ABS = 2e-2
REL_L2 = 5e-3
MASK_REL = 1e-4


def _rule_size(s, top_p=None, keep_frac=None):
    """Number of blocks the selection rule itself keeps in a row of scores s."""
    nb = s.shape[0]
    if keep_frac is not None:
        return min(max(int(np.ceil(float(np.float32(keep_frac)) * nb)), 1), nb)
    p = float(np.float32(top_p))
    if p >= 1:
        return nb
    cs = np.cumsum(s[np.argsort(-s, kind="stable")])
    hit = np.nonzero(cs >= p)[0]
    return int(hit[0]) + 1 if hit.size else nb


def mask_mismatch(S, heads, g_rp, g_ci, o_rp, o_ci, top_p=None, keep_frac=None, band=1):
    """Rows where the GPU's and the oracle's lists differ, as (tolerated, failing).

    S: oracle block scores, shape [..., nb, nb] with the (b, h) pairs flattened
    in row order; rows r = (b * heads + h) * nb + i; top_p / keep_frac: per-head
    float32 arrays (one of them is None).  A differing row is tolerated when
      (a) every block in the symmetric difference lies outside the band and its
          score is within 1e-4 relative of tau, the smallest score the rule
          selected in that row (fixed mode: the k-th score), or
      (b) (top-p mode) the GPU set lies between the oracle's sets at p(1-1e-4)
          and p(1+1e-4).
    """
    nb = S.shape[-1]
    S = S.reshape(-1, nb, nb)
    tolerated, failing = [], []
    for r in range(len(o_rp) - 1):
        G = g_ci[g_rp[r]: g_rp[r + 1]]
        R = o_ci[o_rp[r]: o_rp[r + 1]]
        if G.size == R.size and np.array_equal(G, R):
            continue
        bh, i = divmod(r, nb)
        h = bh % heads
        s = S[bh, i]
        Gs, Rs = set(G.tolist()), set(R.tolist())
        band_set = set(range(max(0, i - band + 1), min(nb, i + band)))
        k = _rule_size(s, top_p=None if top_p is None else top_p[h],
                       keep_frac=None if keep_frac is None else keep_frac[h])
        tau = s[np.argsort(-s, kind="stable")[k - 1]]
        ok_a = all((j not in band_set) and abs(s[j] - tau) <= MASK_REL * tau for j in Gs ^ Rs)
        ok_b = False
        if top_p is not None:
            p = float(top_p[h])
            lo = set(select_row(s, i, band, top_p=np.float32(p * (1 - MASK_REL))).tolist())
            hi = set(select_row(s, i, band, top_p=np.float32(min(1.0, p * (1 + MASK_REL)))).tolist())
            ok_b = lo <= Gs <= hi
        (tolerated if (ok_a or ok_b) else failing).append(r)
    return tolerated, failing


class ErrorAccumulator:
    """max-abs and relative L2 error of GPU rows (bf16 bits or float) against
    oracle float64 rows, over everything added; also per key (e.g. per head)."""

    def __init__(self):
        self.max_abs = 0.0
        self.err2 = 0.0
        self.ref2 = 0.0
        self.rows = 0
        self.per_key = {}

    def add(self, gpu_rows, ref_rows, key=None):
        g = widen(gpu_rows)
        d = g - ref_rows
        e2, r2 = float(np.sum(d * d)), float(np.sum(ref_rows * ref_rows))
        self.max_abs = max(self.max_abs, float(np.max(np.abs(d))) if d.size else 0.0)
        self.err2 += e2
        self.ref2 += r2
        self.rows += ref_rows.shape[0]
        if key is not None:
            k = self.per_key.setdefault(key, [0.0, 0.0])
            k[0] += e2
            k[1] += r2

    @property
    def rel_l2(self):
        return float(np.sqrt(self.err2 / self.ref2)) if self.ref2 > 0 else 0.0

    def rel_l2_per_key(self):
        return {k: float(np.sqrt(e / r)) if r > 0 else 0.0 for k, (e, r) in self.per_key.items()}
