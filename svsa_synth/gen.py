"""Seeded synthetic Q, K, V in natural (t, h, w) row-major token order.

Recipe (stands in for Wan2.1 / HunyuanVideo attention activations, which are
not available):

* Q, K, V ~ N(0, 1) i.i.d. float32, one independent PCG64 stream per
  (seed, config id, tensor id, batch, head).
* Q and K also get ``s_h * PE(t, h, w)``: the *same* smooth 3D sinusoidal
  positional vector for both.  Channels are split D/4 | 3D/8 | 3D/8 over the
  t | h | w axes; an axis of length L with n sin/cos pairs uses frequencies
  w_k = f_h * (pi/4) * ((pi/L) / (pi/4)) ** (k / (n-1)), laid out as
  [sin(pos*w_0..w_{n-1}), cos(pos*w_0..w_{n-1})]; the whole vector is scaled by
  sqrt(64/D).  This imitates the locality and per-axis periodicity that the
  PSA paper derives for RoPE-3D logits (its Sec. 3.1, eq. 1-5).
* s_h = 1.5 (tiny, small) or s_h ~ U[0.5, 3.0] per head (Wan/HV shapes);
  f_h = 1, except the small case where f_h = 2 ** U[-2, 0] per head.
* Values are formed in float32 and rounded to bf16 (round to nearest even).
  The tiny case also keeps the float32 values.
* The per-head keep fraction of the fixed-sparsity mode is drawn here too,
  keep_frac_h ~ U[0.1, 0.5] (float32), so both sides receive it as an input.

Only draws and rounding live here; no step of the attention method does.
"""
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
import os

import numpy as np

from .configs import Config, get_config

Q_ID, K_ID, V_ID = 0, 1, 2
_PARAM_ID = 100


def f32_to_bf16_bits(x):
    """float32 array -> uint16 bf16 bit patterns, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 rounding expects finite values")
    u = x.view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u            # cannot wrap: finite float32 bits are <= 0xFF7FFFFF
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    """uint16 bf16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def head_params(cfg: Config, seed: int):
    """Per-head positional scale s_h, frequency multiplier f_h, keep fraction."""
    g = _rng(seed, cfg.cfg_id, _PARAM_ID)
    H = cfg.heads
    u_scale = g.uniform(0.5, 3.0, size=H)
    u_freq = g.uniform(-2.0, 0.0, size=H)
    u_keep = g.uniform(0.1, 0.5, size=H)
    scales = np.full(H, 1.5) if cfg.pe_scale == "fixed" else u_scale
    fmuls = 2.0 ** u_freq if cfg.pe_freq == "per_head" else np.ones(H)
    return scales.astype(np.float64), fmuls.astype(np.float64), u_keep.astype(np.float32)


def positional_term(grid, head_dim, fmul=1.0):
    """PE(t, h, w) as float32 [T*H*W, D] in natural row-major token order."""
    T, H, W = grid
    D = head_dim
    d_t = D // 4
    d_h = (D - d_t) // 2
    d_w = D - d_t - d_h
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    parts = []
    for pos, L, d_a in ((t, T, d_t), (h, H, d_h), (w, W, d_w)):
        n = d_a // 2
        hi, lo = np.pi / 4.0, np.pi / L
        k = np.arange(n) / max(n - 1, 1)
        omega = fmul * hi * (lo / hi) ** k
        ang = pos.reshape(-1, 1).astype(np.float64) * omega[None, :]
        parts += [np.sin(ang), np.cos(ang)]
    pe = np.concatenate(parts, axis=1) * np.sqrt(64.0 / D)
    assert pe.shape == (T * H * W, D)
    return pe.astype(np.float32)


@dataclass
class Inputs:
    cfg: Config
    seed: int
    q: np.ndarray          # uint16 bf16 bits [B, Hh, N, D]
    k: np.ndarray
    v: np.ndarray
    scales: np.ndarray     # s_h
    fmuls: np.ndarray      # f_h
    keep_frac: np.ndarray  # float32 [Hh]
    q32: np.ndarray = None  # float32 values before rounding (tiny case only)
    k32: np.ndarray = None
    v32: np.ndarray = None

    @property
    def heads(self):
        return self.q.shape[1]


def make_inputs(cfg, seed=0, heads=None, keep_f32=None, threads=None):
    """Build the seeded inputs of ``cfg`` (a Config or a config name).

    ``heads`` optionally restricts generation to a list of head indices (the
    draws of a head do not depend on which other heads are generated).
    """
    if isinstance(cfg, str):
        cfg = get_config(cfg)
    head_list = list(range(cfg.heads)) if heads is None else [int(h) for h in heads]
    if keep_f32 is None:
        keep_f32 = cfg.src_dtype == "fp32"
    scales, fmuls, keep = head_params(cfg, seed)
    B, N, D = cfg.batch, cfg.N, cfg.head_dim
    nh = len(head_list)
    out = {n: np.empty((B, nh, N, D), np.uint16) for n in "qkv"}
    f32 = {n: np.empty((B, nh, N, D), np.float32) for n in "qkv"} if keep_f32 else None
    pe_cache = {}

    def pe_for(f):
        key = float(f)
        if key not in pe_cache:
            pe_cache[key] = positional_term(cfg.grid, D, f)
        return pe_cache[key]

    for hi in head_list:  # fill the cache serially (cheap, avoids races)
        pe_for(fmuls[hi])

    def one(job):
        b, slot, h = job
        pe = pe_for(fmuls[h])
        for name, tid in (("q", Q_ID), ("k", K_ID), ("v", V_ID)):
            x = _rng(seed, cfg.cfg_id, tid, b, h).standard_normal((N, D), dtype=np.float32)
            if name != "v":
                x += np.float32(scales[h]) * pe
            out[name][b, slot] = f32_to_bf16_bits(x)
            if f32 is not None:
                f32[name][b, slot] = x

    jobs = [(b, s, h) for b in range(B) for s, h in enumerate(head_list)]
    nthreads = threads or min(len(jobs), max(1, min(16, os.cpu_count() or 1)))
    if nthreads > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, jobs))
    else:
        for j in jobs:
            one(j)
    sel = np.array(head_list)
    return Inputs(cfg, seed, out["q"], out["k"], out["v"], scales[sel], fmuls[sel], keep[sel],
                  *( (f32["q"], f32["k"], f32["v"]) if f32 is not None else (None, None, None)))


_STRIPE_ID = 200


def stripe_params(heads, seed=0, stream=0):
    """Seeded per-head stripe-mask parameters (Tw, To, Ts, Sw, So, Ss), int32
    [heads, 6], drawn uniformly from the search ranges the PSA paper lists for
    Wan 2.1 (App., PSA-Search settings): Tw < 7, To in {0, +-1, +-2}, Ts in
    {1, 2, 3, inf}, Sw < 5, So in {0, +-1}, Ss in {1, 3, 5, 6, inf}; inf is
    encoded as 0.  Draws only: the mask itself is built elsewhere."""
    g = _rng(seed, _STRIPE_ID, stream)
    tw = g.integers(1, 7, size=heads)
    to = g.choice([0, 1, -1, 2, -2], size=heads)
    ts = g.choice([1, 2, 3, 0], size=heads)
    sw = g.integers(1, 5, size=heads)
    so = g.choice([0, 1, -1], size=heads)
    ss = g.choice([1, 3, 5, 6, 0], size=heads)
    return np.stack([tw, to, ts, sw, so, ss], axis=1).astype(np.int32)


def flow_sigmas(steps, shift=5.0):
    """Noise levels of a flow-matching sampler (x = (1 - s) x0 + s eps) with a
    time shift: t_k = 1 - k / steps, s_k = shift t / (1 + (shift - 1) t).  An
    input of the SNR-guided top-p schedule (the pages give no noise schedule;
    this stands in for the denoising loop of a rectified-flow video model)."""
    t = 1.0 - np.arange(steps, dtype=np.float64) / steps
    return shift * t / (1.0 + (shift - 1.0) * t)


_CLUSTER_ID = 300


def cluster_seeds(n, clusters, batch, heads, seed=0, stream=0):
    """Seeded initial centroid picks: int64 [batch, heads, clusters] distinct
    token indices per (b, h), ascending (k-means starts from these tokens)."""
    out = np.empty((batch, heads, clusters), np.int64)
    for b in range(batch):
        for h in range(heads):
            g = _rng(seed, _CLUSTER_ID, stream, b, h)
            out[b, h] = np.sort(g.choice(n, size=clusters, replace=False))
    return out


def cluster_labels(n, clusters, batch, heads, seed=0, stream=1, empty=0):
    """Seeded labels int32 [batch, heads, n], uniform over the clusters except
    `empty` seeded clusters per (b, h) that receive no token."""
    out = np.empty((batch, heads, n), np.int32)
    for b in range(batch):
        for h in range(heads):
            g = _rng(seed, _CLUSTER_ID, stream, b, h)
            used = np.sort(g.choice(clusters, size=clusters - empty, replace=False))
            out[b, h] = used[g.integers(0, used.size, size=n)]
    return out
