"""Variable-size (cluster) blocks on the GPU against the fp64 oracle, through
the C ABI: k-means steps, the metric, the padded layout and permutation
(integer work: bit-exact), cluster means and the cluster mask, and attention
over kept key clusters.

Tolerances: layout / permutation bit-exact; means and metric to float64
rounding (1e-13 relative); a k-means label may differ from the oracle's only
where the two centroids' distances differ by less than the assignment
kernel's error bound (bf16 x against a two-term bf16 split of G c, fp32
accumulation: 2^-12 |x| max|G c| + 2^-20 max|c^T G c|); the mask only at
scores within 1e-4 of the row's threshold; attention max-abs 2e-2, rel-L2 5e-3.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import svsa_oracle as orc  # noqa: E402
from svsa_synth import cluster_labels, cluster_seeds, get_config  # noqa: E402

from tests import gpu_cases as gc  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _m():
    import block_sparse_attention_17_amd as m
    return m


def _metric(heads, D, seed):
    """Seeded symmetric positive definite metrics float64 [1, heads, D, D]."""
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((heads, D, D))
    return (np.matmul(A, np.swapaxes(A, 1, 2)) / D + np.eye(D))[None]


def _dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).cuda()


def _gpu_kmeans(x_bits, cents0, iters, G):
    m = _m()
    B, H, N, D = x_bits.shape
    C = cents0.shape[2]
    cents = _dev(cents0, torch.float64)
    labels = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    sizes = torch.empty((B, H, C), dtype=torch.int32, device="cuda")
    ws = torch.empty(m.svsa_kmeans_workspace_bytes(B, H, N, C, D), dtype=torch.uint8,
                     device="cuda")
    met = None if G is None else _dev(G, torch.float64)
    gc.log(f"k-means on the GPU: {B}x{H}x{N}x{D}, {C} clusters, {iters} iterations, "
           f"metric={G is not None}")
    m.svsa_kmeans(gc.bits_to_dev(x_bits), cents, labels, sizes, ws, iters, metric=met)
    torch.cuda.synchronize()
    return cents.cpu().numpy(), labels.cpu().numpy(), sizes.cpu().numpy()


def _assign_tolerance(x, cents, G):
    """Per-token bound on the assignment kernel's distance error (both sides)."""
    gcv = cents if G is None else cents @ G
    cq = np.abs(np.einsum("cd,cd->c", cents, gcv))
    xn = np.linalg.norm(x, axis=1)
    return 2.0 ** -12 * xn * np.linalg.norm(gcv, axis=1).max() + 2.0 ** -20 * cq.max()


@pytest.mark.parametrize("name,C,use_metric", [("small", 32, False), ("small", 32, True),
                                                ("tiny_pad3d", 12, True)])
def test_kmeans_one_iteration_matches_oracle(name, C, use_metric):
    inp = gc.inputs(name)
    x = inp.q
    B, H, N, D = x.shape
    seeds = cluster_seeds(N, C, B, H, seed=3)
    xw = orc.widen(x)
    cents0 = np.stack([np.stack([xw[b, h, seeds[b, h]] for h in range(H)]) for b in range(B)])
    G = _metric(H, D, 5) if use_metric else None
    cents, labels, sizes = _gpu_kmeans(x, cents0, 1, G)
    tolerated = 0
    for b in range(B):
        for h in range(H):
            Gh = None if G is None else G[b, h]
            d = orc.quad_distances(xw[b, h], cents0[b, h], Gh)
            lab_o = np.argmin(d, axis=1)
            diff = np.nonzero(labels[b, h] != lab_o)[0]
            tol = _assign_tolerance(xw[b, h], cents0[b, h], Gh)
            gap = d[diff, labels[b, h][diff]] - d[diff, lab_o[diff]]
            assert np.all(gap <= tol[diff]), (b, h, diff[gap > tol[diff]][:5])
            tolerated += diff.size
            if diff.size == 0:
                c_o, s_o, _ = orc.kmeans(xw[b, h], cents0[b, h], 1, Gh)
                assert np.array_equal(sizes[b, h], s_o)
                np.testing.assert_allclose(cents[b, h], c_o, rtol=1e-13, atol=1e-15)
            # every head (also one with tolerated near-tie labels): the update
            # step on the GPU's own labels
            _check_update(x[b:b + 1, h:h + 1], labels[b, h], cents0[b, h], cents[b, h],
                          sizes[b, h])
    gc.log(f"{name}: {tolerated} near-tie labels of {B * H * N}")
    assert tolerated <= max(2, B * H * N // 1000)


def _check_update(x_bits, labels, cents0, cents, sizes):
    """The means step of one head against the oracle on the GPU's labels:
    sizes are the label counts, a non-empty cluster's centroid is the float64
    mean of its members, an empty cluster keeps its initial centroid."""
    C = cents0.shape[0]
    m_o, s_o = orc.cluster_means(x_bits, labels[None, None], C)
    assert np.array_equal(sizes, s_o[0, 0])
    ne = s_o[0, 0] > 0
    np.testing.assert_allclose(cents[ne], m_o[0, 0][ne], rtol=1e-13, atol=1e-15)
    assert np.array_equal(cents[~ne], cents0[~ne])


def _blobs(heads, n, C, D, seed):
    """Seeded well-separated clusters (centres N(0, 25), unit noise), bf16 bits,
    and one seeded member of each blob as its initial centroid."""
    from svsa_synth import f32_to_bf16_bits
    rng = np.random.default_rng(seed)
    centres = 5.0 * rng.standard_normal((heads, C, D))
    lab = rng.integers(0, C, size=(heads, n))
    lab[:, :C] = np.arange(C)
    x = centres[np.arange(heads)[:, None], lab] + rng.standard_normal((heads, n, D))
    bits = f32_to_bf16_bits(x.astype(np.float32))[None]
    return bits, np.broadcast_to(np.arange(C), (1, heads, C))


def test_kmeans_iterations_match_oracle():
    """Four Lloyd iterations under a metric, exactly equal to the oracle's on
    well-separated blobs (every assignment margin far above the kernel's
    error bound, checked)."""
    H, N, D, C = 4, 2048, 64, 8
    x, seeds = _blobs(H, N, C, D, seed=21)
    xw = orc.widen(x)
    cents0 = np.stack([xw[0, h, seeds[0, h]] for h in range(H)])[None]
    G = _metric(H, D, 6)
    cents, labels, sizes = _gpu_kmeans(x, cents0, 4, G)
    for h in range(H):
        c = cents0[0, h].copy()
        for _ in range(4):
            d = orc.quad_distances(xw[0, h], c, G[0, h])
            srt = np.sort(d, axis=1)
            assert np.all(srt[:, 1] - srt[:, 0] > 4 * _assign_tolerance(xw[0, h], c, G[0, h]))
            c, _, _ = orc.kmeans(xw[0, h], c, 1, G[0, h])
        c_o, s_o, l_o = orc.kmeans(xw[0, h], cents0[0, h], 4, G[0, h])
        assert np.array_equal(labels[0, h], l_o)
        assert np.array_equal(sizes[0, h], s_o)
        np.testing.assert_allclose(cents[0, h], c_o, rtol=1e-12, atol=1e-14)


def test_kmeans_loop_is_chained_steps_and_ends_on_means():
    """On the real inputs: one call of 4 iterations equals 4 chained calls of
    one iteration (bitwise), and the returned centroids are the means of the
    returned labels (empty clusters aside)."""
    inp = gc.inputs("small")
    x = inp.q[:, :4]
    B, H, N, D = x.shape
    C = 16
    seeds = cluster_seeds(N, C, B, H, seed=4)
    xw = orc.widen(x)
    cents0 = np.stack([np.stack([xw[b, h, seeds[b, h]] for h in range(H)]) for b in range(B)])
    G = _metric(H, D, 6)
    c4, l4, s4 = _gpu_kmeans(x, cents0, 4, G)
    c = cents0
    for _ in range(4):
        c, l1, s1 = _gpu_kmeans(x, c, 1, G)
    assert np.array_equal(l4, l1) and np.array_equal(s4, s1) and np.array_equal(c4, c)
    for h in range(H):
        for k in range(C):
            members = xw[0, h, l4[0, h] == k]
            assert members.shape[0] == s4[0, h, k]
            if members.shape[0]:
                np.testing.assert_allclose(c4[0, h, k], members.mean(axis=0), rtol=1e-12,
                                           atol=1e-14)


def test_cluster_metric_matches_oracle():
    m = _m()
    rng = np.random.default_rng(12)
    H, C, D = 3, 50, 128
    cents = rng.standard_normal((1, H, C, D))
    sizes = rng.integers(0, 40, size=(1, H, C)).astype(np.int32)
    out = torch.empty((1, H, D, D), dtype=torch.float64, device="cuda")
    m.svsa_cluster_metric(_dev(cents, torch.float64), _dev(sizes, torch.int32), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for h in range(H):
        ref = orc.cluster_metric(cents[0, h], sizes[0, h])
        np.testing.assert_allclose(got[0, h], ref, rtol=1e-12, atol=1e-10)


def _gpu_layout(labels, C, align):
    m = _m()
    B, H, N = labels.shape
    cap = m.svsa_cluster_capacity(N, C, align)
    i32 = dict(dtype=torch.int32, device="cuda")
    start = torch.empty((B, H, C + 1), **i32)
    sizes = torch.empty((B, H, C), **i32)
    slot = torch.empty((B, H, N), **i32)
    token = torch.full((B, H, cap), -7, **i32)
    ws = torch.empty(m.svsa_cluster_layout_workspace_bytes(B, H, N, C), dtype=torch.uint8,
                     device="cuda")
    m.svsa_cluster_layout(_dev(labels, torch.int32), C, align, start, sizes, slot, token, ws)
    torch.cuda.synchronize()
    return start, sizes, slot, token, cap


@pytest.mark.parametrize("align", [1, 32, 64])
def test_cluster_layout_bit_exact(align):
    N, C = 3000, 45
    labels = cluster_labels(N, C, 2, 3, seed=7, empty=5)
    start, sizes, slot, token, cap = _gpu_layout(labels, C, align)
    start, sizes, slot, token = (t.cpu().numpy() for t in (start, sizes, slot, token))
    for b in range(2):
        for h in range(3):
            st_o, sl_o, tk_o = orc.cluster_layout(labels[b, h], C, align)
            assert np.array_equal(start[b, h], st_o)
            assert np.array_equal(sizes[b, h], np.bincount(labels[b, h], minlength=C))
            assert np.array_equal(slot[b, h], sl_o)
            assert np.array_equal(token[b, h, : st_o[-1]], tk_o)
            assert st_o[-1] <= cap


def test_cluster_permute_bit_exact_and_round_trip():
    m = _m()
    inp = gc.inputs("small")
    B, H, N, D = inp.k.shape
    C, align = 40, 64
    labels = cluster_labels(N, C, B, H, seed=8, empty=3)
    start, sizes, slot, token, cap = _gpu_layout(labels, C, align)
    kd = gc.bits_to_dev(inp.k)
    kp = torch.full((B, H, cap, D), 3.0, dtype=torch.bfloat16, device="cuda")
    m.svsa_cluster_permute(kd, kp, N, C, align, token, start)
    back = torch.empty_like(kd)
    m.svsa_cluster_permute(kp, back, N, C, align, slot, start, inverse=True)
    torch.cuda.synchronize()
    kp_bits = gc.dev_to_bits(kp)
    for h in range(H):
        st_o, _, tk_o = orc.cluster_layout(labels[0, h], C, align)
        ok = tk_o >= 0
        assert np.array_equal(kp_bits[0, h, : st_o[-1]][ok], inp.k[0, h, tk_o[ok]])
        assert np.all(kp_bits[0, h, : st_o[-1]][~ok] == 0)
    assert torch.equal(back.view(torch.int16), kd.view(torch.int16))


class _ClusterCase:
    """Seeded labels on a config's inputs: GPU layout / means / permutation and
    the oracle's means, scores and mask on the same labels."""

    def __init__(self, name, nq, nk, align, k_empty=4, seed=9):
        m = _m()
        self.cfg = cfg = get_config(name)
        self.inp = inp = gc.inputs(name)
        B, H, N, D = inp.q.shape
        self.B, self.H, self.N, self.D, self.nq, self.nk, self.align = B, H, N, D, nq, nk, align
        self.qlab = cluster_labels(N, nq, B, H, seed=seed, stream=1)
        self.klab = cluster_labels(N, nk, B, H, seed=seed, stream=2, empty=k_empty)
        gc.log(f"{name}: cluster case nq={nq} nk={nk} align={align}")
        f64 = dict(dtype=torch.float64, device="cuda")
        i32 = dict(dtype=torch.int32, device="cuda")
        self.qd, self.kd, self.vd = (gc.bits_to_dev(a) for a in (inp.q, inp.k, inp.v))
        # GPU means
        self.qbar = torch.zeros((B, H, nq, D), **f64)
        self.kbar = torch.zeros((B, H, nk, D), **f64)
        self.qs = torch.empty((B, H, nq), **i32)
        self.ks = torch.empty((B, H, nk), **i32)
        ws = torch.empty(max(m.svsa_cluster_means_workspace_bytes(B, H, N, nq),
                             m.svsa_cluster_means_workspace_bytes(B, H, N, nk)),
                         dtype=torch.uint8, device="cuda")
        m.svsa_cluster_means(self.qd, _dev(self.qlab, torch.int32), self.qbar, self.qs, ws)
        m.svsa_cluster_means(self.kd, _dev(self.klab, torch.int32), self.kbar, self.ks, ws)
        # GPU layouts and permuted tensors
        self.q_start, _, self.q_slot, self.q_token, self.cap_q = _gpu_layout(self.qlab, nq, align)
        self.k_start, _, _, self.k_token, self.cap_k = _gpu_layout(self.klab, nk, align)
        bf = dict(dtype=torch.bfloat16, device="cuda")
        self.qp = torch.empty((B, H, self.cap_q, D), **bf)
        self.kp = torch.empty((B, H, self.cap_k, D), **bf)
        self.vp = torch.empty((B, H, self.cap_k, D), **bf)
        self.op = torch.empty((B, H, self.cap_q, D), **bf)
        m.svsa_cluster_permute(self.qd, self.qp, N, nq, align, self.q_token, self.q_start)
        m.svsa_cluster_permute(self.kd, self.kp, N, nk, align, self.k_token, self.k_start)
        m.svsa_cluster_permute(self.vd, self.vp, N, nk, align, self.k_token, self.k_start)
        torch.cuda.synchronize()
        # oracle on the same labels
        self.qbar_o, self.qs_o = orc.cluster_means(inp.q, self.qlab, nq)
        self.kbar_o, self.ks_o = orc.cluster_means(inp.k, self.klab, nk)
        self.S = np.stack([np.stack([orc.cluster_scores(self.qbar_o[b, h], self.kbar_o[b, h],
                                                        self.ks_o[b, h], 1 / np.sqrt(D))
                                     for h in range(H)]) for b in range(B)])

    def gpu_mask(self, top_p):
        m = _m()
        B, H = self.B, self.H
        rows = B * H * self.nq
        rp = torch.empty(rows + 1, dtype=torch.int32, device="cuda")
        ci = torch.empty(rows * self.nk, dtype=torch.int32, device="cuda")
        ws = torch.empty(m.svsa_cluster_mask_workspace_bytes(B, H, self.nq, self.nk),
                         dtype=torch.uint8, device="cuda")
        m.svsa_cluster_mask(self.qbar, self.kbar, self.ks, 1 / np.sqrt(self.D), rp, ci, ws,
                            top_p=top_p)
        torch.cuda.synchronize()
        rph = rp.cpu().numpy().astype(np.int64)
        return rph, ci[: int(rph[-1])].cpu().numpy()

    def gpu_attention(self, rp, ci, fill=None):
        m = _m()
        ws = torch.empty(m.svsa_cluster_attn_workspace_bytes(self.B, self.H, self.N, self.nq,
                                                             self.N, self.nk, self.align),
                         dtype=torch.uint8, device="cuda")
        if fill is not None:       # stale workspace contents must not matter
            ws.fill_(fill)
        gc.log(f"{self.cfg.name}: cluster attention on {int(rp[-1])} kept cluster pairs")
        m.svsa_cluster_attn(self.qp, self.kp, self.vp, self.op, self.N, self.q_start, self.qs,
                            self.N, self.k_start, self.ks, self.align, 1 / np.sqrt(self.D),
                            _dev(rp.astype(np.int32), torch.int32),
                            _dev(ci.astype(np.int32), torch.int32), ws)
        out = torch.empty_like(self.qd)
        m.svsa_cluster_permute(self.op, out, self.N, self.nq, self.align, self.q_slot,
                               self.q_start, inverse=True)
        torch.cuda.synchronize()
        return gc.dev_to_bits(out)


def _cluster_mask_failures(S, g_rp, g_ci, o_rp, o_ci, top_p):
    bad = []
    B, H, nq, nk = S.shape
    for r in range(len(o_rp) - 1):
        G = set(g_ci[g_rp[r]: g_rp[r + 1]].tolist())
        R = set(o_ci[o_rp[r]: o_rp[r + 1]].tolist())
        if G == R:
            continue
        b_h, i = divmod(r, nq)
        b, h = divmod(b_h, H)
        s = S[b, h, i]
        tau = s[list(R)].min()
        if not all(abs(s[j] - tau) <= gc.MASK_REL * tau for j in G ^ R):
            bad.append(r)
    return bad


@pytest.mark.parametrize("name,nq,nk,align", [("small", 24, 40, 64), ("tiny_pad3d", 6, 9, 64)])
def test_cluster_means_and_mask_match_oracle(name, nq, nk, align):
    c = _ClusterCase(name, nq, nk, align)
    assert np.array_equal(c.qs.cpu().numpy(), c.qs_o)
    assert np.array_equal(c.ks.cpu().numpy(), c.ks_o)
    kb = c.kbar.cpu().numpy()
    ne = c.ks_o > 0
    np.testing.assert_allclose(c.qbar.cpu().numpy(), c.qbar_o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(kb[ne], c.kbar_o[ne], rtol=1e-13, atol=1e-15)
    for p in (0.5, 0.9, 1.0):
        tp = np.full(c.H, p, np.float32)
        g_rp, g_ci = c.gpu_mask(tp)
        o_rp, o_ci = orc.cluster_mask(c.S, top_p=tp)
        assert np.array_equal(g_rp.shape, o_rp.shape)
        bad = _cluster_mask_failures(c.S, g_rp, g_ci, o_rp, o_ci, tp)
        assert not bad, (p, bad[:5])


@pytest.mark.parametrize("name,nq,nk,align", [("small", 24, 40, 64), ("small", 24, 40, 32),
                                               ("tiny_pad3d", 6, 9, 64)])
def test_cluster_attention_matches_oracle(name, nq, nk, align):
    c = _ClusterCase(name, nq, nk, align)
    tp = np.full(c.H, 0.9, np.float32)
    o_rp, o_ci = orc.cluster_mask(c.S, top_p=tp)
    out = c.gpu_attention(o_rp, o_ci)
    g_all, r_all = [], []
    scale = 1 / np.sqrt(c.D)
    for b in range(c.B):
        for h in range(c.H):
            for i in range(nq):
                r = (b * c.H + h) * nq + i
                toks, ref = orc.cluster_attention_rows(c.inp.q[b, h], c.inp.k[b, h],
                                                       c.inp.v[b, h], c.qlab[b, h],
                                                       c.klab[b, h], i, o_ci[o_rp[r]: o_rp[r + 1]],
                                                       scale)
                g_all.append(orc.widen(out[b, h, toks]).ravel())
                r_all.append(ref.ravel())
    g, r = np.concatenate(g_all), np.concatenate(r_all)
    max_abs = float(np.abs(g - r).max())
    rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
    gc.log(f"{name} align {align}: cluster attention max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2


@pytest.mark.parametrize("align", [64, 32])
def test_cluster_attention_empty_rows_give_zeros(align):
    """Empty rows give zeros and the other rows match the oracle, with every
    workspace byte 0xFF before the call (the padded tail of each head's query
    layout is a group with an empty union list)."""
    c = _ClusterCase("small", 24, 40, align)
    nq, H = c.nq, c.H
    cols = [[] if (i % 5 == 0) else [i % c.nk, (3 * i) % c.nk] for _ in range(H) for i in range(nq)]
    rp = np.zeros(H * nq + 1, np.int64)
    rp[1:] = np.cumsum([len(x) for x in cols])
    ci = np.array([j for x in cols for j in x], np.int32)
    out = c.gpu_attention(rp, ci, fill=0xFF)
    g_all, r_all = [], []
    for h in range(H):
        for i in range(nq):
            toks = np.nonzero(c.qlab[0, h] == i)[0]
            if i % 5 == 0:
                assert np.all(orc.widen(out[0, h, toks]) == 0)
                continue
            r = h * nq + i
            kept = ci[rp[r]: rp[r + 1]]
            if not np.isin(c.klab[0, h], kept).any():     # only empty key clusters kept
                assert np.all(orc.widen(out[0, h, toks]) == 0)
                continue
            toks, ref = orc.cluster_attention_rows(c.inp.q[0, h], c.inp.k[0, h], c.inp.v[0, h],
                                                   c.qlab[0, h], c.klab[0, h], i, kept,
                                                   1 / np.sqrt(c.D))
            g_all.append(orc.widen(out[0, h, toks]).ravel())
            r_all.append(ref.ravel())
    g, r = np.concatenate(g_all), np.concatenate(r_all)
    assert np.abs(g - r).max() <= gc.MAX_ABS
    assert np.linalg.norm(g - r) / np.linalg.norm(r) <= gc.REL_L2


def test_clustered_attention_all_kept_equals_dense():
    """Whole cluster path (k-means both ways, layouts, mask, attention, token
    order) with every key cluster kept equals dense attention, on the first
    (feature-space) call and on a warm call under the cluster metrics."""
    m = _m()
    inp = gc.inputs("small")
    B, H, N, D = inp.q.shape
    nq, nk = 16, 32
    ca = m.ClusteredAttention(B, H, D, N, nq, nk, align=64, q_iters=2, k_iters=2)
    xq, xk = orc.widen(inp.q), orc.widen(inp.k)
    sq = cluster_seeds(N, nq, B, H, seed=1, stream=1)
    sk = cluster_seeds(N, nk, B, H, seed=1, stream=2)
    qc = np.stack([np.stack([xq[b, h, sq[b, h]] for h in range(H)]) for b in range(B)])
    kc = np.stack([np.stack([xk[b, h, sk[b, h]] for h in range(H)]) for b in range(B)])
    ca.set_centroids(_dev(qc, torch.float64), _dev(kc, torch.float64))
    ref = orc.dense_attention(inp.q, inp.k, inp.v, 1 / np.sqrt(D))
    qd, kd, vd = (gc.bits_to_dev(a) for a in (inp.q, inp.k, inp.v))
    for call in range(2):
        gc.log(f"clustered pipeline call {call}")
        out = ca(qd, kd, vd, top_p=np.ones(H, np.float32))
        torch.cuda.synchronize()
        got = orc.widen(gc.dev_to_bits(out))
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert np.abs(got - ref).max() <= gc.MAX_ABS and rel <= gc.REL_L2
        assert int(ca.row_ptr[-1].item()) == B * H * nq * nk
        sizes = ca.qsize.cpu().numpy()
        assert sizes.sum() == B * H * N


@pytest.mark.parametrize("N,nq,nk,block", [(3000, 40, 30, 64), (2048, 24, 40, 32),
                                           (500, 12, 9, 8)])
def test_tail_merge_bit_exact(N, nq, nk, block):
    """Integer work: labels and merged kept sets equal the oracle's exactly, on
    seeded labels and kept sets with planted identical rows."""
    m = _m()
    H = 3
    rng = np.random.default_rng(N + nq)
    labels = cluster_labels(N, nq, 1, H, seed=nq, stream=3, empty=2)
    K = rng.random((H, nq, nk)) < 0.35
    K[:, 5] = K[:, 2]
    K[:, nq - 1] = K[:, 0]
    rp = np.zeros(H * nq + 1, np.int64)
    rp[1:] = np.cumsum(K.reshape(-1, nk).sum(1))
    ci = np.concatenate([np.nonzero(r)[0] for r in K.reshape(-1, nk)]).astype(np.int32)
    lab_d = _dev(labels, torch.int32)
    rp2 = torch.empty(H * nq + 1, dtype=torch.int32, device="cuda")
    ci2 = torch.empty(H * nq * nk, dtype=torch.int32, device="cuda")
    ws = torch.empty(m.svsa_tail_merge_workspace_bytes(1, H, N, nq, nk), dtype=torch.uint8,
                     device="cuda")
    gc.log(f"tail merge on the GPU: {H} heads, {N} tokens, {nq} clusters, block {block}")
    m.svsa_tail_merge(lab_d, nq, nk, block, _dev(rp.astype(np.int32), torch.int32),
                      _dev(ci, torch.int32), rp2, ci2, ws)
    torch.cuda.synchronize()
    g_lab = lab_d.cpu().numpy()
    g_rp = rp2.cpu().numpy().astype(np.int64)
    g_ci = ci2[: int(g_rp[-1])].cpu().numpy()
    moved = 0
    for h in range(H):
        o_lab, o_R, _ = orc.tail_merge(labels[0, h], K[h], block)
        assert np.array_equal(g_lab[0, h], o_lab), h
        for i in range(nq):
            r = h * nq + i
            assert np.array_equal(g_ci[g_rp[r]: g_rp[r + 1]], np.nonzero(o_R[i])[0]), (h, i)
        moved += int(np.sum(o_lab != labels[0, h]))
    gc.log(f"tail merge: {moved} tokens relabelled")
    assert moved > 0


def test_clustered_attention_tail_merge_all_kept_equals_dense():
    """With every key cluster kept all kept sets are equal, so tail merging
    folds each head into one query cluster; the output is still dense
    attention."""
    m = _m()
    inp = gc.inputs("small")
    B, H, N, D = inp.q.shape
    nq, nk = 16, 32
    ca = m.ClusteredAttention(B, H, D, N, nq, nk, align=64, q_iters=2, k_iters=2,
                              tail_merge=True)
    xq, xk = orc.widen(inp.q), orc.widen(inp.k)
    sq = cluster_seeds(N, nq, B, H, seed=1, stream=1)
    sk = cluster_seeds(N, nk, B, H, seed=1, stream=2)
    qc = np.stack([np.stack([xq[b, h, sq[b, h]] for h in range(H)]) for b in range(B)])
    kc = np.stack([np.stack([xk[b, h, sk[b, h]] for h in range(H)]) for b in range(B)])
    ca.set_centroids(_dev(qc, torch.float64), _dev(kc, torch.float64))
    ref = orc.dense_attention(inp.q, inp.k, inp.v, 1 / np.sqrt(D))
    qd, kd, vd = (gc.bits_to_dev(a) for a in (inp.q, inp.k, inp.v))
    out = ca(qd, kd, vd, top_p=np.ones(H, np.float32))
    torch.cuda.synchronize()
    got = orc.widen(gc.dev_to_bits(out))
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert np.abs(got - ref).max() <= gc.MAX_ABS and rel <= gc.REL_L2
    sizes = ca.qsize.cpu().numpy().reshape(B * H, nq)
    assert np.all(np.count_nonzero(sizes, axis=1) == 1)


# ---------------------------------------------------------------- full size
def _wan720_heads(heads=(0, 17)):
    inp = gc.inputs("wan720")
    sel = list(heads)
    return inp.q[:, sel], inp.k[:, sel], inp.v[:, sel]


def test_kmeans_assignment_full_size_sampled():
    """Wan-720p shape (75,600 tokens, D 128, 1000 centroids, metric): one
    assignment; 3000 seeded tokens per head re-decided by the oracle."""
    q, k, _ = _wan720_heads()
    B, H, N, D = k.shape
    C = 1000
    seeds = cluster_seeds(N, C, B, H, seed=5)
    xw = orc.widen(k)
    cents0 = np.stack([np.stack([xw[b, h, seeds[b, h]] for h in range(H)]) for b in range(B)])
    G = _metric(H, D, 8)
    cents, labels, sizes = _gpu_kmeans(k, cents0, 1, G)
    assert sizes.sum() == B * H * N
    for h in range(H):
        gc.log(f"wan720 k-means: means of head {h} on the GPU labels")
        _check_update(k[:, h:h + 1], labels[0, h], cents0[0, h], cents[0, h], sizes[0, h])
    rng = np.random.default_rng(14)
    tolerated = 0
    for h in range(H):
        toks = np.sort(rng.choice(N, 3000, replace=False))
        for part in np.array_split(toks, 12):
            d = orc.quad_distances(xw[0, h, part], cents0[0, h], G[0, h])
            lab_o = np.argmin(d, axis=1)
            diff = np.nonzero(labels[0, h, part] != lab_o)[0]
            tol = _assign_tolerance(xw[0, h, part], cents0[0, h], G[0, h])
            gap = d[diff, labels[0, h, part][diff]] - d[diff, lab_o[diff]]
            assert np.all(gap <= tol[diff])
            tolerated += diff.size
    gc.log(f"wan720 k-means sample: {tolerated} near-tie labels of {2 * 3000}")
    assert tolerated <= 6


@pytest.mark.parametrize("align", [64, 32])
def test_cluster_mask_and_attention_full_size_sampled(align):
    """Wan-720p shape with 400 query / 1000 key clusters (seeded labels, ten
    empty key clusters), align 64 or 32 (32: 32-token schedule entries streamed
    two per 64-key tile): GPU means and cluster mask against the oracle's over
    all rows, attention with the oracle's mask on 12 sampled query clusters per
    head, and tail merging of the oracle's mask."""
    m = _m()
    q, k, v = _wan720_heads()
    B, H, N, D = q.shape
    nq, nk = 400, 1000
    qlab = cluster_labels(N, nq, B, H, seed=31, stream=1)
    klab = cluster_labels(N, nk, B, H, seed=31, stream=2, empty=10)
    f64 = dict(dtype=torch.float64, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    qd, kd, vd = (gc.bits_to_dev(a) for a in (q, k, v))
    qbar, kbar = torch.zeros((B, H, nq, D), **f64), torch.zeros((B, H, nk, D), **f64)
    qs, ks = torch.empty((B, H, nq), **i32), torch.empty((B, H, nk), **i32)
    ws = torch.empty(m.svsa_cluster_means_workspace_bytes(B, H, N, nk), dtype=torch.uint8,
                     device="cuda")
    gc.log("wan720 clusters: GPU means")
    m.svsa_cluster_means(qd, _dev(qlab, torch.int32), qbar, qs, ws)
    m.svsa_cluster_means(kd, _dev(klab, torch.int32), kbar, ks, ws)
    torch.cuda.synchronize()
    gc.log("wan720 clusters: oracle means and scores")
    qbar_o, qs_o = orc.cluster_means(q, qlab, nq)
    kbar_o, ks_o = orc.cluster_means(k, klab, nk)
    assert np.array_equal(qs.cpu().numpy(), qs_o) and np.array_equal(ks.cpu().numpy(), ks_o)
    np.testing.assert_allclose(qbar.cpu().numpy(), qbar_o, rtol=1e-13, atol=1e-15)
    ne = ks_o > 0
    np.testing.assert_allclose(kbar.cpu().numpy()[ne], kbar_o[ne], rtol=1e-13, atol=1e-15)
    S = np.stack([np.stack([orc.cluster_scores(qbar_o[0, h], kbar_o[0, h], ks_o[0, h],
                                               1 / np.sqrt(D)) for h in range(H)])])
    tp = np.full(H, 0.9, np.float32)
    o_rp, o_ci = orc.cluster_mask(S, top_p=tp)
    # GPU mask over every row
    rows = B * H * nq
    rp = torch.empty(rows + 1, **i32)
    ci = torch.empty(rows * nk, **i32)
    mws = torch.empty(m.svsa_cluster_mask_workspace_bytes(B, H, nq, nk), dtype=torch.uint8,
                      device="cuda")
    m.svsa_cluster_mask(qbar, kbar, ks, 1 / np.sqrt(D), rp, ci, mws, top_p=tp)
    torch.cuda.synchronize()
    g_rp = rp.cpu().numpy().astype(np.int64)
    g_ci = ci[: int(g_rp[-1])].cpu().numpy()
    bad = _cluster_mask_failures(S, g_rp, g_ci, o_rp, o_ci, tp)
    assert not bad, bad[:5]
    # attention with the oracle's mask
    lws = torch.empty(m.svsa_cluster_layout_workspace_bytes(B, H, N, nk), dtype=torch.uint8,
                      device="cuda")
    lay = {}
    for tag, lab, C in (("q", qlab, nq), ("k", klab, nk)):
        cap = m.svsa_cluster_capacity(N, C, align)
        t = dict(start=torch.empty((B, H, C + 1), **i32), sizes=torch.empty((B, H, C), **i32),
                 slot=torch.empty((B, H, N), **i32), token=torch.empty((B, H, cap), **i32),
                 cap=cap)
        m.svsa_cluster_layout(_dev(lab, torch.int32), C, align, t["start"], t["sizes"],
                              t["slot"], t["token"], lws)
        lay[tag] = t
    bf = dict(dtype=torch.bfloat16, device="cuda")
    qp = torch.empty((B, H, lay["q"]["cap"], D), **bf)
    kp = torch.empty((B, H, lay["k"]["cap"], D), **bf)
    vp = torch.empty_like(kp)
    op = torch.empty_like(qp)
    m.svsa_cluster_permute(qd, qp, N, nq, align, lay["q"]["token"], lay["q"]["start"])
    m.svsa_cluster_permute(kd, kp, N, nk, align, lay["k"]["token"], lay["k"]["start"])
    m.svsa_cluster_permute(vd, vp, N, nk, align, lay["k"]["token"], lay["k"]["start"])
    aws = torch.empty(m.svsa_cluster_attn_workspace_bytes(B, H, N, nq, N, nk, align),
                      dtype=torch.uint8, device="cuda")
    gc.log(f"wan720 clusters: attention on {int(o_rp[-1])} kept pairs")
    m.svsa_cluster_attn(qp, kp, vp, op, N, lay["q"]["start"], lay["q"]["sizes"], N,
                        lay["k"]["start"], lay["k"]["sizes"], align, 1 / np.sqrt(D),
                        _dev(o_rp.astype(np.int32), torch.int32),
                        _dev(o_ci.astype(np.int32), torch.int32), aws)
    out = torch.empty_like(qd)
    m.svsa_cluster_permute(op, out, N, nq, align, lay["q"]["slot"], lay["q"]["start"],
                           inverse=True)
    torch.cuda.synchronize()
    out_bits = gc.dev_to_bits(out)
    rng = np.random.default_rng(15)
    g_all, r_all = [], []
    for h in range(H):
        counts = np.diff(o_rp)[h * nq:(h + 1) * nq]
        pick = {int(np.argmax(counts)), int(np.argmin(counts))}
        pick |= set(rng.choice(nq, 10, replace=False).tolist())
        for i in sorted(pick):
            r = h * nq + i
            toks, ref = orc.cluster_attention_rows(q[0, h], k[0, h], v[0, h], qlab[0, h],
                                                   klab[0, h], i, o_ci[o_rp[r]: o_rp[r + 1]],
                                                   1 / np.sqrt(D))
            g_all.append(orc.widen(out_bits[0, h, toks]).ravel())
            r_all.append(ref.ravel())
    g, r = np.concatenate(g_all), np.concatenate(r_all)
    max_abs = float(np.abs(g - r).max())
    rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
    gc.log(f"wan720 clusters: attention max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2
    # tail merging of the oracle's mask, bit-exact
    lab_d = _dev(qlab, torch.int32)
    rp2 = torch.empty(rows + 1, **i32)
    ci2 = torch.empty(rows * nk, **i32)
    tws = torch.empty(m.svsa_tail_merge_workspace_bytes(B, H, N, nq, nk), dtype=torch.uint8,
                      device="cuda")
    m.svsa_tail_merge(lab_d, nq, nk, align, _dev(o_rp.astype(np.int32), torch.int32),
                      _dev(o_ci.astype(np.int32), torch.int32), rp2, ci2, tws)
    torch.cuda.synchronize()
    t_lab = lab_d.cpu().numpy()
    t_rp = rp2.cpu().numpy().astype(np.int64)
    t_ci = ci2[: int(t_rp[-1])].cpu().numpy()
    for h in range(H):
        K = np.zeros((nq, nk), bool)
        for i in range(nq):
            K[i, o_ci[o_rp[h * nq + i]: o_rp[h * nq + i + 1]]] = True
        lab_o, R_o, _ = orc.tail_merge(qlab[0, h], K, align)
        assert np.array_equal(t_lab[0, h], lab_o)
        for i in range(nq):
            r = h * nq + i
            assert np.array_equal(t_ci[t_rp[r]: t_rp[r + 1]], np.nonzero(R_o[i])[0])


def test_cluster_attention_at_the_key_sub_block_limit():
    """4096 key clusters over 262,144 tokens (align 64: 8,128 key sub-blocks,
    near the 8,192 the schedule entries can index) and 512 query clusters:
    the mask over every row and attention on sampled query clusters."""
    c = _ClusterCase("maxnb", 512, 4096, 64, k_empty=0, seed=19)
    assert c.cap_k // 64 > 8000
    tp = np.full(c.H, 0.9, np.float32)
    g_rp, g_ci = c.gpu_mask(tp)
    o_rp, o_ci = orc.cluster_mask(c.S, top_p=tp)
    assert not _cluster_mask_failures(c.S, g_rp, g_ci, o_rp, o_ci, tp)
    out = c.gpu_attention(o_rp, o_ci)
    rng = np.random.default_rng(20)
    counts = np.diff(o_rp)
    pick = {int(np.argmax(counts)), int(np.argmin(counts))} | set(rng.choice(512, 6, replace=False).tolist())
    g_all, r_all = [], []
    for i in sorted(pick):
        toks, ref = orc.cluster_attention_rows(c.inp.q[0, 0], c.inp.k[0, 0], c.inp.v[0, 0],
                                               c.qlab[0, 0], c.klab[0, 0], i,
                                               o_ci[o_rp[i]: o_rp[i + 1]], 1 / np.sqrt(c.D))
        g_all.append(orc.widen(out[0, 0, toks]).ravel())
        r_all.append(ref.ravel())
    g, r = np.concatenate(g_all), np.concatenate(r_all)
    max_abs = float(np.abs(g - r).max())
    rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
    gc.log(f"maxnb clusters: attention max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= gc.MAX_ABS and rel <= gc.REL_L2
