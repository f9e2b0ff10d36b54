"""ctypes binding of libsvsa.so: argument marshalling only.

Every function here has the name of the C entry point it wraps and does no
arithmetic of the method: it checks tensor properties, turns torch tensors
into device pointers and the current torch stream into a hipStream_t, calls
the library, and raises ``SvsaError`` on a non-zero status.  torch provides
device memory and streams; all computation runs in the HIP kernels.

The library must be built (``python block_sparse_attention_17_amd/_build.py``);
importing this module without it raises immediately: there is no fallback.
"""
import ctypes
import os
from dataclasses import dataclass

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsvsa.so")

SVSA_BF16, SVSA_F32 = 0, 1
SVSA_OK = 0


class SvsaError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")


class _Geom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "H", "W", "tt", "th", "tw", "pad3d")]


@dataclass(frozen=True)
class Geometry:
    """Latent grid (T, H, W), tile shape (tt, th, tw) and block layout (pad3d:
    one block per tile with padding inside the sequence, else tail padding)."""
    T: int
    H: int
    W: int
    tt: int
    th: int
    tw: int
    pad3d: bool = False

    @property
    def N(self):
        return self.T * self.H * self.W

    @property
    def Bk(self):
        return self.tt * self.th * self.tw

    @property
    def tile_grid(self):
        return (-(-self.T // self.tt), -(-self.H // self.th), -(-self.W // self.tw))

    @property
    def nb(self):
        if self.pad3d:
            nT, nH, nW = self.tile_grid
            return nT * nH * nW
        return -(-self.N // self.Bk)

    @property
    def N_pad(self):
        return self.nb * self.Bk

    def valid_counts(self):
        """int64 [nb]: valid tokens of each block (its first slots)."""
        if not self.pad3d:
            n = np.full(self.nb, self.Bk, np.int64)
            n[-1] = self.N - (self.nb - 1) * self.Bk
            return n
        nT, nH, nW = self.tile_grid
        ext = lambda L, t, n: np.minimum(t, L - np.arange(n) * t)
        return (ext(self.T, self.tt, nT)[:, None, None] * ext(self.H, self.th, nH)[None, :, None]
                * ext(self.W, self.tw, nW)[None, None, :]).astype(np.int64).ravel()

    def c(self):
        return _Geom(self.T, self.H, self.W, self.tt, self.th, self.tw, int(bool(self.pad3d)))

    @staticmethod
    def from_config(cfg):
        return Geometry(*cfg.grid, *cfg.tile, pad3d=getattr(cfg, "pad3d", False))


def _load():
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python block_sparse_attention_17_amd/_build.py` "
            "(the block-sparse attention path has no non-HIP fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, sz, dbl, flt = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_size_t, ctypes.c_double, ctypes.c_float)
    gp = ctypes.POINTER(_Geom)
    fp = ctypes.POINTER(ctypes.c_float)
    sig = {
        "svsa_tile_permute": (ctypes.c_int, [vp, vp, i32, i32, i32, i32, gp, i32, vp]),
        "svsa_pool": (ctypes.c_int, [vp, i32, vp, i32, i32, i32, gp, vp]),
        "svsa_tile_permute_pool": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, i32, gp, vp]),
        "svsa_block_mask_workspace_bytes": (sz, [i32, i32, i32]),
        "svsa_block_mask": (ctypes.c_int, [vp, vp, i32, i32, i32, i32, dbl, fp, fp, i32, vp, vp,
                                           i64, vp, sz, vp]),
        "svsa_block_mask_noalloc": (ctypes.c_int, [vp, vp, i32, i32, i32, i32, dbl, fp, fp, i32,
                                                   vp, vp, i64, vp]),
        "svsa_stripe_mask_workspace_bytes": (sz, [i32, i32, gp]),
        "svsa_stripe_mask": (ctypes.c_int, [gp, i32, i32, ctypes.POINTER(ctypes.c_int32), i32, vp,
                                            vp, i64, vp, sz, vp]),
        "svsa_attn_workspace_bytes": (sz, [i32, i32, gp]),
        "svsa_block_sparse_attn": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, gp, flt, vp, vp,
                                                  vp, sz, vp]),
        "svsa_attn_stage_v": (ctypes.c_int, [vp, i32, i32, i32, gp, vp, sz, vp]),
        "svsa_block_sparse_attn_ex": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, gp, flt, vp,
                                                     vp, i32, vp, sz, vp]),
        "svsa_snr_top_p": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), i32, i32, flt, flt,
                                          fp]),
        "svsa_kmeans_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "svsa_kmeans": (ctypes.c_int, [vp, i32, i32, i32, i32, vp, vp, i32, i32, vp, vp, vp, sz,
                                       vp]),
        "svsa_cluster_metric": (ctypes.c_int, [vp, vp, i32, i32, i32, i32, vp, vp]),
        "svsa_cluster_means_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "svsa_cluster_means": (ctypes.c_int, [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, sz,
                                              vp]),
        "svsa_cluster_capacity": (i64, [i32, i32, i32]),
        "svsa_cluster_layout_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "svsa_cluster_layout": (ctypes.c_int, [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                               sz, vp]),
        "svsa_cluster_permute": (ctypes.c_int, [vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp,
                                                i32, vp]),
        "svsa_cluster_mask_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "svsa_cluster_mask": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, i32, i32, dbl, fp, fp, vp,
                                             vp, i64, vp, sz, vp]),
        "svsa_tail_merge_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "svsa_tail_merge": (ctypes.c_int, [vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp,
                                           i64, vp, sz, vp]),
        "svsa_cluster_attn_workspace_bytes": (sz, [i32, i32, i32, i32, i32, i32, i32]),
        "svsa_cluster_attn": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, i32,
                                             i32, vp, vp, i32, flt, vp, vp, vp, sz, vp]),
        "svsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "svsa_version": (ctypes.c_int, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()

EXPORTED = ("svsa_tile_permute", "svsa_pool", "svsa_tile_permute_pool",
            "svsa_block_mask_workspace_bytes", "svsa_block_mask", "svsa_block_mask_noalloc",
            "svsa_stripe_mask_workspace_bytes", "svsa_stripe_mask",
            "svsa_attn_workspace_bytes", "svsa_block_sparse_attn", "svsa_block_sparse_attn_ex",
            "svsa_attn_stage_v",
            "svsa_snr_top_p",
            "svsa_kmeans_workspace_bytes", "svsa_kmeans", "svsa_cluster_metric",
            "svsa_cluster_means_workspace_bytes", "svsa_cluster_means",
            "svsa_cluster_capacity", "svsa_cluster_layout_workspace_bytes",
            "svsa_cluster_layout", "svsa_cluster_permute",
            "svsa_cluster_mask_workspace_bytes", "svsa_cluster_mask",
            "svsa_cluster_attn_workspace_bytes", "svsa_cluster_attn",
            "svsa_tail_merge_workspace_bytes", "svsa_tail_merge",
            "svsa_status_string", "svsa_version")


def library_path():
    return _LIB_PATH


def library():
    return _lib


def status_string(status):
    return _lib.svsa_status_string(int(status)).decode()


svsa_status_string = status_string


def svsa_version():
    return _lib.svsa_version()


def _check(fn, status):
    if status != SVSA_OK:
        raise SvsaError(fn, status)


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t, name, dtypes=None, device=True):
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return ctypes.c_void_p(t.data_ptr())


def _tensor(t, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")


def _shape(t, name, shape):
    """Refuse a tensor whose shape is not exactly `shape` (the C ABI sees no sizes)."""
    if t is None:
        return
    _tensor(t, name)
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _at_least(t, name, n):
    """Refuse a 1-D index array with fewer than n entries."""
    if t is None:
        return
    _tensor(t, name)
    if t.dim() != 1 or t.numel() < int(n):
        raise ValueError(f"{name} must be 1-D with at least {int(n)} entries, "
                         f"got shape {tuple(t.shape)}")


def _ndim(t, name, n):
    _tensor(t, name)
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {tuple(t.shape)}")


def _same_device(**tensors):
    """Every given device tensor must live on one device."""
    devs = {n: t.device for n, t in tensors.items() if t is not None and hasattr(t, "device")}
    if len(set(devs.values())) > 1:
        raise ValueError(f"tensors on different devices: {devs}")


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return SVSA_BF16
    if t.dtype == torch.float32:
        return SVSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def svsa_tile_permute(src, dst, geom, inverse=False, stream=None):
    """dst <- tile-ordered src (inverse=False) or natural-ordered src (inverse=True)."""
    import torch
    _ndim(src, "src", 4)
    B, Hh, _, D = src.shape
    n_src, n_dst = (geom.N_pad, geom.N) if inverse else (geom.N, geom.N_pad)
    _shape(src, "src", (B, Hh, n_src, D))
    _shape(dst, "dst", (B, Hh, n_dst, D))
    _same_device(src=src, dst=dst)
    _check("svsa_tile_permute", _lib.svsa_tile_permute(
        _ptr(src, "src", (torch.bfloat16, torch.float32)), _ptr(dst, "dst", (src.dtype,)),
        _dtype_code(src), B, Hh, D, ctypes.byref(geom.c()), int(bool(inverse)), _stream(stream)))
    return dst


def svsa_pool(x_tiled, out, geom, stream=None):
    """out (float64 [B, Hh, nb, D]) <- per-block means of the valid rows of x_tiled."""
    import torch
    _ndim(x_tiled, "x_tiled", 4)
    B, Hh, _, D = x_tiled.shape
    _shape(x_tiled, "x_tiled", (B, Hh, geom.N_pad, D))
    _shape(out, "out", (B, Hh, geom.nb, D))
    _same_device(x_tiled=x_tiled, out=out)
    _check("svsa_pool", _lib.svsa_pool(
        _ptr(x_tiled, "x_tiled", (torch.bfloat16, torch.float32)), _dtype_code(x_tiled),
        _ptr(out, "out", (torch.float64,)), B, Hh, D, ctypes.byref(geom.c()), _stream(stream)))
    return out


def svsa_tile_permute_pool(src, dst, means, geom, stream=None):
    """dst <- tile-ordered src and means (float64 [B, Hh, nb, D]) <- its block means, one pass."""
    import torch
    _ndim(src, "src", 4)
    B, Hh, _, D = src.shape
    _shape(src, "src", (B, Hh, geom.N, D))
    _shape(dst, "dst", (B, Hh, geom.N_pad, D))
    _shape(means, "means", (B, Hh, geom.nb, D))
    _same_device(src=src, dst=dst, means=means)
    _check("svsa_tile_permute_pool", _lib.svsa_tile_permute_pool(
        _ptr(src, "src", (torch.bfloat16, torch.float32)), _ptr(dst, "dst", (src.dtype,)),
        _ptr(means, "means", (torch.float64,)), _dtype_code(src), B, Hh, D,
        ctypes.byref(geom.c()), _stream(stream)))
    return dst


def svsa_snr_top_p(sigmas, first_sparse, p_min, tau):
    """float32 [steps] per-step top-p from the noise levels (host call, no GPU)."""
    sig = np.ascontiguousarray(np.asarray(sigmas, dtype=np.float64).ravel())
    out = np.empty(sig.size, np.float32)
    _check("svsa_snr_top_p", _lib.svsa_snr_top_p(
        sig.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), sig.size, int(first_sparse),
        float(p_min), float(tau), out.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
    return out


def svsa_block_mask_workspace_bytes(batch, heads, nb):
    return int(_lib.svsa_block_mask_workspace_bytes(batch, heads, nb))


def _host_f32(a, heads, name):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.broadcast_to(np.asarray(a, dtype=np.float32), (heads,)))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def svsa_block_mask(qbar, kbar, softmax_scale, row_ptr, col_idx, workspace, top_p=None,
                    keep_frac=None, band_width=1, stream=None):
    """CSR (row_ptr, col_idx) of kept key blocks from float64 block summaries."""
    import torch
    _ndim(qbar, "qbar", 4)
    B, Hh, nb, D = qbar.shape
    _shape(kbar, "kbar", (B, Hh, nb, D))
    _at_least(row_ptr, "row_ptr", B * Hh * nb + 1)
    _ndim(col_idx, "col_idx", 1)
    _same_device(qbar=qbar, kbar=kbar, row_ptr=row_ptr, col_idx=col_idx, workspace=workspace)
    tp_arr, tp = _host_f32(top_p, Hh, "top_p")
    kf_arr, kf = _host_f32(keep_frac, Hh, "keep_frac")
    _check("svsa_block_mask", _lib.svsa_block_mask(
        _ptr(qbar, "qbar", (torch.float64,)), _ptr(kbar, "kbar", (torch.float64,)), B, Hh, nb, D,
        float(softmax_scale), tp, kf, int(band_width), _ptr(row_ptr, "row_ptr", (torch.int32,)),
        _ptr(col_idx, "col_idx", (torch.int32,)), col_idx.numel(),
        _ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream(stream)))
    del tp_arr, kf_arr
    return row_ptr, col_idx


def svsa_block_mask_noalloc(qbar, kbar, softmax_scale, row_ptr, col_idx, top_p=None,
                            keep_frac=None, band_width=1, stream=None):
    """svsa_block_mask with the library's own device scratch (no workspace, no
    allocation); calls overlapping in time on one device race."""
    import torch
    _ndim(qbar, "qbar", 4)
    B, Hh, nb, D = qbar.shape
    _shape(kbar, "kbar", (B, Hh, nb, D))
    _at_least(row_ptr, "row_ptr", B * Hh * nb + 1)
    _ndim(col_idx, "col_idx", 1)
    _same_device(qbar=qbar, kbar=kbar, row_ptr=row_ptr, col_idx=col_idx)
    tp_arr, tp = _host_f32(top_p, Hh, "top_p")
    kf_arr, kf = _host_f32(keep_frac, Hh, "keep_frac")
    _check("svsa_block_mask_noalloc", _lib.svsa_block_mask_noalloc(
        _ptr(qbar, "qbar", (torch.float64,)), _ptr(kbar, "kbar", (torch.float64,)), B, Hh, nb, D,
        float(softmax_scale), tp, kf, int(band_width), _ptr(row_ptr, "row_ptr", (torch.int32,)),
        _ptr(col_idx, "col_idx", (torch.int32,)), col_idx.numel(), _stream(stream)))
    del tp_arr, kf_arr
    return row_ptr, col_idx


def svsa_stripe_mask_workspace_bytes(batch, heads, geom):
    return int(_lib.svsa_stripe_mask_workspace_bytes(batch, heads, ctypes.byref(geom.c())))


def svsa_stripe_mask(geom, batch, params, row_ptr, col_idx, workspace, band_width=0,
                     stream=None):
    """CSR of the PSA stripe mask; params: [heads, 6] ints (Tw, To, Ts, Sw, So, Ss)."""
    import torch
    arr = np.ascontiguousarray(np.asarray(params, dtype=np.int32).reshape(-1, 6))
    heads = arr.shape[0]
    _at_least(row_ptr, "row_ptr", int(batch) * heads * geom.nb + 1)
    _ndim(col_idx, "col_idx", 1)
    _same_device(row_ptr=row_ptr, col_idx=col_idx, workspace=workspace)
    _check("svsa_stripe_mask", _lib.svsa_stripe_mask(
        ctypes.byref(geom.c()), int(batch), int(heads),
        arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(band_width),
        _ptr(row_ptr, "row_ptr", (torch.int32,)), _ptr(col_idx, "col_idx", (torch.int32,)),
        col_idx.numel(), _ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(),
        _stream(stream)))
    del arr
    return row_ptr, col_idx


def svsa_attn_workspace_bytes(batch, heads, geom):
    return int(_lib.svsa_attn_workspace_bytes(batch, heads, ctypes.byref(geom.c())))


def svsa_block_sparse_attn(q, k, v, out, geom, softmax_scale, row_ptr, col_idx, workspace,
                           stream=None):
    """out (bf16, tile order) <- block-sparse attention of q, k, v over the CSR lists.
    v=None: V as staged into `workspace` by svsa_attn_stage_v."""
    import torch
    _attn_shapes(q, k, v, out, geom, row_ptr, col_idx, workspace, natural=False)
    B, Hh, _, D = q.shape
    bf = (torch.bfloat16,)
    _check("svsa_block_sparse_attn", _lib.svsa_block_sparse_attn(
        _ptr(q, "q", bf), _ptr(k, "k", bf), _ptr(v, "v", bf), _ptr(out, "out", bf), B, Hh, D,
        ctypes.byref(geom.c()), float(softmax_scale), _ptr(row_ptr, "row_ptr", (torch.int32,)),
        _ptr(col_idx, "col_idx", (torch.int32,)), _ptr(workspace, "workspace", (torch.uint8,)),
        workspace.numel(), _stream(stream)))
    return out


SVSA_ATTN_OUT_NATURAL = 1
SVSA_ATTN_POSITIONAL_GROUPS = 2
SVSA_ATTN_GROUPS_BY_LIST = 4
SVSA_ATTN_STEP_PAIRS = 8


def _attn_shapes(q, k, v, out, geom, row_ptr, col_idx, workspace, natural):
    """q, k, v (if given) tiled [B, Hh, N_pad, D]; out tiled, or natural
    [B, Hh, N, D] with SVSA_ATTN_OUT_NATURAL; row_ptr >= B*Hh*nb + 1 entries."""
    _ndim(q, "q", 4)
    B, Hh, _, D = q.shape
    _shape(q, "q", (B, Hh, geom.N_pad, D))
    _shape(k, "k", (B, Hh, geom.N_pad, D))
    _shape(v, "v", (B, Hh, geom.N_pad, D))
    _shape(out, "out", (B, Hh, geom.N if natural else geom.N_pad, D))
    _at_least(row_ptr, "row_ptr", B * Hh * geom.nb + 1)
    _ndim(col_idx, "col_idx", 1)
    _same_device(q=q, k=k, v=v, out=out, row_ptr=row_ptr, col_idx=col_idx, workspace=workspace)


def svsa_block_sparse_attn_ex(q, k, v, out, geom, softmax_scale, row_ptr, col_idx, workspace,
                              flags=0, stream=None):
    """svsa_block_sparse_attn with flags; SVSA_ATTN_OUT_NATURAL: out is bf16
    [B, Hh, N, D] in natural order (the inverse reorder done by the kernel);
    SVSA_ATTN_POSITIONAL_GROUPS: query blocks grouped by position only;
    SVSA_ATTN_GROUPS_BY_LIST: grouped by their lists whatever the size;
    SVSA_ATTN_STEP_PAIRS: the union list walked in steps of one or two key
    blocks with disjoint keepers (64-token blocks)."""
    import torch
    _attn_shapes(q, k, v, out, geom, row_ptr, col_idx, workspace,
                 natural=bool(int(flags) & SVSA_ATTN_OUT_NATURAL))
    B, Hh, _, D = q.shape
    bf = (torch.bfloat16,)
    _check("svsa_block_sparse_attn_ex", _lib.svsa_block_sparse_attn_ex(
        _ptr(q, "q", bf), _ptr(k, "k", bf), _ptr(v, "v", bf), _ptr(out, "out", bf), B, Hh, D,
        ctypes.byref(geom.c()), float(softmax_scale), _ptr(row_ptr, "row_ptr", (torch.int32,)),
        _ptr(col_idx, "col_idx", (torch.int32,)), int(flags),
        _ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream(stream)))
    return out


def svsa_attn_stage_v(v, workspace, geom, stream=None):
    """Natural-order V (bf16 [B, Hh, N, D]) -> the attention workspace's V^T, tile order."""
    import torch
    _ndim(v, "v", 4)
    B, Hh, _, D = v.shape
    _shape(v, "v", (B, Hh, geom.N, D))
    _same_device(v=v, workspace=workspace)
    _check("svsa_attn_stage_v", _lib.svsa_attn_stage_v(
        _ptr(v, "v", (torch.bfloat16,)), B, Hh, D, ctypes.byref(geom.c()),
        _ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream(stream)))
    return workspace


# ---------------------------------------------------------------------------
# Variable-size blocks (clusters)
# ---------------------------------------------------------------------------
def svsa_kmeans_workspace_bytes(batch, heads, n, clusters, head_dim):
    return int(_lib.svsa_kmeans_workspace_bytes(batch, heads, n, clusters, head_dim))


def svsa_kmeans(x, centroids, labels, sizes, workspace, iters, metric=None, stream=None):
    """Lloyd iterations under the quadratic form `metric` (None: identity);
    centroids float64 [B, Hh, C, D] are updated in place."""
    import torch
    _ndim(x, "x", 4)
    B_, Hh, N, D = x.shape
    _ndim(centroids, "centroids", 4)
    C = centroids.shape[2]
    _shape(centroids, "centroids", (B_, Hh, C, D))
    _shape(metric, "metric", (B_, Hh, D, D))
    _shape(labels, "labels", (B_, Hh, N))
    _shape(sizes, "sizes", (B_, Hh, C))
    _same_device(x=x, metric=metric, centroids=centroids, labels=labels, sizes=sizes,
                 workspace=workspace)
    _check("svsa_kmeans", _lib.svsa_kmeans(
        _ptr(x, "x", (torch.bfloat16,)), B_, Hh, N, D,
        _ptr(metric, "metric", (torch.float64,)), _ptr(centroids, "centroids", (torch.float64,)),
        C, int(iters), _ptr(labels, "labels", (torch.int32,)),
        _ptr(sizes, "sizes", (torch.int32,)), _ptr(workspace, "workspace", (torch.uint8,)),
        workspace.numel(), _stream(stream)))
    return centroids, labels, sizes


def svsa_cluster_means_workspace_bytes(batch, heads, n, clusters):
    return int(_lib.svsa_cluster_means_workspace_bytes(batch, heads, n, clusters))


def svsa_cluster_means(x, labels, centroids, sizes, workspace, stream=None):
    """centroids (float64 [B, Hh, C, D]) <- means of the tokens of each label."""
    import torch
    _ndim(x, "x", 4)
    B_, Hh, N, D = x.shape
    _ndim(centroids, "centroids", 4)
    C = centroids.shape[2]
    _shape(labels, "labels", (B_, Hh, N))
    _shape(centroids, "centroids", (B_, Hh, C, D))
    _shape(sizes, "sizes", (B_, Hh, C))
    _same_device(x=x, labels=labels, centroids=centroids, sizes=sizes, workspace=workspace)
    _check("svsa_cluster_means", _lib.svsa_cluster_means(
        _ptr(x, "x", (torch.bfloat16,)), _ptr(labels, "labels", (torch.int32,)), B_, Hh, N, D, C,
        _ptr(centroids, "centroids", (torch.float64,)), _ptr(sizes, "sizes", (torch.int32,)),
        _ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream(stream)))
    return centroids, sizes


def svsa_cluster_metric(centroids, sizes, metric, stream=None):
    import torch
    _ndim(centroids, "centroids", 4)
    B_, Hh, C, D = centroids.shape
    _shape(sizes, "sizes", (B_, Hh, C))
    _shape(metric, "metric", (B_, Hh, D, D))
    _same_device(centroids=centroids, sizes=sizes, metric=metric)
    _check("svsa_cluster_metric", _lib.svsa_cluster_metric(
        _ptr(centroids, "centroids", (torch.float64,)), _ptr(sizes, "sizes", (torch.int32,)),
        B_, Hh, C, D, _ptr(metric, "metric", (torch.float64,)), _stream(stream)))
    return metric


def svsa_cluster_capacity(n, clusters, align):
    return int(_lib.svsa_cluster_capacity(n, clusters, align))


def svsa_cluster_layout_workspace_bytes(batch, heads, n, clusters):
    return int(_lib.svsa_cluster_layout_workspace_bytes(batch, heads, n, clusters))


def svsa_cluster_layout(labels, clusters, align, start, sizes, slot, token, workspace,
                        stream=None):
    import torch
    _ndim(labels, "labels", 3)
    B_, Hh, N = labels.shape
    _shape(start, "start", (B_, Hh, int(clusters) + 1))
    _shape(sizes, "sizes", (B_, Hh, int(clusters)))
    _shape(slot, "slot", (B_, Hh, N))
    _shape(token, "token", (B_, Hh, svsa_cluster_capacity(N, clusters, align)))
    _same_device(labels=labels, start=start, sizes=sizes, slot=slot, token=token,
                 workspace=workspace)
    i32 = (torch.int32,)
    _check("svsa_cluster_layout", _lib.svsa_cluster_layout(
        _ptr(labels, "labels", i32), B_, Hh, N, int(clusters), int(align),
        _ptr(start, "start", i32), _ptr(sizes, "sizes", i32), _ptr(slot, "slot", i32),
        _ptr(token, "token", i32), _ptr(workspace, "workspace", (torch.uint8,)),
        workspace.numel(), _stream(stream)))
    return start, sizes, slot, token


def svsa_cluster_permute(src, dst, n, clusters, align, map_, start, inverse=False, stream=None):
    import torch
    _ndim(src, "src", 4)
    B_, Hh, _, D = src.shape
    cap = svsa_cluster_capacity(n, clusters, align)
    n_src, n_dst = (cap, n) if inverse else (n, cap)
    _shape(src, "src", (B_, Hh, n_src, D))
    _shape(dst, "dst", (B_, Hh, n_dst, D))
    _shape(map_, "map", (B_, Hh, n if inverse else cap))
    _shape(start, "start", (B_, Hh, int(clusters) + 1))
    _same_device(src=src, dst=dst, map=map_, start=start)
    _check("svsa_cluster_permute", _lib.svsa_cluster_permute(
        _ptr(src, "src", (torch.bfloat16, torch.float32)), _ptr(dst, "dst", (src.dtype,)),
        _dtype_code(src), B_, Hh, int(n), D, int(clusters), int(align),
        _ptr(map_, "map", (torch.int32,)), _ptr(start, "start", (torch.int32,)),
        int(bool(inverse)), _stream(stream)))
    return dst


def svsa_cluster_mask_workspace_bytes(batch, heads, nq, nk):
    return int(_lib.svsa_cluster_mask_workspace_bytes(batch, heads, nq, nk))


def svsa_cluster_mask(qbar, kbar, ksizes, softmax_scale, row_ptr, col_idx, workspace,
                      top_p=None, keep_frac=None, stream=None):
    import torch
    _ndim(qbar, "qbar", 4)
    B_, Hh, nq, D = qbar.shape
    _ndim(kbar, "kbar", 4)
    nk = kbar.shape[2]
    _shape(kbar, "kbar", (B_, Hh, nk, D))
    _shape(ksizes, "ksizes", (B_, Hh, nk))
    _at_least(row_ptr, "row_ptr", B_ * Hh * nq + 1)
    _ndim(col_idx, "col_idx", 1)
    _same_device(qbar=qbar, kbar=kbar, ksizes=ksizes, row_ptr=row_ptr, col_idx=col_idx,
                 workspace=workspace)
    tp_arr, tp = _host_f32(top_p, Hh, "top_p")
    kf_arr, kf = _host_f32(keep_frac, Hh, "keep_frac")
    _check("svsa_cluster_mask", _lib.svsa_cluster_mask(
        _ptr(qbar, "qbar", (torch.float64,)), _ptr(kbar, "kbar", (torch.float64,)),
        _ptr(ksizes, "ksizes", (torch.int32,)), B_, Hh, nq, nk, D, float(softmax_scale), tp, kf,
        _ptr(row_ptr, "row_ptr", (torch.int32,)), _ptr(col_idx, "col_idx", (torch.int32,)),
        col_idx.numel(), _ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(),
        _stream(stream)))
    del tp_arr, kf_arr
    return row_ptr, col_idx


def svsa_cluster_attn_workspace_bytes(batch, heads, n_q, nq, n_k, nk, align):
    return int(_lib.svsa_cluster_attn_workspace_bytes(batch, heads, n_q, nq, n_k, nk, align))


def svsa_cluster_attn(q, k, v, out, n_q, q_start, q_size, n_k, k_start, k_size, align,
                      softmax_scale, row_ptr, col_idx, workspace, stream=None):
    """out (bf16, query cluster layout) <- attention over the kept key clusters."""
    import torch
    _ndim(q, "q", 4)
    B_, Hh, _, D = q.shape
    bf, i32 = (torch.bfloat16,), (torch.int32,)
    nq, nk = q_size.shape[-1], k_size.shape[-1]
    cap_q = svsa_cluster_capacity(n_q, nq, align)
    cap_k = svsa_cluster_capacity(n_k, nk, align)
    _shape(q, "q", (B_, Hh, cap_q, D))
    _shape(k, "k", (B_, Hh, cap_k, D))
    _shape(v, "v", (B_, Hh, cap_k, D))
    _shape(out, "out", (B_, Hh, cap_q, D))
    _shape(q_start, "q_start", (B_, Hh, nq + 1))
    _shape(q_size, "q_size", (B_, Hh, nq))
    _shape(k_start, "k_start", (B_, Hh, nk + 1))
    _shape(k_size, "k_size", (B_, Hh, nk))
    _at_least(row_ptr, "row_ptr", B_ * Hh * nq + 1)
    _ndim(col_idx, "col_idx", 1)
    _same_device(q=q, k=k, v=v, out=out, q_start=q_start, q_size=q_size, k_start=k_start,
                 k_size=k_size, row_ptr=row_ptr, col_idx=col_idx, workspace=workspace)
    _check("svsa_cluster_attn", _lib.svsa_cluster_attn(
        _ptr(q, "q", bf), _ptr(k, "k", bf), _ptr(v, "v", bf), _ptr(out, "out", bf), B_, Hh, D,
        int(n_q), int(nq), _ptr(q_start, "q_start", i32), _ptr(q_size, "q_size", i32), int(n_k),
        int(nk), _ptr(k_start, "k_start", i32), _ptr(k_size, "k_size", i32), int(align),
        float(softmax_scale), _ptr(row_ptr, "row_ptr", i32), _ptr(col_idx, "col_idx", i32),
        _ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream(stream)))
    return out


def svsa_tail_merge_workspace_bytes(batch, heads, n, nq, nk):
    return int(_lib.svsa_tail_merge_workspace_bytes(batch, heads, n, nq, nk))


def svsa_tail_merge(labels, nq, nk, block, row_ptr, col_idx, row_ptr_out, col_idx_out,
                    workspace, rounds=2, stream=None):
    """Query labels (in place) and the cluster mask after tail merging."""
    import torch
    _ndim(labels, "labels", 3)
    B_, Hh, N = labels.shape
    _at_least(row_ptr, "row_ptr", B_ * Hh * int(nq) + 1)
    _at_least(row_ptr_out, "row_ptr_out", B_ * Hh * int(nq) + 1)
    _ndim(col_idx, "col_idx", 1)
    _ndim(col_idx_out, "col_idx_out", 1)
    _same_device(labels=labels, row_ptr=row_ptr, col_idx=col_idx, row_ptr_out=row_ptr_out,
                 col_idx_out=col_idx_out, workspace=workspace)
    i32 = (torch.int32,)
    _check("svsa_tail_merge", _lib.svsa_tail_merge(
        _ptr(labels, "labels", i32), B_, Hh, N, int(nq), int(nk), int(block), int(rounds),
        _ptr(row_ptr, "row_ptr", i32), _ptr(col_idx, "col_idx", i32),
        _ptr(row_ptr_out, "row_ptr_out", i32), _ptr(col_idx_out, "col_idx_out", i32),
        col_idx_out.numel(), _ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(),
        _stream(stream)))
    return labels, row_ptr_out, col_idx_out
