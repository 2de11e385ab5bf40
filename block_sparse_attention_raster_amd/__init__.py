"""Top-k block-sparse attention over a raster-ordered (T, H, W) latent grid,
for AMD Instinct MI355X (gfx950).

Every step runs in the HIP library libvsa.so (include/vsa.h); this module
only checks tensors and passes pointers, strides and the current stream.
PyTorch provides device memory and streams. Importing the package does not
load the library; the first call does, and raises if it is missing.

    import block_sparse_attention_raster_amd as vsa
    out = vsa.forward(q, k, v, latent_shape=(31, 22, 40), cube_shape=(4, 8, 8), topk=64)

q, k, v: bfloat16 or float16 CUDA (HIP) tensors [B, heads, N, head_dim] of
one dtype, with the last dimension contiguous and N = prefix_len + T*H*W
tokens in raster order. The output has their dtype. k and v may lie on a
grid of their own (``latent_shape_k``, ``cube_shape_k``), as in fastbsa's
``flash_attn_bsa_3d``, which this module also provides.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

from . import _lib
from ._lib import VsaError

__all__ = ["Plan", "Route", "VsaError", "plan", "plan_for", "select", "pool", "score_topk", "attend", "forward",
           "flash_attn_bsa_3d", "topk_for_sparsity", "route", "describe"]


class Plan:
    """A validated problem and its derived geometry (a copy of vsa_plan_t)."""

    def __init__(self, raw: _lib.VsaPlan):
        self.raw = raw

    def __getattr__(self, name):
        raw = self.__dict__["raw"]
        if hasattr(raw, name):
            v = getattr(raw, name)
            return tuple(v) if name in ("nblk", "nblk_k") else v
        if hasattr(raw.p, name):
            v = getattr(raw.p, name)
            return tuple(v) if name in ("latent", "cube", "latent_k", "cube_k") else v
        raise AttributeError(name)

    @property
    def kv_strides(self):
        return (self.kv_stride_b, self.kv_stride_h, self.kv_stride_n)

    def valid_counts(self, side: str = "q"):
        """Valid token count of every block (prefix blocks, then cubes) of
        q's grid (``side="q"``) or of k's (``"k"``), from vsa_block_counts;
        an int64 numpy array."""
        import numpy as np
        sides = {"q": _lib.VSA_SIDE_Q, "k": _lib.VSA_SIDE_K}
        if side not in sides:
            raise ValueError("side must be 'q' or 'k'")
        L = _lib.lib()
        n = L.vsa_block_counts(ctypes.byref(self.raw), sides[side], None, 0)
        if n < 0:
            raise VsaError(n, "vsa_block_counts")
        buf = (ctypes.c_int32 * n)()
        _lib.check(0 if L.vsa_block_counts(ctypes.byref(self.raw), sides[side], buf, n) == n else -1,
                   "vsa_block_counts")
        return np.frombuffer(buf, dtype=np.int32).astype(np.int64)

    def __repr__(self):
        return f"Plan({describe(self)})"


_DTYPES = {"bf16": _lib.VSA_DTYPE_BF16, "f16": _lib.VSA_DTYPE_F16}


def plan(batch: int, heads: int, head_dim: int, latent: Sequence[int], cube: Sequence[int], topk: int,
         prefix_len: int = 0, strides: Optional[Sequence[int]] = None,
         o_strides: Optional[Sequence[int]] = None, dtype: str = "bf16",
         latent_k: Optional[Sequence[int]] = None, cube_k: Optional[Sequence[int]] = None,
         kv_strides: Optional[Sequence[int]] = None) -> Plan:
    """Validate a problem and derive its geometry (vsa_plan). ``strides``
    are the (b, h, n) element strides of q (and of k and v unless
    ``kv_strides`` is given); the default is a contiguous
    [B, heads, N, head_dim] layout. ``o_strides`` default to ``strides``.
    ``dtype`` is "bf16" or "f16", the element type of q, k, v and o.
    ``latent_k`` and ``cube_k`` put k and v on a grid of their own (default:
    q's); ``kv_strides`` then default to a contiguous layout of that grid."""
    raw = _lib.VsaPlan()
    pr = _problem(batch, heads, head_dim, latent, cube, topk, prefix_len, strides, o_strides, dtype,
                  latent_k, cube_k, kv_strides)
    _lib.check(_lib.lib().vsa_plan(ctypes.byref(pr), ctypes.byref(raw)), "vsa_plan")
    return Plan(raw)


def _problem(batch, heads, head_dim, latent, cube, topk, prefix_len=0, strides=None, o_strides=None,
             dtype="bf16", latent_k=None, cube_k=None, kv_strides=None) -> _lib.VsaProblem:
    if dtype not in _DTYPES:
        raise ValueError(f"dtype must be one of {sorted(_DTYPES)}, got {dtype!r}")
    # zeros ask vsa_plan for its default layout (contiguous; o like q; k and
    # v like q on q's grid, else contiguous on their own grid)
    strides = (0, 0, 0) if strides is None else strides
    o_strides = (0, 0, 0) if o_strides is None else o_strides
    kv_strides = (0, 0, 0) if kv_strides is None else kv_strides
    latent_k = (0, 0, 0) if latent_k is None else tuple(latent_k)
    cube_k = (0, 0, 0) if cube_k is None else tuple(cube_k)
    pr = _lib.VsaProblem()
    pr.batch, pr.heads, pr.head_dim = int(batch), int(heads), int(head_dim)
    pr.latent[:] = [int(x) for x in latent]
    pr.cube[:] = [int(x) for x in cube]
    pr.topk, pr.prefix_len, pr.dtype = int(topk), int(prefix_len), _DTYPES[dtype]
    pr.stride_b, pr.stride_h, pr.stride_n = (int(s) for s in strides)
    pr.o_stride_b, pr.o_stride_h, pr.o_stride_n = (int(s) for s in o_strides)
    pr.latent_k[:] = [int(x) for x in latent_k]
    pr.cube_k[:] = [int(x) for x in cube_k]
    pr.kv_stride_b, pr.kv_stride_h, pr.kv_stride_n = (int(s) for s in kv_strides)
    return pr


def _torch_dtype(pl: Plan):
    import torch
    return torch.float16 if pl.dtype == _lib.VSA_DTYPE_F16 else torch.bfloat16


def _check_device(t, name, device):
    """Every buffer the kernels touch must live on q's GPU: a host pointer
    or another device's memory would reach the kernels unchecked."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must be on the GPU device of q ({device}), got {t.device}")


def _check_qkv(t, name, shape, strides, dtype, device=None):
    _check_device(t, name, device)
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (the plan's dtype), got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.stride(3) != 1 or tuple(t.stride()[:3]) != tuple(strides):
        raise ValueError(f"{name} strides {t.stride()} do not match the plan's {tuple(strides)} "
                         "(head_dim must be contiguous)")


def plan_for(q, latent: Sequence[int], cube: Sequence[int], topk: int, prefix_len: int = 0,
             out=None, k=None, latent_k: Optional[Sequence[int]] = None,
             cube_k: Optional[Sequence[int]] = None) -> Plan:
    """Plan from q's shape, strides and dtype (out's strides and k's, if
    given; k and v must share strides)."""
    import torch
    B, Hh, N, D = q.shape
    o_strides = out.stride()[:3] if out is not None else q.stride()[:3]
    kv_strides = k.stride()[:3] if k is not None else None
    names = {torch.bfloat16: "bf16", torch.float16: "f16"}
    if q.dtype not in names:
        raise TypeError(f"q must be bfloat16 or float16, got {q.dtype}")
    return plan(B, Hh, D, latent, cube, topk, prefix_len, q.stride()[:3], o_strides, names[q.dtype],
                latent_k, cube_k, kv_strides)


def _stream_ptr(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _qk_checked(pl: Plan, q, k):
    shape = (pl.batch, pl.heads, pl.seq_len, pl.head_dim)
    kshape = (pl.batch, pl.heads, pl.seq_len_k, pl.head_dim)
    dt = _torch_dtype(pl)
    _check_qkv(q, "q", shape, (pl.stride_b, pl.stride_h, pl.stride_n), dt)
    _check_qkv(k, "k", kshape, pl.kv_strides, dt, q.device)
    return q.device


def _workspace_checked(pl: Plan, workspace, dev):
    import torch
    if workspace is None:
        return torch.empty(pl.workspace_bytes, dtype=torch.uint8, device=dev)
    _check_device(workspace, "workspace", dev)
    if workspace.numel() * workspace.element_size() < pl.workspace_bytes or not workspace.is_contiguous():
        raise ValueError("workspace too small or not contiguous")
    return workspace


def _sel_checked(pl: Plan, sel, dev):
    import torch
    if sel is None:
        return torch.empty((pl.batch, pl.heads, pl.num_q_blocks, pl.topk), dtype=torch.int32, device=dev)
    _check_device(sel, "sel", dev)
    if sel.dtype != torch.int32 or sel.numel() != pl.sel_elems or not sel.is_contiguous():
        raise ValueError("sel must be a contiguous int32 tensor of plan.sel_elems elements")
    return sel


def select(pl: Plan, q, k, workspace=None, sel=None):
    """Pool, score and select (vsa_select). Returns (sel, workspace):
    sel int32 [B, heads, num_q_blocks, topk] ascending cube ids; workspace
    holds float32 qbar then kbar (see include/vsa.h)."""
    import torch
    dev = _qk_checked(pl, q, k)
    workspace = _workspace_checked(pl, workspace, dev)
    sel = _sel_checked(pl, sel, dev)
    with torch.cuda.device(dev):
        st = _lib.lib().vsa_select(ctypes.byref(pl.raw), q.data_ptr(), k.data_ptr(), workspace.data_ptr(),
                                   sel.data_ptr(), _stream_ptr(dev))
    _lib.check(st, "vsa_select")
    return sel, workspace


def pool(pl: Plan, q, k, workspace=None):
    """The pooling half of select (vsa_pool): qbar and kbar into the
    workspace, which is returned."""
    import torch
    dev = _qk_checked(pl, q, k)
    workspace = _workspace_checked(pl, workspace, dev)
    with torch.cuda.device(dev):
        st = _lib.lib().vsa_pool(ctypes.byref(pl.raw), q.data_ptr(), k.data_ptr(), workspace.data_ptr(),
                                 _stream_ptr(dev))
    _lib.check(st, "vsa_pool")
    return workspace


def score_topk(pl: Plan, workspace, sel=None):
    """The selection half of select (vsa_score_topk): scores the pooled
    means the workspace holds and writes the kept cube ids; returns sel."""
    import torch
    _check_device(workspace, "workspace", None)
    dev = workspace.device
    workspace = _workspace_checked(pl, workspace, dev)
    sel = _sel_checked(pl, sel, dev)
    with torch.cuda.device(dev):
        st = _lib.lib().vsa_score_topk(ctypes.byref(pl.raw), workspace.data_ptr(), sel.data_ptr(),
                                       _stream_ptr(dev))
    _lib.check(st, "vsa_score_topk")
    return sel


def attend(pl: Plan, q, k, v, sel, out=None):
    """Block-sparse attention over the kept blocks (vsa_attend)."""
    import torch
    shape = (pl.batch, pl.heads, pl.seq_len, pl.head_dim)
    strides = (pl.stride_b, pl.stride_h, pl.stride_n)
    kshape = (pl.batch, pl.heads, pl.seq_len_k, pl.head_dim)
    dt = _torch_dtype(pl)
    _check_qkv(q, "q", shape, strides, dt)
    dev = q.device
    for t, n in ((k, "k"), (v, "v")):
        _check_qkv(t, n, kshape, pl.kv_strides, dt, dev)
    if out is None:
        out = torch.empty_strided(shape, (pl.o_stride_b, pl.o_stride_h, pl.o_stride_n, 1),
                                  dtype=dt, device=dev)
    else:
        _check_qkv(out, "out", shape, (pl.o_stride_b, pl.o_stride_h, pl.o_stride_n), dt, dev)
    _check_device(sel, "sel", dev)
    if sel.dtype != torch.int32 or sel.numel() != pl.sel_elems or not sel.is_contiguous():
        raise ValueError("sel must be a contiguous int32 tensor of plan.sel_elems elements")
    with torch.cuda.device(dev):
        st = _lib.lib().vsa_attend(ctypes.byref(pl.raw), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                   sel.data_ptr(), out.data_ptr(), _stream_ptr(dev))
    _lib.check(st, "vsa_attend")
    return out


def forward(q, k, v, latent_shape: Sequence[int], cube_shape: Sequence[int], topk: int,
            prefix_len: int = 0, out=None, return_sel: bool = False,
            latent_shape_k: Optional[Sequence[int]] = None, cube_shape_k: Optional[Sequence[int]] = None):
    """Select then attend on the current stream. Returns out (and sel).
    ``latent_shape_k`` / ``cube_shape_k`` give k and v a grid of their own."""
    pl = plan_for(q, latent_shape, cube_shape, topk, prefix_len, out, k, latent_shape_k, cube_shape_k)
    sel, _ = select(pl, q, k)
    out = attend(pl, q, k, v, sel, out)
    return (out, sel) if return_sel else out


def topk_for_sparsity(num_blocks: int, sparsity: float) -> int:
    """Key cubes kept for a sparsity in [0, 1) (vsa_topk_for_sparsity):
    floor(num_blocks * (1 - sparsity)), at least 1."""
    r = _lib.lib().vsa_topk_for_sparsity(int(num_blocks), float(sparsity))
    if r < 0:
        raise VsaError(r, "vsa_topk_for_sparsity")
    return r


def flash_attn_bsa_3d(q, k, v, latent_shape_q: Sequence[int], latent_shape_k: Sequence[int],
                      sparsity: Optional[float] = None, chunk_3d_shape_q: Sequence[int] = (4, 4, 4),
                      chunk_3d_shape_k: Sequence[int] = (4, 4, 4), topk: Optional[int] = None,
                      prefix_len: int = 0, out=None):
    """fastbsa's call (package page, section "Use"): q on ``latent_shape_q``
    cut into ``chunk_3d_shape_q`` chunks, k and v on ``latent_shape_k`` cut
    into ``chunk_3d_shape_k``; each query chunk keeps the top (1 - sparsity)
    of the key chunks (or ``topk`` of them). Layout [B, heads, N, head_dim]
    as in ``forward``. Returns the output."""
    if (sparsity is None) == (topk is None):
        raise ValueError("give exactly one of sparsity and topk")
    if topk is None:
        # the key-chunk count from a plan of the problem (top-k 1 is always
        # valid); the sparsity then fixes top-k
        probe = plan_for(q, latent_shape_q, chunk_3d_shape_q, 1, prefix_len, out, k, latent_shape_k,
                         chunk_3d_shape_k)
        topk = topk_for_sparsity(probe.num_blocks, sparsity)
    return forward(q, k, v, latent_shape_q, chunk_3d_shape_q, topk, prefix_len, out,
                   latent_shape_k=latent_shape_k, cube_shape_k=chunk_3d_shape_k)


_ROUTES = {_lib.VSA_ROUTE_VSA: "VSA", _lib.VSA_ROUTE_VSA_ALL_BLOCKS: "VSA_ALL_BLOCKS",
           _lib.VSA_ROUTE_DENSE: "SDPA"}
_MODES = {"native": _lib.VSA_CHECKPOINT_NATIVE, "dmd": _lib.VSA_CHECKPOINT_DMD}


class Route:
    """A routing decision (vsa_route): ``route`` is "VSA", "VSA_ALL_BLOCKS"
    or "SDPA" (dense attention, which the caller runs; this library has no
    dense path), ``reason`` a VSA_REASON_* code, ``plan`` the plan to run
    the sparse kernels with (None on a dense route without geometry)."""

    def __init__(self, raw: _lib.VsaRoute):
        self.raw = raw
        self.route = _ROUTES[raw.route]
        self.reason = raw.reason
        self.status = raw.status
        self.topk = raw.topk
        self.plan = Plan(_lib.VsaPlan.from_buffer_copy(raw.plan)) if raw.has_plan else None

    @property
    def sparse(self) -> bool:
        return self.route != "SDPA"

    def log_line(self) -> str:
        buf = ctypes.create_string_buffer(768)
        n = _lib.lib().vsa_describe_route(ctypes.byref(self.raw), buf, len(buf))
        if n < 0:
            raise VsaError(n, "vsa_describe_route")
        return buf.value.decode()

    def __repr__(self):
        return f"Route({self.log_line()})"


def route(batch: int, heads: int, head_dim: int, latent: Sequence[int], cube: Sequence[int], topk: int,
          prefix_len: int = 0, checkpoint_mode: str = "native", **kw) -> Route:
    """Routing decision for a problem (vsa_route; the user guide's Wan rules:
    topk > num_blocks and, on a native checkpoint, topk == num_blocks go to
    dense attention; a DMD checkpoint keeps every block on the sparse path).
    ``kw`` are ``plan``'s optional arguments."""
    if checkpoint_mode not in _MODES:
        raise ValueError(f"checkpoint_mode must be one of {sorted(_MODES)}")
    pr = _problem(batch, heads, head_dim, latent, cube, topk, prefix_len, **kw)
    raw = _lib.VsaRoute()
    _lib.check(_lib.lib().vsa_route(ctypes.byref(pr), _MODES[checkpoint_mode], ctypes.byref(raw)), "vsa_route")
    return Route(raw)


def describe(pl: Plan) -> str:
    """The Wan routing-log fields for this plan (vsa_describe)."""
    buf = ctypes.create_string_buffer(512)
    n = _lib.lib().vsa_describe(ctypes.byref(pl.raw), buf, len(buf))
    if n < 0:
        raise VsaError(n, "vsa_describe")
    return buf.value.decode()
