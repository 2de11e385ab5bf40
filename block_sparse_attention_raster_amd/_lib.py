"""ctypes view of libvsa.so's C ABI (include/vsa.h). Marshalling only."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libvsa.so")

VSA_OK = 0
VSA_ERR_INVALID_ARG = -1
VSA_ERR_TOPK = -2
VSA_ERR_UNSUPPORTED = -3
VSA_ERR_ALIGN = -4
VSA_ERR_OVERFLOW = -5
VSA_ERR_DEVICE = -6
VSA_ERR_LAUNCH = -7
VSA_ERR_SCRATCH = -8
VSA_DTYPE_BF16 = 0
VSA_DTYPE_F16 = 1
VSA_SIDE_Q = 0
VSA_SIDE_K = 1

EXPORTED = ("vsa_plan", "vsa_topk_for_sparsity", "vsa_select", "vsa_attend", "vsa_forward",
            "vsa_describe", "vsa_status_str", "vsa_route", "vsa_describe_route", "vsa_block_counts",
            "vsa_pool", "vsa_score_topk", "vsa_forward_noalloc")

VSA_ROUTE_VSA = 0
VSA_ROUTE_VSA_ALL_BLOCKS = 1
VSA_ROUTE_DENSE = 2
VSA_CHECKPOINT_NATIVE = 0
VSA_CHECKPOINT_DMD = 1
VSA_REASON_NONE = 0
VSA_REASON_TOPK_ABOVE_BLOCKS = 1
VSA_REASON_ALL_BLOCKS_NATIVE = 2
VSA_REASON_UNSUPPORTED = 3


class VsaProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("latent", ctypes.c_int32 * 3), ("cube", ctypes.c_int32 * 3),
        ("topk", ctypes.c_int32), ("prefix_len", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64),
        ("o_stride_b", ctypes.c_int64), ("o_stride_h", ctypes.c_int64), ("o_stride_n", ctypes.c_int64),
        ("latent_k", ctypes.c_int32 * 3), ("cube_k", ctypes.c_int32 * 3),
        ("kv_stride_b", ctypes.c_int64), ("kv_stride_h", ctypes.c_int64), ("kv_stride_n", ctypes.c_int64),
    ]


class VsaPlan(ctypes.Structure):
    _fields_ = [
        ("p", VsaProblem),
        ("nblk", ctypes.c_int32 * 3),
        ("num_blocks", ctypes.c_int32), ("num_prefix_blocks", ctypes.c_int32),
        ("num_q_blocks", ctypes.c_int32), ("cube_volume", ctypes.c_int32),
        ("seq_len", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
        ("kbar_offset", ctypes.c_int64), ("sel_elems", ctypes.c_int64),
        ("scale", ctypes.c_float),
        ("select_rows", ctypes.c_int32), ("attend_variant", ctypes.c_int32),
        ("attend_tiles", ctypes.c_int32),
        ("nblk_k", ctypes.c_int32 * 3), ("num_prefix_blocks_k", ctypes.c_int32),
        ("cube_volume_k", ctypes.c_int32), ("seq_len_k", ctypes.c_int64),
    ]


class VsaRoute(ctypes.Structure):
    _fields_ = [
        ("route", ctypes.c_int32), ("reason", ctypes.c_int32), ("status", ctypes.c_int32),
        ("checkpoint_mode", ctypes.c_int32), ("topk", ctypes.c_int32), ("has_plan", ctypes.c_int32),
        ("plan", VsaPlan),
    ]


class VsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


_lib = None


def hip_runtimes_mapped() -> set:
    """Distinct HIP runtime files (libamdhip64) mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return {os.path.realpath(line.split()[-1]) for line in f if "libamdhip64" in line}
    except OSError:  # pragma: no cover - not Linux
        return set()


def lib() -> ctypes.CDLL:
    """Load libvsa.so once. Raises if it has not been built: there is no
    fallback path.

    The library must share PyTorch's HIP runtime (PyTorch owns the device
    memory and streams it is given). PyTorch ships its own copy of the
    runtime, so torch is imported first: the library's dependency then
    resolves to the copy already loaded. Loaded the other way round, the
    process would hold two runtimes, and the library's would not see the
    memory or the device that torch's set up; that state raises here."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing; build it with "
                "`python -m block_sparse_attention_raster_amd.build` (hipcc, gfx950)")
        try:
            import torch  # noqa: F401  (loads torch's HIP runtime before this library)
        except ImportError:  # pragma: no cover - the binding is used with torch
            pass
        L = ctypes.CDLL(LIB_PATH)
        runtimes = hip_runtimes_mapped()
        if len(runtimes) > 1:
            raise RuntimeError(
                "two HIP runtimes are loaded in this process (" + ", ".join(sorted(runtimes)) + "): "
                f"{LIB_PATH} must use the one torch uses; import torch before loading it")
        vp = ctypes.c_void_p
        L.vsa_plan.argtypes = [ctypes.POINTER(VsaProblem), ctypes.POINTER(VsaPlan)]
        L.vsa_plan.restype = ctypes.c_int
        L.vsa_topk_for_sparsity.argtypes = [ctypes.c_int32, ctypes.c_double]
        L.vsa_topk_for_sparsity.restype = ctypes.c_int
        L.vsa_select.argtypes = [ctypes.POINTER(VsaPlan), vp, vp, vp, vp, vp]
        L.vsa_select.restype = ctypes.c_int
        L.vsa_pool.argtypes = [ctypes.POINTER(VsaPlan), vp, vp, vp, vp]
        L.vsa_pool.restype = ctypes.c_int
        L.vsa_score_topk.argtypes = [ctypes.POINTER(VsaPlan), vp, vp, vp]
        L.vsa_score_topk.restype = ctypes.c_int
        L.vsa_attend.argtypes = [ctypes.POINTER(VsaPlan), vp, vp, vp, vp, vp, vp]
        L.vsa_attend.restype = ctypes.c_int
        L.vsa_forward.argtypes = [ctypes.POINTER(VsaPlan), vp, vp, vp, vp, vp, vp, vp]
        L.vsa_forward.restype = ctypes.c_int
        L.vsa_forward_noalloc.argtypes = [ctypes.POINTER(VsaPlan), vp, vp, vp, vp, vp, vp]
        L.vsa_forward_noalloc.restype = ctypes.c_int
        L.vsa_describe.argtypes = [ctypes.POINTER(VsaPlan), ctypes.c_char_p, ctypes.c_size_t]
        L.vsa_describe.restype = ctypes.c_int
        L.vsa_route.argtypes = [ctypes.POINTER(VsaProblem), ctypes.c_int32, ctypes.POINTER(VsaRoute)]
        L.vsa_route.restype = ctypes.c_int
        L.vsa_describe_route.argtypes = [ctypes.POINTER(VsaRoute), ctypes.c_char_p, ctypes.c_size_t]
        L.vsa_describe_route.restype = ctypes.c_int
        L.vsa_block_counts.argtypes = [ctypes.POINTER(VsaPlan), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                       ctypes.c_int64]
        L.vsa_block_counts.restype = ctypes.c_int
        L.vsa_status_str.argtypes = [ctypes.c_int]
        L.vsa_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().vsa_status_str(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != VSA_OK:
        raise VsaError(status, where)
