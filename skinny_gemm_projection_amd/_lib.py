"""ctypes view of libskinny_gemm.so (the C ABI in include/skinny_gemm.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any entry point.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libskinny_gemm.so")

SG_OK = 0
STATUS_NAMES = {0: "SG_OK", 1: "SG_ERR_NULL", 2: "SG_ERR_SHAPE", 3: "SG_ERR_UNSUPPORTED",
                4: "SG_ERR_ALIGN", 5: "SG_ERR_WORKSPACE", 6: "SG_ERR_PLAN", 7: "SG_ERR_HIP"}

SG_KERNEL_NONE = 0
SG_KERNEL_GEMV = 1
SG_KERNEL_SPLITK_VALU = 2
SG_KERNEL_SPLITK_MFMA = 3
SG_KERNEL_REDUCE = 4
SG_KERNEL_MOE_TABLE = 5
SG_KERNEL_GROUPED = 6
SG_KERNEL_PREFETCH = 7
SG_KERNEL_ROUTER_TOPK = 8
SG_KERNEL_MXFP4 = 9
SG_KERNEL_FP8 = 10
SG_NUM_COUNTERS = 11
KERNEL_NAMES = {0: "none", 1: "gemv", 2: "splitk_valu", 3: "splitk_mfma", 4: "reduce",
                5: "moe_table", 6: "grouped", 7: "prefetch", 8: "router_topk", 9: "mxfp4",
                10: "fp8"}


class SgPlan(ctypes.Structure):
    """Mirror of sg_plan."""
    _fields_ = [("M", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("kernel", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("k_chunk", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("two_pass", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}

    def __repr__(self) -> str:
        d = self.as_dict()
        d["kernel"] = KERNEL_NAMES.get(d["kernel"], d["kernel"])
        return f"SgPlan({d})"


class SgMoeStep(ctypes.Structure):
    """Mirror of sg_moe_step."""
    _fields_ = [("x", ctypes.c_void_p), ("W_router", ctypes.c_void_p),
                ("W_experts", ctypes.c_void_p), ("W_shared", ctypes.c_void_p),
                ("scores", ctypes.c_void_p), ("topk_ids", ctypes.c_void_p),
                ("topk_scores", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("shared_out", ctypes.c_void_p),
                ("T", ctypes.c_int32), ("K", ctypes.c_int32), ("E", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("N", ctypes.c_int32), ("N_shared", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


SG_MOE_STEP_FUSED_SHARED = 1
SG_MOE_STEP_SHARED_IN_ROUTED = 2
SG_NOALLOC_MAX_WORKSPACE = 16 << 20


class SkinnyGemmError(RuntimeError):
    """A non-SG_OK status from the library; .status holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"libskinny_gemm.so not found at {path}; build it with "
            "`python -m skinny_gemm_projection_amd.build` (there is no fallback path)")
    lib = ctypes.CDLL(path)
    i32, p, sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER(SgPlan)
    lib.skinny_gemm_plan.argtypes = [i32, i32, i32, P]
    lib.skinny_gemm_plan_force.argtypes = [i32, i32, i32, i32, i32, i32, i32, P]
    lib.skinny_gemm.argtypes = [P, p, p, p, p, p, sz, p]
    lib.skinny_gemm_residual.argtypes = [P, p, p, p, p, p, p, sz, p]
    lib.skinny_gemm_noalloc.argtypes = [P, p, p, p, p, p]
    lib.grouped_skinny_gemm_workspace.argtypes = [i32, i32, i32, i32, i32]
    lib.grouped_skinny_gemm_workspace.restype = sz
    lib.grouped_skinny_gemm.argtypes = [p, i32, p, i32, i32, i32, p, i32, p, p, p, p, p, sz, p]
    lib.skinny_gemm_prefetch.argtypes = [p, sz, p]
    lib.skinny_gemm_read_probe.argtypes = [p, i32, i32, i32, i32, p]
    lib.skinny_gemm_router_topk.argtypes = [p, i32, i32, i32, p, p, p]
    lib.skinny_gemm_mxfp4.argtypes = [i32, i32, i32, p, p, p, p, p, p, p, sz, p]
    lib.skinny_gemm_fp8.argtypes = [i32, i32, i32, p, p, p, p, p, p, p, sz, p]
    for name in ("skinny_gemm_fp8_workspace", "skinny_gemm_mxfp4_workspace"):
        getattr(lib, name).argtypes = [i32, i32, i32]
        getattr(lib, name).restype = sz
    lib.skinny_moe_step_workspace.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.skinny_moe_step_workspace.restype = sz
    lib.skinny_moe_step.argtypes = [ctypes.POINTER(SgMoeStep), p, sz, p, p, p, p]
    lib.skinny_gemm_status_str.argtypes = [ctypes.c_int]
    lib.skinny_gemm_status_str.restype = ctypes.c_char_p
    lib.skinny_gemm_get_counters.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
    lib.skinny_gemm_get_counters.restype = None
    lib.skinny_gemm_reset_counters.argtypes = []
    lib.skinny_gemm_reset_counters.restype = None
    for name in ("skinny_gemm_plan", "skinny_gemm_plan_force", "skinny_gemm",
                 "skinny_gemm_residual", "skinny_gemm_noalloc", "grouped_skinny_gemm", "skinny_gemm_prefetch",
                 "skinny_gemm_router_topk", "skinny_moe_step", "skinny_gemm_mxfp4",
                 "skinny_gemm_fp8"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != SG_OK:
        msg = load().skinny_gemm_status_str(status).decode()
        raise SkinnyGemmError(status, msg)
