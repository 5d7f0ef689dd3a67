"""Python binding of libskinny_gemm.so: the batch-1..64 decode projection
y = x W^T (+ fused residual) and its routed-expert variant on MI355X.

Each function has the name of the C entry point it calls (include/
skinny_gemm.h) and only marshals arguments: torch tensors become device
pointers, the current torch stream becomes the hipStream_t, and a missing
workspace is allocated with torch (PyTorch provides memory and streams; every
step of the computation runs in the library's HIP kernels).  A non-SG_OK
status raises SkinnyGemmError.  There is no fallback: if the library is not
built, importing it raises.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (KERNEL_NAMES, SG_KERNEL_GEMV, SG_KERNEL_GROUPED, SG_KERNEL_MOE_TABLE,
                   SG_KERNEL_FP8, SG_KERNEL_MXFP4, SG_KERNEL_NONE, SG_KERNEL_PREFETCH, SG_KERNEL_REDUCE,
                   SG_KERNEL_ROUTER_TOPK,
                   SG_KERNEL_SPLITK_MFMA, SG_KERNEL_SPLITK_VALU, SG_NOALLOC_MAX_WORKSPACE,
                   SG_NUM_COUNTERS, SgMoeStep,
                   SgPlan, SkinnyGemmError)

__all__ = [
    "skinny_gemm_plan", "skinny_gemm_plan_force", "skinny_gemm", "skinny_gemm_residual",
    "skinny_gemm_noalloc", "SG_NOALLOC_MAX_WORKSPACE", "grouped_skinny_gemm_workspace",
    "grouped_skinny_gemm", "skinny_gemm_prefetch", "skinny_gemm_read_probe",
    "skinny_gemm_router_topk", "router_topk", "skinny_moe_step_workspace", "skinny_moe_step",
    "concat_router_shared", "MOE_STEP_MODES", "skinny_gemm_mxfp4", "SG_KERNEL_MXFP4",
    "skinny_gemm_fp8", "SG_KERNEL_FP8", "skinny_gemm_fp8_workspace", "skinny_gemm_mxfp4_workspace",
    "skinny_gemm_status_str", "skinny_gemm_get_counters", "skinny_gemm_reset_counters",
    "SgPlan", "SkinnyGemmError", "KERNEL_NAMES", "SG_KERNEL_NONE", "SG_KERNEL_GEMV",
    "SG_KERNEL_SPLITK_VALU", "SG_KERNEL_SPLITK_MFMA", "SG_KERNEL_REDUCE", "SG_KERNEL_MOE_TABLE",
    "SG_KERNEL_GROUPED", "SG_KERNEL_PREFETCH", "SG_KERNEL_ROUTER_TOPK", "SG_NUM_COUNTERS",
    "library_path",
]


def library_path() -> str:
    return _lib.LIB_PATH


def _c():
    return _lib.load()


def _ptr(t, dtype, name, device=None):
    """Device pointer of a contiguous tensor of the expected dtype (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t.data_ptr() or None


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _shape(t, shape, name):
    """The C ABI cannot see buffer sizes: refuse tensors whose shape disagrees with the plan."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} does not match the plan's {tuple(shape)}")


def _at_least(t, count, name):
    if t is not None and t.numel() < count:
        raise ValueError(f"{name}: needs at least {count} elements, has {t.numel()}")


def _workspace(nbytes: int, workspace, device):
    if nbytes == 0:
        return workspace, (workspace.numel() if workspace is not None else 0)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
        raise TypeError("workspace: expected a device tensor")
    return workspace, workspace.numel() * workspace.element_size()


def skinny_gemm_plan(M: int, N: int, K: int) -> SgPlan:
    """plan(M, N, K): kernel, split factor and workspace for y[M,N] = x[M,K] W[N,K]^T."""
    plan = SgPlan()
    _lib.check(_c().skinny_gemm_plan(M, N, K, ctypes.byref(plan)))
    return plan


def skinny_gemm_plan_force(M: int, N: int, K: int, kernel: int, split_k: int = 0,
                           two_pass: int = -1, tile_n: int = 0) -> SgPlan:
    """plan with the kernel (SG_KERNEL_*), split factor, reduction mode
    (0 in-kernel, 1 second pass, -1 library's choice) and, on the matrix
    cores, row tiling (16 team kernel, 128 or 256 chunk kernel, 0 library's
    choice) chosen by the caller."""
    plan = SgPlan()
    _lib.check(_c().skinny_gemm_plan_force(M, N, K, kernel, split_k, two_pass, tile_n,
                                           ctypes.byref(plan)))
    return plan


def skinny_gemm(plan: SgPlan, x: torch.Tensor, W: torch.Tensor, y_f32=None, y_bf16=None,
                workspace=None, stream=None):
    """y = x W^T into y_f32 (float32 [M,N]) and/or y_bf16 (bfloat16 [M,N])."""
    dev = x.device
    M, N, K = plan.M, plan.N, plan.K
    _shape(x, (M, K), "x"), _shape(W, (N, K), "W")
    _shape(y_f32, (M, N), "y_f32"), _shape(y_bf16, (M, N), "y_bf16")
    ws, ws_bytes = _workspace(plan.workspace_bytes, workspace, dev)
    st = _c().skinny_gemm(ctypes.byref(plan), _ptr(x, torch.bfloat16, "x", dev),
                          _ptr(W, torch.bfloat16, "W", dev),
                          _ptr(y_f32, torch.float32, "y_f32", dev),
                          _ptr(y_bf16, torch.bfloat16, "y_bf16", dev),
                          _ptr(ws, torch.uint8, "workspace", dev) if ws is not None else None,
                          ws_bytes, _stream(stream))
    _lib.check(st)
    return ws


def skinny_gemm_noalloc(plan: SgPlan, x: torch.Tensor, W: torch.Tensor, y_f32=None,
                        y_bf16=None, stream=None):
    """skinny_gemm without a workspace: split-K partials go to the library's own
    per-GPU scratch array (calls overlapping on one GPU race on it)."""
    dev = x.device
    M, N, K = plan.M, plan.N, plan.K
    _shape(x, (M, K), "x"), _shape(W, (N, K), "W")
    _shape(y_f32, (M, N), "y_f32"), _shape(y_bf16, (M, N), "y_bf16")
    st = _c().skinny_gemm_noalloc(ctypes.byref(plan), _ptr(x, torch.bfloat16, "x", dev),
                                  _ptr(W, torch.bfloat16, "W", dev),
                                  _ptr(y_f32, torch.float32, "y_f32", dev),
                                  _ptr(y_bf16, torch.bfloat16, "y_bf16", dev), _stream(stream))
    _lib.check(st)


def skinny_gemm_residual(plan: SgPlan, x: torch.Tensor, W: torch.Tensor, r: torch.Tensor,
                         out_bf16=None, out_f32=None, workspace=None, stream=None):
    """out = r + x W^T (one rounding) into out_bf16 (may be r itself) and/or out_f32."""
    dev = x.device
    M, N, K = plan.M, plan.N, plan.K
    _shape(x, (M, K), "x"), _shape(W, (N, K), "W"), _shape(r, (M, N), "r")
    _shape(out_f32, (M, N), "out_f32"), _shape(out_bf16, (M, N), "out_bf16")
    ws, ws_bytes = _workspace(plan.workspace_bytes, workspace, dev)
    st = _c().skinny_gemm_residual(ctypes.byref(plan), _ptr(x, torch.bfloat16, "x", dev),
                                   _ptr(W, torch.bfloat16, "W", dev),
                                   _ptr(r, torch.bfloat16, "r", dev),
                                   _ptr(out_bf16, torch.bfloat16, "out_bf16", dev),
                                   _ptr(out_f32, torch.float32, "out_f32", dev),
                                   _ptr(ws, torch.uint8, "workspace", dev) if ws is not None else None,
                                   ws_bytes, _stream(stream))
    _lib.check(st)
    return ws


def grouped_skinny_gemm_workspace(T: int, E: int, topk: int, N: int, K: int) -> int:
    return int(_c().grouped_skinny_gemm_workspace(T, E, topk, N, K))


def grouped_skinny_gemm(x: torch.Tensor, W: torch.Tensor, topk_ids: torch.Tensor, out: torch.Tensor,
                        expert_offsets=None, sorted_pairs=None, invalid_count=None,
                        workspace=None, stream=None):
    """out[t,j,:] = W[topk_ids[t,j]] @ x[t] for x [T,K], W [E,N,K], topk_ids [T,topk] int32."""
    dev = x.device
    T, K = x.shape
    E, N, K2 = W.shape
    if K2 != K or topk_ids.dim() != 2 or topk_ids.shape[0] != T:
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, W {tuple(W.shape)}, "
                         f"topk_ids {tuple(topk_ids.shape)}")
    topk = topk_ids.shape[1]
    _shape(out, (T, topk, N), "out")
    _at_least(expert_offsets, E + 1, "expert_offsets")
    _at_least(sorted_pairs, T * topk, "sorted_pairs")
    _at_least(invalid_count, 1, "invalid_count")
    need = grouped_skinny_gemm_workspace(T, E, topk, N, K)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _c().grouped_skinny_gemm(
        _ptr(x, torch.bfloat16, "x", dev), T, _ptr(W, torch.bfloat16, "W", dev), E, N, K,
        _ptr(topk_ids, torch.int32, "topk_ids", dev), topk, _ptr(out, torch.float32, "out", dev),
        _ptr(expert_offsets, torch.int32, "expert_offsets", dev),
        _ptr(sorted_pairs, torch.int32, "sorted_pairs", dev),
        _ptr(invalid_count, torch.int32, "invalid_count", dev),
        _ptr(workspace, torch.uint8, "workspace", dev), ws_bytes, _stream(stream))
    _lib.check(st)
    return workspace


def skinny_gemm_prefetch(W: torch.Tensor, nbytes: int | None = None, stream=None) -> None:
    """Warm [W, W + nbytes) into the GPU caches on `stream` (static weights only)."""
    if not W.is_cuda or not W.is_contiguous():
        raise ValueError("W: must be a contiguous device tensor")
    total = W.numel() * W.element_size()
    nbytes = total if nbytes is None else int(nbytes)
    if nbytes > total:
        raise ValueError("nbytes exceeds the tensor")
    _lib.check(_c().skinny_gemm_prefetch(W.data_ptr() or None, nbytes, _stream(stream)))


def skinny_gemm_read_probe(W: torch.Tensor, rows_per_iter: int, grid: int, stream=None) -> None:
    """Read W ([rows, row_bytes] contiguous device tensor) with the M <= 2 projection
    kernel's load shape and no arithmetic (a measurement of the read rate alone)."""
    if not W.is_cuda or not W.is_contiguous() or W.dim() != 2:
        raise ValueError("W: must be a contiguous 2-D device tensor")
    rows, row_bytes = W.shape[0], W.shape[1] * W.element_size()
    _lib.check(_c().skinny_gemm_read_probe(W.data_ptr() or None, rows, row_bytes, rows_per_iter,
                                           grid, _stream(stream)))


def skinny_gemm_router_topk(scores: torch.Tensor, k: int, topk_ids=None, topk_scores=None,
                            stream=None):
    """topk_ids (int32 [T,k]) and, if given, topk_scores (float32 [T,k]) from router
    scores (float32 [T,E]): larger score first, ties to the lower expert id, NaN as -inf."""
    if scores.dtype != torch.float32 or scores.dim() != 2 or not scores.is_contiguous():
        raise ValueError("scores: expected a contiguous float32 [T, E] tensor")
    T, E = scores.shape
    dev = scores.device
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    _shape(topk_ids, (T, k), "topk_ids"), _shape(topk_scores, (T, k), "topk_scores")
    st = _c().skinny_gemm_router_topk(
        _ptr(scores, torch.float32, "scores", dev), T, E, k,
        _ptr(topk_ids, torch.int32, "topk_ids", dev),
        _ptr(topk_scores, torch.float32, "topk_scores", dev), _stream(stream))
    _lib.check(st)
    return topk_ids


def router_topk(x: torch.Tensor, W_router: torch.Tensor, k: int, stream=None):
    """Expert selection for MoE decode: router scores y = x W_router^T (fp32, the
    planned skinny projection), then their top-k.  Returns (topk_ids [T,k] int32,
    topk_scores [T,k] float32, scores [T,E] float32)."""
    T, E = x.shape[0], W_router.shape[0]
    plan = skinny_gemm_plan(T, E, x.shape[1])
    scores = torch.empty((T, E), dtype=torch.float32, device=x.device)
    skinny_gemm(plan, x, W_router, y_f32=scores, stream=stream)
    top = torch.empty((T, k), dtype=torch.float32, device=x.device)
    ids = skinny_gemm_router_topk(scores, k, topk_scores=top, stream=stream)
    return ids, top, scores


def skinny_moe_step_workspace(T: int, K: int, E: int, topk: int, N: int, N_shared: int) -> int:
    return int(_c().skinny_moe_step_workspace(T, K, E, topk, N, N_shared))


_SIDE = {}  # device -> (side stream, fork event, join event), made once per device


def _side_resources(device):
    res = _SIDE.get(device)
    if res is None:
        with torch.cuda.device(device):
            side = torch.cuda.Stream(device=device)  # default priority
            fork, join = torch.cuda.Event(), torch.cuda.Event()
            cur = torch.cuda.current_stream(device)
            fork.record(cur)  # torch creates the hipEvent_t at its first record
            join.record(cur)
        res = (side, fork, join)
        _SIDE[device] = res
    return res


def skinny_gemm_fp8_workspace(M: int, N: int, K: int) -> int:
    """Workspace bytes skinny_gemm_fp8 needs for an M x N x K projection (0 when none)."""
    return int(_c().skinny_gemm_fp8_workspace(M, N, K))


def skinny_gemm_mxfp4_workspace(M: int, N: int, K: int) -> int:
    """Workspace bytes skinny_gemm_mxfp4 needs for an M x N x K projection (0 when none)."""
    return int(_c().skinny_gemm_mxfp4_workspace(M, N, K))


def skinny_gemm_mxfp4(x: torch.Tensor, W_codes: torch.Tensor, W_scales: torch.Tensor,
                      y_f32=None, y_bf16=None, r=None, workspace=None, stream=None):
    """y = x W^T for MXFP4 weights: W_codes uint8 [N, K/2] (two e2m1 codes a byte, low
    nibble first), W_scales uint8 [N, K/32] (e8m0 block scales); x bf16 [M, K], M <= 64.
    Writes y_f32 and/or y_bf16 [M, N]; with r (bf16 [M, N]) the fused residual
    y = r + x W^T.  Allocates y_f32 when no output is given, and the workspace (when
    the chunk kernel splits K) when none is given; returns the outputs."""
    dev = x.device
    M, K = x.shape
    N = W_codes.shape[0]
    if W_codes.shape != (N, K // 2) or W_scales.shape != (N, K // 32) or K % 32:
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, W_codes {tuple(W_codes.shape)}, "
                         f"W_scales {tuple(W_scales.shape)}")
    if y_f32 is None and y_bf16 is None:
        y_f32 = torch.empty((M, N), dtype=torch.float32, device=dev)
    for t, name in ((y_f32, "y_f32"), (y_bf16, "y_bf16"), (r, "r")):
        _shape(t, (M, N), name)
    ws, ws_bytes = _workspace(skinny_gemm_mxfp4_workspace(M, N, K), workspace, dev)
    st = _c().skinny_gemm_mxfp4(
        M, N, K, _ptr(x, torch.bfloat16, "x", dev), _ptr(W_codes, torch.uint8, "W_codes", dev),
        _ptr(W_scales, torch.uint8, "W_scales", dev), _ptr(r, torch.bfloat16, "r", dev),
        _ptr(y_f32, torch.float32, "y_f32", dev), _ptr(y_bf16, torch.bfloat16, "y_bf16", dev),
        _ptr(ws, torch.uint8, "workspace", dev) if ws is not None else None, ws_bytes,
        _stream(stream))
    _lib.check(st)
    return y_f32, y_bf16


def skinny_gemm_fp8(x: torch.Tensor, W_codes: torch.Tensor, W_scales: torch.Tensor,
                    y_f32=None, y_bf16=None, r=None, workspace=None, stream=None):
    """y = x W^T for FP8 weights: W_codes uint8 [N, K] (OCP E4M3 codes), W_scales float32
    [ceil(N/128), ceil(K/128)] (one scale per 128 x 128 block); x bf16 [M, K], M <= 64.
    Writes y_f32 and/or y_bf16 [M, N]; with r (bf16 [M, N]) the fused residual
    y = r + x W^T.  Allocates y_f32 when no output is given, and the workspace (when
    the chunk kernel splits K) when none is given; returns the outputs."""
    dev = x.device
    M, K = x.shape
    N = W_codes.shape[0]
    if W_codes.shape != (N, K) or W_scales.shape != (-(-N // 128), -(-K // 128)):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, W_codes {tuple(W_codes.shape)}, "
                         f"W_scales {tuple(W_scales.shape)}")
    if y_f32 is None and y_bf16 is None:
        y_f32 = torch.empty((M, N), dtype=torch.float32, device=dev)
    for t, name in ((y_f32, "y_f32"), (y_bf16, "y_bf16"), (r, "r")):
        _shape(t, (M, N), name)
    ws, ws_bytes = _workspace(skinny_gemm_fp8_workspace(M, N, K), workspace, dev)
    st = _c().skinny_gemm_fp8(
        M, N, K, _ptr(x, torch.bfloat16, "x", dev), _ptr(W_codes, torch.uint8, "W_codes", dev),
        _ptr(W_scales, torch.float32, "W_scales", dev), _ptr(r, torch.bfloat16, "r", dev),
        _ptr(y_f32, torch.float32, "y_f32", dev), _ptr(y_bf16, torch.bfloat16, "y_bf16", dev),
        _ptr(ws, torch.uint8, "workspace", dev) if ws is not None else None, ws_bytes,
        _stream(stream))
    _lib.check(st)
    return y_f32, y_bf16


def concat_router_shared(W_router: torch.Tensor, W_shared: torch.Tensor):
    """One [E + N_shared, K] tensor holding the router rows, then the shared expert's;
    returns its two views (W_router, W_shared) -- the weight layout the fused step reads."""
    both = torch.cat([W_router, W_shared], dim=0).contiguous()
    return both[:W_router.shape[0]], both[W_router.shape[0]:]


MOE_STEP_MODES = ("fused", "side_stream", "serial", "shared_in_routed")


def skinny_moe_step(x: torch.Tensor, W_router: torch.Tensor, W_experts: torch.Tensor,
                    W_shared, topk: int, mode: str = "fused", workspace=None, stream=None):
    """One MoE decode step: router scores, top-k and routed-expert projection on `stream`,
    plus the shared expert's projection (W_shared [N_shared,K], or None):
      "fused"       -- in the router's GEMM; W_shared must be stored right after W_router
                       (the two views concat_router_shared returns);
      "side_stream" -- on a side stream that overlaps the routing phase;
      "serial"      -- after the routed experts on `stream`;
      "shared_in_routed" -- up to 4 tokens (E <= 512), inside the routed-expert launch,
                       streamed while it ranks the scores (else as "serial").
    Returns (topk_ids [T,topk] int32, topk_scores [T,topk], scores [T,E], out [T,topk,N],
    shared_out [T,N_shared]; fp32).  In fused mode scores and shared_out are column
    views of one [T, E + N_shared] buffer."""
    if mode not in MOE_STEP_MODES:
        raise ValueError(f"mode: one of {MOE_STEP_MODES}")
    dev = x.device
    T, K = x.shape
    E, N, K2 = W_experts.shape
    N_shared = 0 if W_shared is None else W_shared.shape[0]
    if W_router.shape != (E, K) or K2 != K or (W_shared is not None and W_shared.shape[1] != K):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, W_router {tuple(W_router.shape)}, "
                         f"W_experts {tuple(W_experts.shape)}")
    fused = mode == "fused" and N_shared > 0
    if fused and W_shared.data_ptr() != W_router.data_ptr() + E * K * W_router.element_size():
        raise ValueError("fused mode: W_shared must follow W_router in memory "
                         "(use concat_router_shared)")
    f32 = dict(dtype=torch.float32, device=dev)
    ids = torch.empty((T, topk), dtype=torch.int32, device=dev)
    top = torch.empty((T, topk), **f32)
    out = torch.empty((T, topk, N), **f32)
    if fused:
        y = torch.empty((T, E + N_shared), **f32)
        scores, shared_out = y[:, :E], y[:, E:]
        w_router_ptr = _ptr(W_router, torch.bfloat16, "W_router", dev)
        scores_ptr, shared_ptr, w_shared_ptr = y.data_ptr() or None, None, None
    else:
        scores, shared_out = torch.empty((T, E), **f32), torch.empty((T, N_shared), **f32)
        w_router_ptr = _ptr(W_router, torch.bfloat16, "W_router", dev)
        scores_ptr = _ptr(scores, torch.float32, "scores", dev)
        shared_ptr = _ptr(shared_out, torch.float32, "shared_out", dev)
        w_shared_ptr = _ptr(W_shared, torch.bfloat16, "W_shared", dev)
    need = skinny_moe_step_workspace(T, K, E, topk, N, N_shared)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    step = SgMoeStep(
        _ptr(x, torch.bfloat16, "x", dev), w_router_ptr,
        _ptr(W_experts, torch.bfloat16, "W_experts", dev), w_shared_ptr, scores_ptr,
        _ptr(ids, torch.int32, "topk_ids", dev), _ptr(top, torch.float32, "topk_scores", dev),
        _ptr(out, torch.float32, "out", dev), shared_ptr, T, K, E, topk, N, N_shared,
        _lib.SG_MOE_STEP_FUSED_SHARED if fused
        else _lib.SG_MOE_STEP_SHARED_IN_ROUTED if mode == "shared_in_routed" else 0)
    side = fork = join = None
    if mode == "side_stream":
        s, f, j = _side_resources(dev)
        side, fork, join = s.cuda_stream, f.cuda_event, j.cuda_event
    st = _c().skinny_moe_step(ctypes.byref(step), _ptr(workspace, torch.uint8, "workspace", dev),
                              ws_bytes, _stream(stream), side, fork, join)
    _lib.check(st)
    return ids, top, scores, out, shared_out


def skinny_gemm_status_str(status: int) -> str:
    return _c().skinny_gemm_status_str(status).decode()


def skinny_gemm_get_counters() -> list[int]:
    arr = (ctypes.c_uint64 * SG_NUM_COUNTERS)()
    _c().skinny_gemm_get_counters(arr)
    return list(arr)


def skinny_gemm_reset_counters() -> None:
    _c().skinny_gemm_reset_counters()
