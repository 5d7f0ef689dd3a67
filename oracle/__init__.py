"""CPU oracle for the skinny decode projection (fp64, plain loops in C).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import this package.  It shares no code with the HIP library and never
imports it.

The arithmetic lives in ``oracle.c`` (see its header for the page citations);
this module only builds that file with gcc and marshals numpy arrays to it.
bf16 tensors are passed as their raw uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(out_path: str = _LIB, src_path: str = _SRC) -> str:
    """Compile oracle.c into a shared library with gcc (plain -O2, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-ffp-contract=off", "-o", out_path, src_path, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


def load(path: str = _LIB) -> ctypes.CDLL:
    """Load a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    c_i64, c_p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
    lib.oracle_encode_bf16.argtypes = [c_i64, c_p, c_p]
    lib.oracle_projection.argtypes = [c_i64, c_i64, c_i64, c_p, c_p, c_p, c_p]
    lib.oracle_splitk_partials.argtypes = [c_i64, c_i64, c_i64, c_i64, c_p, c_p, c_p]
    lib.oracle_splitk_sum.argtypes = [c_i64, c_i64, c_p, c_p]
    lib.oracle_residual.argtypes = [c_i64, c_p, c_p, c_p]
    lib.oracle_moe_table.argtypes = [c_i64, c_i64, c_i64, c_p, c_p, c_p, c_p]
    lib.oracle_moe_table.restype = c_i64
    lib.oracle_grouped.argtypes = [c_i64] * 5 + [c_p] * 5
    lib.oracle_router_topk.argtypes = [c_i64, c_i64, c_i64, c_p, c_p, c_p]
    lib.oracle_router_topk.restype = None
    lib.oracle_e2m1_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m1_to_f64.restype = ctypes.c_double
    lib.oracle_e8m0_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_to_f64.restype = ctypes.c_double
    lib.oracle_projection_mxfp4.argtypes = [c_i64, c_i64, c_i64, c_p, c_p, c_p, c_p, c_p]
    lib.oracle_projection_mxfp4.restype = None
    lib.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_f64.restype = ctypes.c_double
    lib.oracle_projection_fp8.argtypes = [c_i64, c_i64, c_i64, c_p, c_p, c_p, c_p, c_p]
    lib.oracle_projection_fp8.restype = None
    for name in ("oracle_encode_bf16", "oracle_projection", "oracle_splitk_partials",
                 "oracle_splitk_sum", "oracle_residual", "oracle_grouped"):
        getattr(lib, name).restype = None
    return lib


def lib() -> ctypes.CDLL:
    """The default oracle library, built on first use if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = load(_LIB)
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _bits(a) -> np.ndarray:
    """Raw bf16 bit patterns as a contiguous uint16 array (accepts torch bf16 tensors)."""
    if hasattr(a, "view") and hasattr(a, "dtype") and str(a.dtype) == "torch.bfloat16":
        import torch
        a = a.detach().to("cpu").contiguous().view(torch.int16).numpy()
    a = np.ascontiguousarray(a)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected bf16 bit patterns (uint16), got {a.dtype}")
    return a


class Oracle:
    """numpy-facing wrapper; every method is one call into oracle.c."""

    def __init__(self, library: ctypes.CDLL | None = None):
        self.c = library if library is not None else lib()

    def bf16_to_f64(self, bits) -> np.ndarray:
        b = _bits(bits)
        return np.array([self.c.oracle_bf16_to_f64(int(v)) for v in b.ravel()],
                        dtype=np.float64).reshape(b.shape)

    def encode_bf16(self, v) -> np.ndarray:
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty(v.shape, dtype=np.uint16)
        self.c.oracle_encode_bf16(v.size, _ptr(v), _ptr(out))
        return out

    def projection(self, x, W, with_scale: bool = True):
        x, W = _bits(x), _bits(W)
        M, K = x.shape
        N, K2 = W.shape
        assert K == K2, (x.shape, W.shape)
        y = np.empty((M, N), dtype=np.float64)
        a = np.empty((M, N), dtype=np.float64) if with_scale else None
        self.c.oracle_projection(M, N, K, _ptr(x), _ptr(W), _ptr(y),
                                 _ptr(a) if a is not None else None)
        return (y, a) if with_scale else y

    def splitk_partials(self, x, W, S: int) -> np.ndarray:
        x, W = _bits(x), _bits(W)
        M, K = x.shape
        N = W.shape[0]
        P = np.empty((S, M, N), dtype=np.float64)
        self.c.oracle_splitk_partials(M, N, K, S, _ptr(x), _ptr(W), _ptr(P))
        return P

    def splitk_sum(self, P) -> np.ndarray:
        P = np.ascontiguousarray(P, dtype=np.float64)
        S = P.shape[0]
        y = np.empty(P.shape[1:], dtype=np.float64)
        self.c.oracle_splitk_sum(S, y.size, _ptr(P), _ptr(y))
        return y

    def residual(self, r, y) -> np.ndarray:
        r = _bits(r)
        y = np.ascontiguousarray(y, dtype=np.float64)
        assert r.shape == y.shape
        out = np.empty(y.shape, dtype=np.float64)
        self.c.oracle_residual(y.size, _ptr(r), _ptr(y), _ptr(out))
        return out

    def moe_table(self, ids, E: int):
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        T, topk = ids.shape
        counts = np.empty(E, dtype=np.int32)
        offsets = np.empty(E + 1, dtype=np.int32)
        sorted_pairs = np.empty(T * topk, dtype=np.int32)
        invalid = self.c.oracle_moe_table(T, topk, E, _ptr(ids), _ptr(counts),
                                          _ptr(offsets), _ptr(sorted_pairs))
        return counts, offsets, sorted_pairs, int(invalid)

    def grouped(self, x, W, ids, with_scale: bool = True):
        x, W = _bits(x), _bits(W)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        T, K = x.shape
        E, N, K2 = W.shape
        assert K == K2 and ids.shape[0] == T
        topk = ids.shape[1]
        out = np.empty((T, topk, N), dtype=np.float64)
        a = np.empty((T, topk, N), dtype=np.float64) if with_scale else None
        self.c.oracle_grouped(T, topk, E, N, K, _ptr(x), _ptr(W), _ptr(ids), _ptr(out),
                              _ptr(a) if a is not None else None)
        return (out, a) if with_scale else out

    def router_topk(self, scores, k: int):
        """ids int32 [T,k] and their scores float32 [T,k] from fp32 scores [T,E]."""
        scores = np.ascontiguousarray(scores, dtype=np.float32)
        T, E = scores.shape
        assert 1 <= k <= E
        ids = np.empty((T, k), dtype=np.int32)
        top = np.empty((T, k), dtype=np.float32)
        self.c.oracle_router_topk(T, E, k, _ptr(scores), _ptr(ids), _ptr(top))
        return ids, top

    def e2m1_to_f64(self, codes) -> np.ndarray:
        codes = np.asarray(codes, dtype=np.uint8).ravel()
        return np.array([self.c.oracle_e2m1_to_f64(int(c)) for c in codes], dtype=np.float64)

    def e8m0_to_f64(self, scales) -> np.ndarray:
        scales = np.asarray(scales, dtype=np.uint8).ravel()
        return np.array([self.c.oracle_e8m0_to_f64(int(s)) for s in scales], dtype=np.float64)

    def e4m3_to_f64(self, codes) -> np.ndarray:
        codes = np.asarray(codes, dtype=np.uint8).ravel()
        return np.array([self.c.oracle_e4m3_to_f64(int(c)) for c in codes], dtype=np.float64)

    def projection_fp8(self, x, Wq, Ws, with_scale: bool = True):
        """y = x W^T for FP8 weights: Wq uint8 [N, K] (e4m3 codes), Ws float32
        [ceil(N/128), ceil(K/128)] (one scale per 128 x 128 block)."""
        x = _bits(x)
        Wq = np.ascontiguousarray(Wq, dtype=np.uint8)
        Ws = np.ascontiguousarray(Ws, dtype=np.float32)
        M, K = x.shape
        N = Wq.shape[0]
        assert Wq.shape == (N, K) and Ws.shape == (-(-N // 128), -(-K // 128)), \
            (x.shape, Wq.shape, Ws.shape)
        y = np.empty((M, N), dtype=np.float64)
        a = np.empty((M, N), dtype=np.float64) if with_scale else None
        self.c.oracle_projection_fp8(M, N, K, _ptr(x), _ptr(Wq), _ptr(Ws), _ptr(y),
                                     _ptr(a) if a is not None else None)
        return (y, a) if with_scale else y

    def projection_mxfp4(self, x, Wq, Ws, with_scale: bool = True):
        """y = x W^T for MXFP4 weights: Wq uint8 [N, K/2] (two e2m1 codes a byte, low
        nibble first), Ws uint8 [N, K/32] (e8m0 block scales)."""
        x = _bits(x)
        Wq = np.ascontiguousarray(Wq, dtype=np.uint8)
        Ws = np.ascontiguousarray(Ws, dtype=np.uint8)
        M, K = x.shape
        N = Wq.shape[0]
        assert K % 32 == 0 and Wq.shape == (N, K // 2) and Ws.shape == (N, K // 32), \
            (x.shape, Wq.shape, Ws.shape)
        y = np.empty((M, N), dtype=np.float64)
        a = np.empty((M, N), dtype=np.float64) if with_scale else None
        self.c.oracle_projection_mxfp4(M, N, K, _ptr(x), _ptr(Wq), _ptr(Ws), _ptr(y),
                                       _ptr(a) if a is not None else None)
        return (y, a) if with_scale else y
