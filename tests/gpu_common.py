"""Shared helpers for the GPU parity tests (imported only by tests marked gpu).

Parity bar, element by element against the fp64 oracle on the same seeded
inputs (both sides read the very same bf16 tensors):
  * fp32 outputs:  |got - ref| <= 1e-3 * A,   A = sum_k |x_k * w_k|
  * bf16 outputs:  |got - ref| <= 1e-3 * A + 2^-8 * |ref|  (one extra RNE, and
    the oracle's own rounding of the exact value)
  * indices, and every output on integer-valued inputs: bit-exact.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import seeded_inputs as si

DEV = "cuda"
_ORACLE = None


def orc() -> oracle.Oracle:
    global _ORACLE
    if _ORACLE is None:
        _ORACLE = oracle.Oracle()
    return _ORACLE


def _threads() -> int:
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, 16, int(cap) if cap.isdigit() and int(cap) > 0 else 16))


def projection_all_rows(xb: np.ndarray, Wb: np.ndarray):
    """oracle_projection (y and A) of every row of W, the rows split over host
    threads: each thread runs the unchanged single-threaded oracle on its slice
    (the C call releases the GIL)."""
    N = Wb.shape[0]
    t = _threads()
    cuts = sorted({int(round(N * i / t)) for i in range(t + 1)})
    with ThreadPoolExecutor(max_workers=t) as pool:
        parts = list(pool.map(lambda ab: orc().projection(xb, Wb[ab[0]:ab[1]]),
                              zip(cuts, cuts[1:])))
    return (np.concatenate([p[0] for p in parts], axis=1),
            np.concatenate([p[1] for p in parts], axis=1))


def announce(msg: str) -> None:
    """Name the case on stdout before its GPU step (flushed, so a hang names it)."""
    print(f"[gpu case] {msg}", flush=True)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    return si.bits(t)


def _report(err, bound, what):
    bad = ~(err <= bound)
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err / np.maximum(bound, 1e-300), 0)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
                             f"worst at {idx}: err {err[idx]:.3e} > bound {bound[idx]:.3e}")


def check_f32(got: torch.Tensor, ref: np.ndarray, A: np.ndarray, what: str, extra=0.0) -> None:
    """fp32 bar 1e-3*A; `extra` adds the rounding of a residual sum (2^-23 * |r + y|)."""
    g = to_np(got).reshape(ref.shape)
    _report(np.abs(g - ref), 1e-3 * A + extra, what)


def check_bf16(got: torch.Tensor, ref: np.ndarray, A: np.ndarray, what: str) -> None:
    g = to_np(got).reshape(ref.shape)
    _report(np.abs(g - ref), 1e-3 * A + 2.0 ** -8 * np.abs(ref), what)


def check_exact(got: torch.Tensor, ref: np.ndarray, what: str) -> None:
    g = to_np(got).reshape(ref.shape)
    bad = g != ref
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} elements differ (must be bit-exact)"


def sample_rows(N: int, count: int, seed: int) -> np.ndarray:
    """Sorted distinct row indices: random ones plus the first and the last (ragged tail)."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, size=min(count, N), replace=False).tolist())
    rows.update({0, N - 1})
    return np.array(sorted(rows), dtype=np.int64)


def counters_delta(before, after):
    return [a - b for a, b in zip(after, before)]
