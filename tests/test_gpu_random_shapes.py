"""GPU parity over seeded random projection shapes: every plan the library picks
for 1 <= M <= 64, ragged N and K (K % 8 == 0), with and without the fused
residual, checked element by element against the fp64 oracle on sampled rows.

The fixed-shape tests cover the workload sizes and forced plans; this sweep
covers the planner's choices in between (split factors, row tiles, the team /
chunk / small-matrix boundaries, chunk tails that end inside a 128-byte line).
"""
import numpy as np
import pytest
import torch

import seeded_inputs as si
import skinny_gemm_projection_amd as sg
from gpu_common import DEV, announce, bits, check_bf16, check_f32, orc, sample_rows

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def _shapes(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        # half the cases at M <= 16 (small-matrix, VALU and team kernels), half above
        M = int(rng.integers(1, 17)) if i % 2 == 0 else int(rng.integers(17, 65))
        N = int(rng.integers(1, 9000))
        K = 8 * int(rng.integers(1, 1300))  # 8 .. 10392
        out.append((i, M, N, K, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("i,M,N,K,residual", _shapes(48, 20261202))
def test_random_shape(i, M, N, K, residual):
    plan = sg.skinny_gemm_plan(M, N, K)
    announce(f"random shape {i}: M={M} N={N} K={K} residual={residual} "
             f"kernel={sg.KERNEL_NAMES[plan.kernel]} S={plan.split_k} tile={plan.tile_n}")
    seed = 30000 + 10 * i
    x = si.normal_bf16((M, K), 1.0, seed, DEV)
    W = si.normal_bf16((N, K), 0.02, seed + 1, DEV)
    y32 = torch.full((M, N), float("nan"), device=DEV)
    y16 = torch.full((M, N), float("nan"), device=DEV, dtype=torch.bfloat16)
    rows = sample_rows(N, min(N, 200), seed + 2)
    rt = torch.as_tensor(rows, device=DEV)
    y, A = orc().projection(bits(x), bits(W)[rows])
    if residual:
        r = si.normal_bf16((M, N), 1.0, seed + 3, DEV)
        sg.skinny_gemm_residual(plan, x, W, r, out_bf16=y16, out_f32=y32)
        torch.cuda.synchronize()
        ref = orc().residual(bits(r)[:, rows], y)
        check_f32(y32[:, rt], ref, A, f"shape {i} residual fp32", extra=2.0 ** -23 * np.abs(ref))
        check_bf16(y16[:, rt], ref, A, f"shape {i} residual bf16")
    else:
        sg.skinny_gemm(plan, x, W, y_f32=y32, y_bf16=y16)
        torch.cuda.synchronize()
        check_f32(y32[:, rt], y, A, f"shape {i} fp32")
        check_bf16(y16[:, rt], y, A, f"shape {i} bf16")
    # every output written (no NaN left from the fill), not only the sampled rows
    assert not torch.isnan(y32).any(), "every fp32 output written"


def _lp_shapes(count, seed, unit):
    """Seeded (M, N, K) for the low-precision paths, K a multiple of `unit`, within
    each path's limits (the vector kernels' x storage bounds K at small M)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        M = int(rng.integers(1, 17))
        N = int(rng.integers(1, 9000))
        if unit == 16:  # FP8: M*K <= 32768 at M <= 2, K <= 16384 at M = 3, 4
            kmax = 32768 // M if M <= 2 else 16384 if M <= 4 else 20000
        else:           # MXFP4: 32768 at M <= 2, 16384 at M = 3..8
            kmax = 32768 if M <= 2 else 16384 if M <= 8 else 20000
        K = unit * int(rng.integers(1, kmax // unit + 1))
        out.append((i, M, N, K, bool(rng.integers(0, 2))))
    return out


def _lp_shapes_wide(count, seed, unit, first):
    """Seeded (M, N, K) with 17 <= M <= 64 (the chunk kernel), K a multiple of `unit`
    up to 20000; numbered from `first`."""
    rng = np.random.default_rng(seed)
    return [(first + i, int(rng.integers(17, 65)), int(rng.integers(1, 9000)),
             unit * int(rng.integers(1, 20000 // unit + 1)), bool(rng.integers(0, 2)))
            for i in range(count)]


@pytest.mark.parametrize("i,M,N,K,residual",
                         _lp_shapes(24, 20261203, 16) + _lp_shapes_wide(16, 20261213, 16, 24))
def test_random_shape_fp8(i, M, N, K, residual):
    announce(f"random fp8 shape {i}: M={M} N={N} K={K} residual={residual}")
    seed = 31000 + 10 * i
    x = si.normal_bf16((M, K), 1.0, seed, DEV)
    codes, scales = si.fp8_weights(N, K, seed + 1, DEV)
    r = si.normal_bf16((M, N), 1.0, seed + 3, DEV) if residual else None
    y32 = torch.full((M, N), float("nan"), device=DEV)
    y16 = torch.full((M, N), float("nan"), device=DEV, dtype=torch.bfloat16)
    sg.skinny_gemm_fp8(x, codes, scales, y_f32=y32, y_bf16=y16, r=r)
    torch.cuda.synchronize()
    c, s, xb = codes.cpu().numpy(), scales.cpu().numpy(), bits(x)
    for n in sample_rows(N, min(N, 24), seed + 2):
        ref, A = orc().projection_fp8(xb, c[n:n + 1], s[n // 128:n // 128 + 1])
        extra = 0.0
        if residual:
            ref = orc().residual(bits(r)[:, n:n + 1], ref)
            extra = 2.0 ** -23 * np.abs(ref)
        check_f32(y32[:, n:n + 1], ref, A, f"fp8 shape {i} row {n}", extra=extra)
        check_bf16(y16[:, n:n + 1], ref, A, f"fp8 shape {i} row {n} bf16")
    assert not torch.isnan(y32).any(), "every fp32 output written"


@pytest.mark.parametrize("i,M,N,K,residual",
                         _lp_shapes(24, 20261204, 32) + _lp_shapes_wide(16, 20261214, 32, 24))
def test_random_shape_mxfp4(i, M, N, K, residual):
    announce(f"random mxfp4 shape {i}: M={M} N={N} K={K} residual={residual}")
    seed = 32000 + 10 * i
    x = si.normal_bf16((M, K), 1.0, seed, DEV)
    codes, scales = si.mxfp4_weights(N, K, seed + 1, DEV)
    r = si.normal_bf16((M, N), 1.0, seed + 3, DEV) if residual else None
    y32 = torch.full((M, N), float("nan"), device=DEV)
    y16 = torch.full((M, N), float("nan"), device=DEV, dtype=torch.bfloat16)
    sg.skinny_gemm_mxfp4(x, codes, scales, y_f32=y32, y_bf16=y16, r=r)
    torch.cuda.synchronize()
    c, s, xb = codes.cpu().numpy(), scales.cpu().numpy(), bits(x)
    for n in sample_rows(N, min(N, 24), seed + 2):
        ref, A = orc().projection_mxfp4(xb, c[n:n + 1], s[n:n + 1])
        extra = 0.0
        if residual:
            ref = orc().residual(bits(r)[:, n:n + 1], ref)
            extra = 2.0 ** -23 * np.abs(ref)
        check_f32(y32[:, n:n + 1], ref, A, f"mxfp4 shape {i} row {n}", extra=extra)
        check_bf16(y16[:, n:n + 1], ref, A, f"mxfp4 shape {i} row {n} bf16")
    assert not torch.isnan(y32).any(), "every fp32 output written"
