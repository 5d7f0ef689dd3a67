"""GPU parity of the projection with FP8 weights (skinny_gemm_fp8: e4m3 codes, one fp32
scale per 128 x 128 block) through the C ABI, M = 1..64 (vector ALU, matrix cores, and
from 8 or 12 rows the chunk kernel with its split-K reduction), against oracle_projection_fp8
on the same seeded codes and scales: fp32 |got - ref| <= 1e-3 * A, bf16 adds 2^-8 |ref|, the
residual adds 2^-23 |r + y|.  Integer-valued activations and weights with power-of-two
scales are bit-exact (every product and partial sum is exact in fp32)."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
import skinny_gemm_projection_amd as sg
from gpu_common import (DEV, announce, bits, check_bf16, check_exact, check_f32, counters_delta,
                        orc, sample_rows)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def host(t):
    return t.cpu().numpy()


def run(x, codes, scales, r=None, f32=True, bf16=True):
    M, N = x.shape[0], codes.shape[0]
    y32 = torch.full((M, N), -7.0, device=DEV) if f32 else None
    y16 = torch.full((M, N), -7.0, device=DEV, dtype=torch.bfloat16) if bf16 else None
    before = sg.skinny_gemm_get_counters()
    sg.skinny_gemm_fp8(x, codes, scales, y_f32=y32, y_bf16=y16, r=r)
    torch.cuda.synchronize()
    d = counters_delta(before, sg.skinny_gemm_get_counters())
    assert d[sg.SG_KERNEL_FP8] == (1 if M > 0 and N > 0 else 0)
    # the chunk kernel adds the reduction when it splits K (the only case with a workspace)
    splits = sg.skinny_gemm_fp8_workspace(M, N, x.shape[1]) > 0
    assert d[sg.SG_KERNEL_REDUCE] == (1 if splits and N > 0 else 0)
    return y32, y16


SHAPES = [(1, 40, 16), (1, 129, 112), (1, 200, 1040), (1, 77, 8192), (1, 33, 8208),
          (1, 300, 20000), (2, 50, 4128), (2, 130, 16384), (3, 70, 2080), (3, 129, 7168),
          (4, 96, 4160), (4, 257, 8192),
          # from M = 3 x stays in registers: K up to 16384 (8-wave teams)
          (3, 140, 12304), (4, 129, 16384), (3, 65, 16384),
          # from M = 5 the matrix-core kernel: 128-column windows split over a team,
          # ragged last window, ragged 16-row tile, any K
          (5, 100, 1040), (6, 131, 4112), (7, 64, 7168), (8, 257, 8192), (8, 33, 16),
          (9, 129, 2064), (11, 300, 7168), (10, 40, 20000), (11, 1, 144), (11, 200, 30000),
          # from 8161 rows two 16-row tiles per wave (ragged last 32-row tile)
          (9, 8200, 144), (11, 8192, 1040), (5, 8177, 2064),
          # 8 to 11 rows with a K whose chunks do not fit in LDS: the matrix-core kernel
          (9, 5, 524288),
          # the chunk kernel (from 8 rows, from 12 where N/32 is a whole multiple of
          # 256): x rows padded to 16, 32, 48, 64; ragged
          # 128-row tiles and windows; one split (K = 16), several, 256-row tiles
          (12, 300, 7168), (16, 40, 20000), (16, 1, 144), (13, 200, 30000),
          (16, 8192, 1040), (14, 8177, 2064),
          (17, 200, 1040), (20, 129, 7168), (32, 300, 4112), (33, 64, 16), (47, 257, 2064),
          (48, 1000, 8192), (64, 33, 30000), (64, 8200, 1040), (17, 6300, 4096),
          (40, 128, 128), (64, 1, 144)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_fp8_small(M, N, K):
    announce(f"fp8 M={M} N={N} K={K}")
    x = si.normal_bf16((M, K), 1.0, 8500 + K + M, DEV)
    codes, scales = si.fp8_weights(N, K, 8600 + N + K, DEV)
    y32, y16 = run(x, codes, scales)
    ref, A = orc().projection_fp8(bits(x), host(codes), host(scales))
    check_f32(y32, ref, A, f"fp8 fp32 M={M} N={N} K={K}")
    check_bf16(y16, ref, A, f"fp8 bf16 M={M} N={N} K={K}")
    # residual epilogue, in place on the bf16 output
    r = si.normal_bf16((M, N), 1.0, 8700 + N, DEV)
    out = r.clone()
    sg.skinny_gemm_fp8(x, codes, scales, y_bf16=out, r=out)
    torch.cuda.synchronize()
    rr = orc().bf16_to_f64(bits(r)).reshape(M, N)
    check_bf16(out, rr + ref, A, f"fp8 residual M={M} N={N} K={K}")
    y32b, _ = run(x, codes, scales, bf16=False)
    assert torch.equal(y32, y32b), "repeat runs bitwise identical"


# e4m3 codes of the integers 1..8 (and their negatives: bit 7)
INT_CODES = [0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50]


@pytest.mark.parametrize("M,N,K", [(1, 300, 4096), (2, 129, 8192), (4, 140, 2064),
                                   (8, 200, 8192), (6, 77, 3088), (16, 150, 8192),
                                   (11, 64, 2064), (17, 300, 8192), (32, 129, 4112),
                                   (64, 260, 8192), (50, 8200, 2064)])
def test_fp8_integer_bit_exact(M, N, K):
    # integer activations and weights, power-of-two block scales: exact sums
    announce(f"fp8 integer M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 1000 + N)
    x = si.integer_bf16((M, K), -3, 3, 8800 + M, DEV)
    c = np.array(INT_CODES, dtype=np.uint8)[rng.integers(0, 8, (N, K))]
    c |= (rng.integers(0, 2, (N, K)) * 0x80).astype(np.uint8)
    codes = torch.from_numpy(c).to(DEV)
    scales = torch.from_numpy(np.ldexp(1.0, rng.integers(-2, 2, (-(-N // 128), -(-K // 128))))
                              .astype(np.float32)).to(DEV)
    y32, y16 = run(x, codes, scales)
    ref = orc().projection_fp8(bits(x), c, host(scales), with_scale=False)
    check_exact(y32, ref, f"fp8 integer M={M}")
    assert np.array_equal(bits(y16), orc().encode_bf16(ref)), "bf16 output bit-exact"


@pytest.mark.parametrize("M,N", [(2, 300), (12, 300), (12, 8200), (20, 300), (64, 8200)])
def test_fp8_nan_code_and_scale(M, N):
    K = 512
    x = si.normal_bf16((M, K), 1.0, 8900 + M, DEV)
    codes, scales = si.fp8_weights(N, K, 8901, DEV)
    codes[5, 17] = 0x7F   # NaN code: row 5
    codes[200, 300] = 0xFF  # NaN code: row 200
    scales[2, 1] = float("nan")  # rows 256..383 (every k block 1 column)
    announce(f"fp8 NaN code and scale M={M} N={N}")
    y32, _ = run(x, codes, scales, bf16=False)
    ref, A = orc().projection_fp8(bits(x), host(codes), host(scales))
    nan_rows = {5, 200} | set(range(256, min(N, 384)))
    got_nan = {n for n in range(N) if torch.isnan(y32[:, n]).all()}
    assert got_nan == nan_rows, sorted(got_nan ^ nan_rows)
    assert set(np.where(np.isnan(ref).all(axis=0))[0].tolist()) == nan_rows
    keep = torch.as_tensor([n for n in range(N) if n not in nan_rows], device=DEV)
    kh = keep.cpu().numpy()
    check_f32(y32[:, keep], ref[:, kh], A[:, kh], "fp8 rows without NaN")


def test_fp8_rejections_touch_nothing():
    x65 = si.normal_bf16((65, 64), 1.0, 1, DEV)
    codes, scales = si.fp8_weights(8, 64, 2, DEV)
    y = torch.full((65, 8), -7.0, device=DEV)
    with pytest.raises(sg.SkinnyGemmError) as e:
        sg.skinny_gemm_fp8(x65, codes, scales, y_f32=y)  # M > 64
    assert e.value.status == 3
    # chunk kernel: a workspace shorter than the split-K partials need
    x20 = si.normal_bf16((20, 4096), 1.0, 6, DEV)
    c20, s20 = si.fp8_weights(4096, 4096, 7, DEV)
    y20 = torch.full((20, 4096), -7.0, device=DEV)
    need = sg.skinny_gemm_fp8_workspace(20, 4096, 4096)
    assert need > 0
    before = sg.skinny_gemm_get_counters()
    with pytest.raises(sg.SkinnyGemmError) as e:
        sg.skinny_gemm_fp8(x20, c20, s20, y_f32=y20,
                           workspace=torch.empty(need - 256, dtype=torch.uint8, device=DEV))
    assert e.value.status == 5
    assert counters_delta(before, sg.skinny_gemm_get_counters()) == [0] * sg.SG_NUM_COUNTERS
    x = si.normal_bf16((4, 16400), 1.0, 3, DEV)
    c2, s2 = si.fp8_weights(8, 16400, 4, DEV)
    y4 = torch.full((4, 8), -7.0, device=DEV)
    with pytest.raises(sg.SkinnyGemmError) as e:
        sg.skinny_gemm_fp8(x, c2, s2, y_f32=y4)  # K > 16384 at M = 4
    assert e.value.status == 3
    x2 = si.normal_bf16((2, 16400), 1.0, 5, DEV)
    y2 = torch.full((2, 8), -7.0, device=DEV)
    with pytest.raises(sg.SkinnyGemmError) as e:
        sg.skinny_gemm_fp8(x2, c2, s2, y_f32=y2)  # M * K > 32768 at M = 2
    assert e.value.status == 3
    st = sg._c().skinny_gemm_fp8(1, 8, 24, x.data_ptr(), c2.data_ptr(), s2.data_ptr(), None,
                                 y4.data_ptr(), None, None, 0, None)  # K % 16
    assert st == 4
    torch.cuda.synchronize()
    assert (y == -7.0).all() and (y4 == -7.0).all() and (y2 == -7.0).all(), \
        "rejected calls write nothing"
    assert (y20 == -7.0).all(), "rejected calls write nothing"


@pytest.mark.parametrize("M", [1, 20])
def test_fp8_empty(M):
    x = si.normal_bf16((M, 0), 1.0, 5, DEV)
    codes = torch.empty((10, 0), dtype=torch.uint8, device=DEV)
    scales = torch.empty((1, 0), dtype=torch.float32, device=DEV)
    y32, _ = run(x, codes, scales, bf16=False)
    assert (y32 == 0).all(), "K = 0: zero sums"
    r = si.normal_bf16((M, 10), 1.0, 6, DEV)
    out = torch.full((M, 10), -7.0, device=DEV)
    sg.skinny_gemm_fp8(x, codes, scales, y_f32=out, r=r)
    torch.cuda.synchronize()
    assert torch.equal(out, r.float()), "K = 0 with a residual: out = r"


@pytest.mark.parametrize("M,N,K,residual", [(1, 8192, 7168, False), (2, 8192, 7168, False),
                                            (4, 4096, 7168, False), (8, 4096, 7168, False),
                                            (16, 4096, 7168, False), (12, 8192, 7168, False),
                                            (32, 4096, 7168, False), (64, 4096, 7168, False),
                                            (64, 8192, 7168, False),
                                            (1, 7168, 8192, True),
                                            (8, 7168, 8192, True), (16, 7168, 8192, True),
                                            (64, 7168, 8192, True)])
def test_fp8_full_size_sampled(M, N, K, residual):
    announce(f"fp8 full M={M} N={N} K={K} residual={residual}")
    x = si.normal_bf16((M, K), 1.0, 9000 + M, DEV)
    codes, scales = si.fp8_weights(N, K, 9100 + N, DEV)
    r = si.normal_bf16((M, N), 1.0, 9200 + M, DEV) if residual else None
    y32, y16 = run(x, codes, scales, r=r)
    c, s, xb = host(codes), host(scales), bits(x)
    for n in sample_rows(N, 48, 9300 + M):
        ref, A = orc().projection_fp8(xb, c[n:n + 1], s[n // 128:n // 128 + 1])
        if residual:
            ref = ref + orc().bf16_to_f64(bits(r[:, n:n + 1])).reshape(M, 1)
        check_f32(y32[:, n:n + 1], ref, A, f"fp8 full row {n}", extra=2.0 ** -23 * np.abs(ref))
        check_bf16(y16[:, n:n + 1], ref, A, f"fp8 full row {n} bf16")
