"""GPU parity of the projection with MXFP4 weights (skinny_gemm_mxfp4) through the
C ABI, M = 1..64 (vector ALU, matrix cores, and from 17 rows -- 12 where N > 5888 --
the chunk kernel with its split-K reduction), against oracle_projection_mxfp4 on the same seeded codes and scales:
fp32 |got - ref| <= 1e-3 * A, bf16 adds 2^-8 |ref|, the residual adds 2^-23 |r + y|;
integer-valued activations with unit scales are bit-exact (every product is a
multiple of 1/2 and every partial sum exact in fp32)."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
import skinny_gemm_projection_amd as sg
from gpu_common import (DEV, announce, bits, check_bf16, check_exact, check_f32, counters_delta,
                        orc, sample_rows)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def np_u8(t):
    return t.cpu().numpy()


def run(x, codes, scales, r=None, f32=True, bf16=True):
    M, N = x.shape[0], codes.shape[0]
    y32 = torch.full((M, N), -7.0, device=DEV) if f32 else None
    y16 = torch.full((M, N), -7.0, device=DEV, dtype=torch.bfloat16) if bf16 else None
    before = sg.skinny_gemm_get_counters()
    sg.skinny_gemm_mxfp4(x, codes, scales, y_f32=y32, y_bf16=y16, r=r)
    torch.cuda.synchronize()
    d = counters_delta(before, sg.skinny_gemm_get_counters())
    assert d[sg.SG_KERNEL_MXFP4] == (1 if M > 0 and N > 0 else 0)
    # the chunk kernel adds the reduction when it splits K (the only case with a workspace)
    splits = sg.skinny_gemm_mxfp4_workspace(M, N, x.shape[1]) > 0
    assert d[sg.SG_KERNEL_REDUCE] == (1 if splits and N > 0 else 0)
    return y32, y16


SHAPES = [(1, 40, 32), (1, 129, 96), (1, 77, 608), (1, 65, 2080), (1, 33, 8224),
          (2, 50, 4128), (2, 17, 8192), (3, 70, 2080), (4, 96, 4160), (5, 31, 640),
          (6, 64, 7168), (7, 45, 2048), (8, 130, 3200), (8, 20, 16384), (9, 40, 2080),
          (12, 33, 608), (13, 70, 8224), (16, 100, 7168), (16, 17, 96), (16, 16, 32),
          # from 8161 rows the matrix-core kernel takes two 16-row tiles a wave
          # (ragged last 32-row tile)
          (9, 8200, 2080), (11, 8192, 608), (10, 8177, 96),
          # 12 to 16 rows: the matrix-core kernel up to N = 5888, the chunk kernel
          # (256-row tiles) above
          (13, 5888, 640), (13, 5889, 640), (16, 8192, 608), (12, 8177, 96),
          # from 17 rows the chunk kernel: x rows padded to 32, 48, 64, ragged
          # 128-row tiles and windows, one split and several, 256-row tiles
          (17, 200, 1056), (20, 129, 7168), (32, 300, 4128), (33, 64, 32), (47, 257, 2080),
          (48, 1000, 8192), (64, 33, 30016), (64, 8200, 1056), (17, 6300, 4096)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_mxfp4_small(M, N, K):
    announce(f"mxfp4 M={M} N={N} K={K}")
    x = si.normal_bf16((M, K), 1.0, 8000 + K + M, DEV)
    codes, scales = si.mxfp4_weights(N, K, 8100 + N + K, DEV)
    y32, y16 = run(x, codes, scales)
    ref, A = orc().projection_mxfp4(bits(x), np_u8(codes), np_u8(scales))
    check_f32(y32, ref, A, f"mxfp4 fp32 M={M} N={N} K={K}")
    check_bf16(y16, ref, A, f"mxfp4 bf16 M={M} N={N} K={K}")
    # residual epilogue, in place on the bf16 output
    r = si.normal_bf16((M, N), 1.0, 8200 + N, DEV)
    out = r.clone()
    sg.skinny_gemm_mxfp4(x, codes, scales, y_bf16=out, r=out)
    torch.cuda.synchronize()
    rr = orc().bf16_to_f64(bits(r)).reshape(M, N)
    check_bf16(out, rr + ref, A, f"mxfp4 residual M={M} N={N} K={K}")
    y32b, _ = run(x, codes, scales, bf16=False)
    assert torch.equal(y32, y32b), "repeat runs bitwise identical"


@pytest.mark.parametrize("M,N,K", [(1, 37, 4096), (2, 64, 7168), (8, 40, 8192), (5, 19, 96),
                                   (16, 48, 4096), (11, 21, 8192), (16, 8200, 1024),
                                   (17, 300, 8192), (40, 129, 4128), (64, 8200, 2080)])
def test_mxfp4_integer_bit_exact(M, N, K):
    announce(f"mxfp4 integer M={M} N={N} K={K}")
    x = si.integer_bf16((M, K), -4, 4, 8300 + K, DEV)
    codes = si.random_bytes((N, K // 2), 0, 255, 8301 + N, DEV)
    scales = torch.full((N, K // 32), 127, dtype=torch.uint8, device=DEV)  # unit scales
    y32, y16 = run(x, codes, scales)
    ref = orc().projection_mxfp4(bits(x), np_u8(codes), np_u8(scales), with_scale=False)
    check_exact(y32, ref, f"mxfp4 integer M={M}")
    check_exact(y16.float(), orc().bf16_to_f64(orc().encode_bf16(ref)).reshape(M, N),
                f"mxfp4 integer bf16 M={M}")


@pytest.mark.parametrize("M,N", [(3, 24), (12, 24), (12, 8200), (20, 300), (64, 8200)])
def test_mxfp4_nan_scale_and_zero_codes(M, N):
    # vector kernel (M = 3), matrix-core kernel with one and with two row tiles a wave
    announce(f"mxfp4 NaN scale, zero codes M={M} N={N}")
    K = 512
    x = si.normal_bf16((M, K), 1.0, 8400 + M, DEV)
    codes, scales = si.mxfp4_weights(N, K, 8401, DEV)
    scales[5, 3] = 255      # NaN block: row 5 is NaN for every m
    scales[N - 5, 0] = 255  # and row N - 5 (the second row tile of the last pair at N = 8200)
    scales[7, :] = 200      # large scale, 2^73 (finite fp32 sums for these x)
    codes[11, :] = 0        # all +0 codes
    codes[12, :] = 0x88     # all -0 codes
    y32, _ = run(x, codes, scales, bf16=False)
    ref, A = orc().projection_mxfp4(bits(x), np_u8(codes), np_u8(scales))
    y = y32.cpu().numpy()
    nan_rows = [5, N - 5]
    assert np.isnan(y[:, nan_rows]).all() and not np.isnan(np.delete(y, nan_rows, axis=1)).any()
    keep = [n for n in range(N) if n not in nan_rows]
    check_f32(y32[:, keep], ref[:, keep], A[:, keep], "mxfp4 NaN/zero rows")
    assert (y[:, 11] == 0).all() and (y[:, 12] == 0).all()


# Every scale code 0..254 is a valid OCP e8m0 scale (2^-127 .. 2^127).  The
# kernels scale each block's fp32 sum, formed at unit scale (the chunk kernel
# for codes outside [64, 190]), so the products stay exact down to
# code 0 (whose weights are below bf16's and fp32's normal range) and up to
# code 254 (whose weights can exceed the largest bf16).
@pytest.mark.parametrize("M,N", [(3, 40), (8, 40), (12, 40), (16, 40), (12, 8200), (16, 8192),
                                 (24, 40), (64, 8192)])
def test_mxfp4_scale_code_range(M, N):
    # vector kernel (M = 3, 8), matrix-core kernel with one (N = 40) and two
    # (N >= 8161) row tiles a wave, chunk kernel (M = 24, 64)
    announce(f"mxfp4 scale codes 0..12, 120, 253, 254, mixed M={M} N={N}")
    K = 640  # 20 blocks: 5 windows of the matrix-core kernel
    KB = K // 32
    codes, scales = si.mxfp4_weights(N, K, 8450 + N, DEV)
    # low codes with x ~ N(0, 1): sums around 2^-120, some block sums subnormal
    low = scales.clone()
    for c in range(13):
        low[c, :] = c                       # rows 0..12: scale code c on every block
    low[13, :] = 120
    low[14, :] = torch.tensor([0, 140] * (KB // 2), dtype=torch.uint8)    # 2^-127 and 2^13
    low[15, :] = torch.tensor([(7 * b) % 41 + 100 for b in range(KB)], dtype=torch.uint8)
    low[N - 1, :] = 1                      # the last row tile too
    low[N - 17, :] = 0
    x = si.normal_bf16((M, K), 1.0, 8460 + M, DEV)
    y32, _ = run(x, codes, low, bf16=False)
    ref, A = orc().projection_mxfp4(bits(x), np_u8(codes), np_u8(low))
    check_f32(y32, ref, A, f"mxfp4 low scale codes M={M} N={N}")
    assert (A[:, 0] > 0).all() and (np.abs(ref[:, 0]) < 2.0 ** -110).all()
    # high codes with tiny x (2^-40 N(0, 1)): weights up to 6 * 2^127, above
    # bf16's largest value, sums finite in fp32
    high = scales.clone()
    high[0, :] = 254
    high[1, :] = 253
    high[2, :] = 120
    high[3, :] = torch.tensor([254, 200] * (KB // 2), dtype=torch.uint8)
    high[N - 1, :] = 254
    xs = si.normal_bf16((M, K), 2.0 ** -40, 8470 + M, DEV)
    y32, _ = run(xs, codes, high, bf16=False)
    ref, A = orc().projection_mxfp4(bits(xs), np_u8(codes), np_u8(high))
    assert np.isfinite(ref).all() and np.abs(ref[:, 0]).max() > 2.0 ** 80
    check_f32(y32, ref, A, f"mxfp4 high scale codes M={M} N={N}")


# The chunk kernel (from 12 rows) takes a window on the matrix cores at its
# blocks' scales when every scale code of the window's rows lies in [64, 190],
# else at unit scale with each block's sum scaled after: one wave switching
# between the two inside its K range, and tiles at the range's two ends (the
# other kernels, scaling every block's sum, run the same inputs).
@pytest.mark.parametrize("M,N", [(3, 40), (12, 40), (16, 40), (12, 8200), (16, 8192), (24, 40),
                                 (64, 8192)])
def test_mxfp4_scale_window_mix(M, N):
    announce(f"mxfp4 scale windows mixed M={M} N={N}")
    K = 640
    KB = K // 32
    codes, scales = si.mxfp4_weights(N, K, 8480 + N, DEV)
    assert int(scales.min()) >= 64 and int(scales.max()) <= 190
    scales[1, 9] = 1                        # window 2 of the first tile at unit scale
    scales[20, 0] = 200                     # the first and last windows of the second tile
    scales[20, KB - 1] = 63
    scales[32:40, :] = 64                   # the range's ends, every block
    if N > 48:
        scales[40:48, :] = 190
    x = si.normal_bf16((M, K), 1.0, 8490 + M, DEV)
    y32, _ = run(x, codes, scales, bf16=False)
    ref, A = orc().projection_mxfp4(bits(x), np_u8(codes), np_u8(scales))
    assert np.isfinite(ref).all()
    check_f32(y32, ref, A, f"mxfp4 scale windows mixed M={M} N={N}")


def test_mxfp4_empty_and_rejected():
    announce("mxfp4 empty and rejected sizes")
    x = si.normal_bf16((2, 64), 1.0, 1, DEV)
    codes, scales = si.mxfp4_weights(8, 64, 2, DEV)
    y = torch.full((2, 8), -7.0, device=DEV)
    # K = 0: y = 0
    sg.skinny_gemm_mxfp4(torch.empty((2, 0), dtype=torch.bfloat16, device=DEV),
                         torch.empty((8, 0), dtype=torch.uint8, device=DEV),
                         torch.empty((8, 0), dtype=torch.uint8, device=DEV), y_f32=y)
    torch.cuda.synchronize()
    assert (y == 0).all()
    lib = sg._c()
    y.fill_(-7.0)
    s = torch.cuda.current_stream().cuda_stream
    cases = [((65, 8, 64), 3),         # batch above the decode path
             ((2, 8, 48), 4),          # K not a multiple of 32
             ((1, 8, 32800), 3),       # K over the vector-ALU split limit at M = 1
             ((2, 8, 32800), 3),       # and at M = 2
             ((5, 8, 16416), 3),       # and from M = 3
             ((2, -1, 64), 2)]
    for (M, N, K), status in cases:
        before = sg.skinny_gemm_get_counters()
        st = lib.skinny_gemm_mxfp4(M, N, K, x.data_ptr(), codes.data_ptr(), scales.data_ptr(),
                                   None, y.data_ptr(), None, None, 0, s)
        assert st == status, ((M, N, K), st)
        assert counters_delta(before, sg.skinny_gemm_get_counters()) == [0] * sg.SG_NUM_COUNTERS
    torch.cuda.synchronize()
    assert (y == -7.0).all(), "a rejected call leaves the output alone"


@pytest.mark.parametrize("M,N,K", [(1, 8192, 7168), (2, 8192, 7168), (4, 4096, 7168),
                                   (8, 4096, 7168), (16, 4096, 7168), (16, 8192, 7168),
                                   (32, 4096, 7168), (64, 4096, 7168), (64, 8192, 7168),
                                   (1, 7168, 8192),
                                   (8, 7168, 8192), (16, 7168, 8192), (64, 7168, 8192)])
def test_mxfp4_full_size(M, N, K):
    # the benchmark's shapes: sampled output rows against the oracle
    announce(f"mxfp4 full M={M} N={N} K={K}")
    x = si.normal_bf16((M, K), 1.0, 8500 + M, DEV)
    codes, scales = si.mxfp4_weights(N, K, 8600 + N, DEV)
    y32, y16 = run(x, codes, scales)
    rows = sample_rows(N, 96, M + N)
    ref, A = orc().projection_mxfp4(bits(x), np_u8(codes)[rows], np_u8(scales)[rows])
    idx = torch.as_tensor(rows, device=DEV)
    check_f32(y32[:, idx], ref, A, f"mxfp4 full fp32 M={M}")
    check_bf16(y16[:, idx], ref, A, f"mxfp4 full bf16 M={M}")
