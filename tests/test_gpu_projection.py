"""GPU parity of the projection paths through the C ABI: small-matrix kernel
(M <= 2), VALU split-K (the planner's choice for 3 <= M <= 7; forced up to
M = 15), bf16 matrix-core split-K (the planner's choice from M = 8, from M = 6
where its workgroups fill the GPU; the in-workgroup team kernel and the chunk
kernel with its reduction), the deterministic reduction and the fused
residual epilogue.

Every output is compared element by element with the fp64 oracle on the same
seeded bf16 inputs: exhaustively at sizes that span several tiles and a
ragged tail, and at the full workload sizes on the plan the planner picks
(the plan the benchmark times) -- every output there too -- and on sampled
rows for the forced split sweep.  Integer-valued inputs make every sum exact, so there all
kernels, splits and output types must match the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import seeded_inputs as si
import skinny_gemm_projection_amd as sg
from gpu_common import (DEV, announce, bits, check_bf16, check_exact, check_f32, counters_delta,
                        orc, projection_all_rows, sample_rows, to_np)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

G, V, F = sg.SG_KERNEL_GEMV, sg.SG_KERNEL_SPLITK_VALU, sg.SG_KERNEL_SPLITK_MFMA


def make(M, N, K, seed, sx=1.0, sw=0.02):
    x = si.normal_bf16((M, K), sx, seed + si.TAG_X, DEV)
    W = si.normal_bf16((N, K), sw, seed + si.TAG_W, DEV)
    return x, W


def run(plan, x, W, r=None, f32=True, bf16=True, inplace=False):
    M, N = plan.M, plan.N
    y32 = torch.full((M, N), float("nan"), device=DEV) if f32 else None
    y16 = None
    if bf16:
        y16 = r if inplace else torch.full((M, N), float("nan"), device=DEV, dtype=torch.bfloat16)
    if r is None:
        ws = sg.skinny_gemm(plan, x, W, y_f32=y32, y_bf16=y16)
    else:
        ws = sg.skinny_gemm_residual(plan, x, W, r, out_bf16=y16, out_f32=y32)
    torch.cuda.synchronize()
    return y32, y16, ws


def oracle_rows(x, W, rows=None):
    """Oracle y and A for all M rows of x against the chosen rows of W (every row of W
    when rows is None, split over host threads)."""
    Wb = bits(W)
    if rows is None:
        return projection_all_rows(bits(x), Wb)
    return orc().projection(bits(x), Wb[rows])


def plan_or_skip(M, N, K, kernel, S, two_pass=-1, tile_n=0):
    try:
        return sg.skinny_gemm_plan_force(M, N, K, kernel, S, two_pass, tile_n)
    except sg.SkinnyGemmError as e:
        assert e.status == 6
        pytest.skip(f"plan rejects kernel {kernel} with S={S} at M={M}, K={K}")


# ------------------------------------------------------------------ small exhaustive shapes

SMALL = [
    # (M, N, K): ragged N (not a multiple of the 64-row tile) and ragged K (not of 512 / 256)
    (1, 1000, 1032), (2, 777, 520), (1, 33, 8), (2, 5, 7168), (1, 1024, 1024),
    (3, 1000, 1032), (4, 513, 2056), (5, 1000, 1032), (8, 300, 4104), (9, 1000, 1032),
    (15, 257, 1032), (16, 1000, 1056), (17, 130, 520), (31, 1000, 1056), (32, 65, 2056),
    (48, 1000, 1056), (63, 200, 264), (64, 1000, 1056),
    # wide matrices: the team kernel with two 16-row tiles a wave (ragged last pair)
    (9, 8161, 520), (12, 8200, 1040), (16, 8177, 264), (13, 9000, 2056),
    # ... with every round unrolled (K <= 8192), from 3 rows where N/16 >= 160
    (7, 8300, 8192), (8, 8161, 7168), (3, 4097, 2056), (5, 4200, 6152), (4, 6000, 8192),
    # the streaming vector-ALU kernel with teams (N/16 < 160): M = 3, 4, 2 to 8 rows a team
    (3, 2101, 4104), (4, 2400, 4104), (4, 2200, 8192), (4, 2544, 7168),
    # the team kernel from 160 workgroups (N/16 >= 160)
    (4, 4000, 4104), (4, 3500, 8192), (4, 3000, 7168), (8, 2560, 7168), (16, 3584, 7168),
    # the chunk kernel with every round unrolled (one x phase), short last chunks:
    # 5 and 8 rounds of 128-row tiles, 16 rounds of 256-row tiles
    (20, 1000, 7000), (24, 4500, 6984), (48, 700, 8192), (40, 9000, 7000),
]


@pytest.mark.parametrize("M,N,K", SMALL, ids=lambda v: str(v))
def test_small_shapes_auto_plan(M, N, K):
    announce(f"small auto M={M} N={N} K={K}")
    x, W = make(M, N, K, 7000 + M)
    plan = sg.skinny_gemm_plan(M, N, K)
    before = sg.skinny_gemm_get_counters()
    y32, y16, _ = run(plan, x, W)
    d = counters_delta(before, sg.skinny_gemm_get_counters())
    assert d[plan.kernel] == 1, f"planned kernel must run: {d}"
    assert d[sg.SG_KERNEL_REDUCE] == (1 if plan.two_pass else 0)
    y, A = oracle_rows(x, W)
    check_f32(y32, y, A, f"fp32 M={M} N={N} K={K} {plan}")
    check_bf16(y16, y, A, f"bf16 M={M} N={N} K={K}")


def _accepted(M, N, K, kernel, S, two_pass=-1, tile_n=0):
    """The planner takes this forced plan (host-only call).  Combinations it rejects
    (a split that leaves an empty chunk, a team split it has no kernel for) are
    covered by the plan tests of the CPU suite, so they are not generated here."""
    try:
        sg.skinny_gemm_plan_force(M, N, K, kernel, S, two_pass, tile_n)
        return True
    except sg.SkinnyGemmError:
        return False


VALU_FORCED = [(M, S, tp) for M in (1, 2, 3, 4, 5, 7, 8, 9, 12, 15) for S in (1, 2, 3, 4, 8, 16)
               for tp in (0, 1) if _accepted(M, 300, 2112, V, S, tp)]


@pytest.mark.parametrize("M,S,two_pass", VALU_FORCED)
def test_valu_forced_splits(M, S, two_pass):
    N, K = 300, 2112  # 264 pieces of 8: chunk widths 2112, 1088, 704, 576, 320, 192 (ragged)
    plan = plan_or_skip(M, N, K, V, S, two_pass)
    announce(f"valu forced M={M} S={S} two_pass={two_pass}")
    x, W = make(M, N, K, 7100 + M)
    y32, _, _ = run(plan, x, W, bf16=False)
    y, A = oracle_rows(x, W)
    check_f32(y32, y, A, f"VALU M={M} S={S} two_pass={two_pass}")


MFMA_FORCED = [(M, S, tile) for M in (1, 4, 16, 17, 33, 48, 64) for S in (1, 2, 3, 4, 8)
               for tile in (16, 128, 256)
               if _accepted(M, 200, 2112, F, S, 0 if tile == 16 else 1, tile)]


@pytest.mark.parametrize("M,S,tile", MFMA_FORCED)
def test_mfma_forced_splits(M, S, tile):
    # N = 200: one ragged 128- or 256-row tile; K = 2112 = 264 pieces: ragged rounds
    N, K = 200, 2112
    plan = plan_or_skip(M, N, K, F, S, 0 if tile == 16 else 1, tile)
    announce(f"mfma forced M={M} S={S} tile={tile}")
    x, W = make(M, N, K, 7200 + M)
    y32, y16, _ = run(plan, x, W)
    y, A = oracle_rows(x, W)
    check_f32(y32, y, A, f"MFMA M={M} S={S}")
    check_bf16(y16, y, A, f"MFMA bf16 M={M} S={S}")


# ------------------------------------------------------------------ integer inputs: bit-exact


@pytest.mark.parametrize("kernel,M,S,tp", [(G, 1, 1, 0), (G, 2, 1, 0), (G, 2, 2, 0), (G, 2, 2, 1),
                                           (V, 3, 2, 0), (V, 4, 2, 1), (V, 8, 4, 0), (V, 8, 4, 1),
                                           (V, 15, 8, 0), (V, 15, 8, 1), (V, 11, 16, 1),
                                           (F, 16, 1, 0), (F, 16, 4, 1), (F, 16, 8, 0),
                                           (F, 64, 2, 1), (F, 64, 8, 0), (F, 64, 16, 1),
                                           (F, 5, 2, 1), (F, 37, 4, 0), (F, 64, 9, 256),
                                           (F, 20, 16, 256), (F, 8, 8, 128)])
def test_integer_inputs_bit_exact(kernel, M, S, tp):
    # tp: 0 / 1 in-kernel / second-pass reduction, or 128 / 256 the chunk kernel's tile
    N, K = 520, 8192  # |sums| <= 16 * 8192 < 2^24: every fp32 partial is exact
    plan = (plan_or_skip(M, N, K, kernel, S, 1, tp) if tp >= 128
            else plan_or_skip(M, N, K, kernel, S, tp))
    announce(f"integer bit-exact kernel={kernel} M={M} S={S}")
    x = si.integer_bf16((M, K), -4, 4, 8000 + M, DEV)
    W = si.integer_bf16((N, K), -4, 4, 8001 + M, DEV)
    r = si.integer_bf16((M, N), -4, 4, 8002 + M, DEV)
    y32, y16, ws = run(plan, x, W)
    y, _ = oracle_rows(x, W)
    check_exact(y32, y, f"fp32 kernel={kernel} M={M} S={S}")
    assert np.array_equal(bits(y16), orc().encode_bf16(y)), "bf16 output bit-exact"
    if plan.two_pass:  # the fp32 partials in the workspace equal the oracle's chunk sums
        if plan.kernel == F and plan.tile_n >= 128:
            # chunk kernel: [S, N, Mp] with M padded to whole 16-row tiles, padding rows zero
            Mp = 16 * -(-M // 16)
            P = ws[: S * N * Mp * 4].view(torch.float32).reshape(S, N, Mp)
            assert not P[:, :, M:].any(), "padding rows of the partials are zero"
            P = P[:, :, :M].transpose(1, 2).contiguous()
        else:
            P = ws[: S * M * N * 4].view(torch.float32).reshape(S, M, N)
        check_exact(P, orc().splitk_partials(bits(x), bits(W), S), "split-K partials")
    o32, o16, _ = run(plan, x, W, r=r)
    ref = orc().residual(bits(r), y)
    check_exact(o32, ref, "residual fp32")
    assert np.array_equal(bits(o16), orc().encode_bf16(ref)), "residual bf16 bit-exact"


# ------------------------------------------------------------------ full workload sizes


def _full_case(M, N, K, seed, kernel=None, S=0, rows=256, residual=False, inplace=False, tp=-1,
               tile=0):
    x, W = make(M, N, K, seed)
    r = si.normal_bf16((M, N), 1.0, seed + si.TAG_R, DEV) if residual else None
    r_before = r.clone() if r is not None else None
    plan = (sg.skinny_gemm_plan(M, N, K) if kernel is None
            else plan_or_skip(M, N, K, kernel, S, tp, tile))
    announce(f"full M={M} N={N} K={K} plan={plan} residual={residual} inplace={inplace}")
    y32, y16, _ = run(plan, x, W, r=r, inplace=inplace)
    sel = np.arange(N) if rows is None else sample_rows(N, rows, seed)
    y, A = oracle_rows(x, W, None if rows is None else sel)
    if residual:
        ref = orc().residual(bits(r_before)[:, sel], y)
        check_f32(y32[:, sel], ref, A, f"residual fp32 {plan}", extra=2.0 ** -23 * np.abs(ref))
        check_bf16(y16[:, sel], ref, A, f"residual bf16 {plan}")
    else:
        check_f32(y32[:, sel], y, A, f"fp32 {plan}")
        check_bf16(y16[:, sel], y, A, f"bf16 {plan}")
    return plan


def test_full_single_projection_1024():
    # M=1, K=N=1024, x and W ~ N(0, 0.02^2): every output checked
    x = si.normal_bf16((1, 1024), 0.02, 1000 + si.TAG_X, DEV)
    W = si.normal_bf16((1024, 1024), 0.02, 1000 + si.TAG_W, DEV)
    plan = sg.skinny_gemm_plan(1, 1024, 1024)
    assert plan.kernel == G
    announce(f"full 1x1024x1024 {plan}")
    y32, _, _ = run(plan, x, W, bf16=False)
    y, A = oracle_rows(x, W)
    check_f32(y32, y, A, "M=1 K=N=1024")


@pytest.mark.parametrize("M", [1, 2])
def test_full_small_batch_7168x8192(M):
    plan = _full_case(M, 8192, 7168, 2000, rows=None)
    assert plan.kernel == G and plan.split_k == 1


@pytest.mark.parametrize("M", [4, 8, 16])
def test_full_larger_batch_8192x7168(M):
    # every output of the bench's wider-matrix rows (the team kernel with one 16-row
    # tile a wave at M = 4 and 8, two at M = 16)
    plan = _full_case(M, 8192, 7168, 2500, rows=None)
    assert plan.split_k > 1


@pytest.mark.parametrize("M", [3, 4, 8, 12, 16, 32, 64])
def test_full_splitk_sweep_auto(M):
    plan = _full_case(M, 4096, 7168, 3000, rows=None)
    assert plan.split_k > 1


@pytest.mark.parametrize("M", [4, 8, 16, 32, 64])
@pytest.mark.parametrize("S", [2, 4, 8, 16])
@pytest.mark.parametrize("tp", [-1, 1])
def test_full_splitk_sweep_forced(M, S, tp):
    kernel = V if M < 8 else F
    _full_case(M, 4096, 7168, 3000, kernel=kernel, S=S, rows=128, tp=tp)


@pytest.mark.parametrize("M,S", [(8, 8), (16, 16), (64, 16), (64, 9)])
def test_full_mfma_32_rows_per_wave(M, S):
    plan = _full_case(M, 4096, 7168, 3100, kernel=F, S=S, rows=128, tp=1, tile=256)
    assert plan.tile_n == 256


@pytest.mark.parametrize("M", [1, 8, 64])
@pytest.mark.parametrize("inplace", [False, True])
def test_full_residual_8192x7168(M, inplace):
    _full_case(M, 7168, 8192, 4000, residual=True, inplace=inplace, rows=None)


# ------------------------------------------------------------------ properties and edge cases


@pytest.mark.parametrize("M,kernel,S,tp", [(1, G, 1, 0), (8, V, 4, 0), (8, V, 4, 1), (12, V, 8, 0),
                                           (64, F, 8, 1), (64, F, 8, 0)])
def test_repeat_runs_are_bitwise_identical(M, kernel, S, tp):
    N, K = 4096, 7168
    plan = plan_or_skip(M, N, K, kernel, S, tp)
    announce(f"determinism M={M} {plan}")
    x, W = make(M, N, K, 5000 + M)
    a32, a16, _ = run(plan, x, W)
    b32, b16, _ = run(plan, x, W)
    assert torch.equal(a32, b32) and torch.equal(a16, b16)


def test_rows_are_independent():
    # the first 4 rows of an M=64 run equal an M=4 run (different kernels) within tolerance,
    # and permuting x's rows permutes y's rows exactly (same kernel, same plan)
    N, K = 1000, 2056
    x, W = make(64, N, K, 5100)
    announce("row independence")
    y64, _, _ = run(sg.skinny_gemm_plan(64, N, K), x, W, bf16=False)
    y4, _, _ = run(sg.skinny_gemm_plan(4, N, K), x[:4].contiguous(), W, bf16=False)
    y, A = oracle_rows(x[:4], W)
    check_f32(y64[:4], y, A, "M=64 prefix")
    check_f32(y4, y, A, "M=4")
    perm = torch.randperm(64, generator=torch.Generator().manual_seed(1)).to(DEV)
    yp, _, _ = run(sg.skinny_gemm_plan(64, N, K), x[perm].contiguous(), W, bf16=False)
    assert torch.equal(yp, y64[perm])


@pytest.mark.parametrize("M", [1, 5, 20])
def test_zero_k_gives_zero_or_residual(M):
    N = 100
    plan = sg.skinny_gemm_plan(M, N, 0)
    announce(f"K=0 M={M} {plan}")
    x = torch.empty((M, 0), dtype=torch.bfloat16, device=DEV)
    W = torch.empty((N, 0), dtype=torch.bfloat16, device=DEV)
    y32, _, _ = run(plan, x, W, bf16=False)
    assert torch.equal(y32, torch.zeros_like(y32))
    r = si.normal_bf16((M, N), 1.0, 5200, DEV)
    _, o16, _ = run(plan, x, W, r=r, f32=False)
    assert torch.equal(o16, r)


def test_zero_weights_pass_residual_through():
    M, N, K = 8, 1000, 1032
    x, _ = make(M, N, K, 5300)
    W = torch.zeros((N, K), dtype=torch.bfloat16, device=DEV)
    r = si.normal_bf16((M, N), 1.0, 5301, DEV)
    for plan in (sg.skinny_gemm_plan(M, N, K), sg.skinny_gemm_plan_force(M, N, K, F, 3),
                 sg.skinny_gemm_plan_force(M, N, K, V, 4, 1)):
        announce(f"zero W residual {plan}")
        o32, o16, _ = run(plan, x, W, r=r)
        assert torch.equal(o16, r)
        assert torch.equal(o32, r.float())


def test_nan_propagates_to_its_row_only():
    M, N, K = 3, 200, 1032
    x, W = make(M, N, K, 5400)
    x[1, 17] = float("nan")
    plan = sg.skinny_gemm_plan(M, N, K)
    announce("nan propagation")
    y32, _, _ = run(plan, x, W, bf16=False)
    assert torch.isnan(y32[1]).all()
    assert torch.isfinite(y32[0]).all() and torch.isfinite(y32[2]).all()


def test_rejected_calls_on_device_buffers():
    M, N, K = 8, 256, 4096
    x, W = make(M, N, K, 5500)
    plan = sg.skinny_gemm_plan_force(M, N, K, V, 2, 1)
    assert plan.workspace_bytes > 16
    y = torch.empty((M, N), device=DEV)
    announce("rejections with device buffers")
    sg.skinny_gemm_reset_counters()
    flat = torch.empty(M * K + 8, dtype=torch.bfloat16, device=DEV)
    shifted = flat[4:4 + M * K].view(M, K)  # 8-byte offset: not 16-byte aligned
    with pytest.raises(sg.SkinnyGemmError) as e:
        sg.skinny_gemm(plan, shifted, W, y_f32=y)
    assert e.value.status == 4
    with pytest.raises(sg.SkinnyGemmError) as e:
        sg.skinny_gemm(plan, x, W, y_f32=y, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert e.value.status == 5
    assert sum(sg.skinny_gemm_get_counters()) == 0
    # a plan whose shape disagrees with the tensors is refused by the binding before the
    # library is called (the C ABI cannot see buffer sizes)
    with pytest.raises(ValueError):
        sg.skinny_gemm(sg.skinny_gemm_plan(M, N + 64, K), x, W, y_f32=y)
    with pytest.raises(ValueError):
        sg.skinny_gemm(plan, x, W, y_f32=torch.empty((M, N - 1), device=DEV))
    with pytest.raises(ValueError):
        sg.skinny_gemm_residual(plan, x, W, torch.empty((M + 1, N), dtype=torch.bfloat16, device=DEV),
                                out_f32=y)
    assert sum(sg.skinny_gemm_get_counters()) == 0
