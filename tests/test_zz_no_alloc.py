"""skinny_gemm_noalloc (the entry point that allocates nothing: split-K partials in
the library's own per-GPU scratch array) through the C ABI, against skinny_gemm
with a caller workspace on the same plan and inputs.  The same kernels run, so
the outputs must be identical bit for bit; the skinny_gemm outputs are checked
against the fp64 oracle on sampled rows (fp32 |d| <= 1e-3 A, bf16 adds
2^-8 |ref|).  Two calls in a row, the second with a smaller input, exercise the
reuse of the scratch array."""
import ctypes

import pytest
import torch

import seeded_inputs as si
import skinny_gemm_projection_amd as sg
from gpu_common import DEV, announce, bits, check_bf16, check_f32, counters_delta, orc, sample_rows

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def noalloc(plan, x, W, y32, y16):
    return sg._c().skinny_gemm_noalloc(ctypes.byref(plan), x.data_ptr(), W.data_ptr(),
                                       y32.data_ptr() if y32 is not None else None,
                                       y16.data_ptr() if y16 is not None else None,
                                       torch.cuda.current_stream().cuda_stream)


def compare(plan, seed):
    M, N, K = plan.M, plan.N, plan.K
    x = si.normal_bf16((M, K), 1.0, seed, DEV)
    W = si.normal_bf16((N, K), 0.02, seed + 1, DEV)
    a32 = torch.full((M, N), float("nan"), device=DEV)
    a16 = torch.full((M, N), float("nan"), device=DEV, dtype=torch.bfloat16)
    sg.skinny_gemm(plan, x, W, y_f32=a32, y_bf16=a16)
    b32 = torch.full((M, N), float("nan"), device=DEV)
    b16 = torch.full((M, N), float("nan"), device=DEV, dtype=torch.bfloat16)
    before = sg.skinny_gemm_get_counters()
    assert noalloc(plan, x, W, b32, b16) == 0
    torch.cuda.synchronize()
    d = counters_delta(before, sg.skinny_gemm_get_counters())
    assert d[plan.kernel] == 1 and d[sg.SG_KERNEL_REDUCE] == (1 if plan.two_pass else 0)
    rows = sample_rows(N, 96, seed)
    ref, A = orc().projection(bits(x), bits(W)[rows])
    idx = torch.as_tensor(rows, device=DEV)
    check_f32(a32[:, idx], ref, A, f"skinny_gemm fp32 {plan}")
    check_bf16(a16[:, idx], ref, A, f"skinny_gemm bf16 {plan}")
    assert torch.equal(a32, b32), f"noalloc fp32 differs from skinny_gemm: {plan}"
    assert torch.equal(a16, b16), f"noalloc bf16 differs from skinny_gemm: {plan}"


@pytest.mark.parametrize("first,second", [
    # chunk kernel + reduction ([S, N, Mp] partials) at the split-K workload size, then smaller
    ((64, 4096, 7168, None), (20, 1000, 1056, None)),
    # vector-ALU two-pass ([S, M, N] partials), then a smaller one
    ((8, 4096, 7168, (2, 8, 1, 0)), (3, 700, 2112, (2, 4, 1, 0))),
    # a plan with no workspace (the small-matrix kernel), then a two-pass one
    ((2, 8192, 7168, None), (32, 520, 2056, None)),
])
def test_noalloc_matches_skinny_gemm(first, second):
    for i, (M, N, K, force) in enumerate((first, second)):
        plan = sg.skinny_gemm_plan(M, N, K) if force is None else \
            sg.skinny_gemm_plan_force(M, N, K, *force)
        assert plan.workspace_bytes <= sg.SG_NOALLOC_MAX_WORKSPACE
        announce(f"noalloc call {i}: {plan}")
        compare(plan, 52000 + 10 * M + i)


def test_noalloc_rejects_a_workspace_over_its_limit():
    M, N, K = 64, 65536, 1024
    plan = sg.skinny_gemm_plan_force(M, N, K, sg.SG_KERNEL_SPLITK_MFMA, 8, 1, 128)
    assert plan.workspace_bytes > sg.SG_NOALLOC_MAX_WORKSPACE
    announce(f"noalloc over the limit: {plan}")
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((N, K), dtype=torch.bfloat16, device=DEV)
    y = torch.full((M, N), -7.0, device=DEV)
    before = sg.skinny_gemm_get_counters()
    assert noalloc(plan, x, W, y, None) == 5  # SG_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert counters_delta(before, sg.skinny_gemm_get_counters()) == [0] * sg.SG_NUM_COUNTERS
    assert bool((y == -7.0).all()), "a rejected call leaves the output alone"
