"""GPU parity of the routed-expert path: per-expert token table (bit-exact)
and grouped projection (element-wise against the oracle), through the C ABI."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
import skinny_gemm_projection_amd as sg
from gpu_common import DEV, announce, bits, check_exact, check_f32, counters_delta, orc

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def run_grouped(x, W, ids):
    T, topk = ids.shape
    E, N, _ = W.shape
    out = torch.full((T, topk, N), float("nan"), device=DEV)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    pairs = torch.full((max(T * topk, 1),), -7, dtype=torch.int32, device=DEV)
    invalid = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    sg.grouped_skinny_gemm(x, W, ids.to(DEV), out, expert_offsets=offsets, sorted_pairs=pairs,
                           invalid_count=invalid)
    torch.cuda.synchronize()
    return out, offsets, pairs[: T * topk], invalid


def check_table(ids, E, offsets, pairs, invalid):
    counts, ref_off, ref_pairs, ref_inv = orc().moe_table(ids.numpy(), E)
    assert np.array_equal(offsets.cpu().numpy(), ref_off), "expert_offsets bit-exact"
    assert np.array_equal(pairs.cpu().numpy(), ref_pairs), "sorted_pairs bit-exact"
    assert int(invalid.item()) == ref_inv, "invalid_count exact"


@pytest.mark.parametrize("T,topk,E,N,K", [(1, 4, 24, 100, 1032), (5, 4, 24, 100, 1032),
                                          (16, 8, 40, 33, 520), (64, 8, 384, 20, 264),
                                          (3, 2, 7, 16, 8)])
def test_grouped_small_exhaustive(T, topk, E, N, K):
    announce(f"grouped small T={T} topk={topk} E={E} N={N} K={K}")
    x = si.normal_bf16((T, K), 1.0, 9000 + T, DEV)
    W = si.normal_bf16((E, N, K), 0.02, 9001 + T, DEV)
    ids = si.routing_table(T, E, topk, 9002 + T)
    before = sg.skinny_gemm_get_counters()
    out, off, pairs, inv = run_grouped(x, W, ids)
    d = counters_delta(before, sg.skinny_gemm_get_counters())
    assert d[sg.SG_KERNEL_MOE_TABLE] == 1 and d[sg.SG_KERNEL_GROUPED] == 1
    check_table(ids, E, off, pairs, inv)
    ref, A = orc().grouped(bits(x), bits(W), ids.numpy())
    check_f32(out, ref, A, f"grouped T={T}")


def test_grouped_integer_bit_exact_with_crowded_expert():
    # tokens crowd onto expert 3 (more than two tokens per expert: the token-pair loop),
    # duplicate ids inside a token, and ids outside [0, E)
    T, topk, E, N, K = 9, 3, 6, 40, 2056
    x = si.integer_bf16((T, K), -4, 4, 9100, DEV)
    W = si.integer_bf16((E, N, K), -4, 4, 9101, DEV)
    ids = torch.tensor([[3, 1, 3], [3, 0, 5], [3, 3, 3], [2, 3, -1], [3, 6, 4], [0, 1, 2],
                        [3, 1000, 3], [5, 4, 3], [3, 2, 1]], dtype=torch.int32)
    announce("grouped integer crowded/duplicate/invalid")
    out, off, pairs, inv = run_grouped(x, W, ids)
    check_table(ids, E, off, pairs, inv)
    assert int(inv.item()) == 3
    ref = orc().grouped(bits(x), bits(W), ids.numpy(), with_scale=False)
    check_exact(out, ref, "grouped integer")
    flat = ids.view(-1)
    for p in range(T * topk):
        if not 0 <= flat[p] < E:
            assert torch.equal(out.view(-1, N)[p], torch.zeros(N, device=DEV)), "invalid id: zero row"


def run_grouped_fused(x, W, ids):
    """The call without table outputs: the fused table + grouped launch (small tables)."""
    T, topk = ids.shape
    E, N, _ = W.shape
    out = torch.full((T, topk, N), float("nan"), device=DEV)
    before = sg.skinny_gemm_get_counters()
    sg.grouped_skinny_gemm(x, W, ids.to(DEV), out)
    torch.cuda.synchronize()
    return out, counters_delta(before, sg.skinny_gemm_get_counters())


@pytest.mark.parametrize("T,topk,E,N,K", [(1, 8, 384, 100, 1032), (5, 4, 24, 100, 1032),
                                          (16, 8, 40, 33, 520), (64, 8, 384, 20, 264),
                                          (3, 2, 7, 16, 8), (64, 8, 4096, 8, 64),
                                          (1, 1, 1, 5, 8)])
def test_grouped_fused_table(T, topk, E, N, K):
    # no table outputs asked for: one launch, each workgroup building its table in LDS;
    # outputs against the oracle and bit-identical to the table-kernel path
    announce(f"grouped fused T={T} topk={topk} E={E} N={N} K={K}")
    x = si.normal_bf16((T, K), 1.0, 9300 + T, DEV)
    W = si.normal_bf16((E, N, K), 0.02, 9301 + T, DEV)
    ids = si.routing_table(T, E, topk, 9302 + T)
    out, d = run_grouped_fused(x, W, ids)
    assert d[sg.SG_KERNEL_MOE_TABLE] == 0 and d[sg.SG_KERNEL_GROUPED] == 1
    ref, A = orc().grouped(bits(x), bits(W), ids.numpy())
    check_f32(out, ref, A, f"grouped fused T={T}")
    out_t = run_grouped(x, W, ids)[0]
    assert torch.equal(out, out_t), "fused and table paths give the same bits"


def test_grouped_fused_integer_crowded_duplicate_invalid():
    T, topk, E, N, K = 9, 3, 6, 40, 2056
    x = si.integer_bf16((T, K), -4, 4, 9400, DEV)
    W = si.integer_bf16((E, N, K), -4, 4, 9401, DEV)
    ids = torch.tensor([[3, 1, 3], [3, 0, 5], [3, 3, 3], [2, 3, -1], [3, 6, 4], [0, 1, 2],
                        [3, 1000, 3], [5, 4, 3], [3, 2, 1]], dtype=torch.int32)
    announce("grouped fused integer crowded/duplicate/invalid")
    out, d = run_grouped_fused(x, W, ids)
    assert d[sg.SG_KERNEL_MOE_TABLE] == 0
    ref = orc().grouped(bits(x), bits(W), ids.numpy(), with_scale=False)
    check_exact(out, ref, "grouped fused integer")
    flat = ids.view(-1)
    for p in range(T * topk):
        if not 0 <= flat[p] < E:
            assert torch.equal(out.view(-1, N)[p], torch.zeros(N, device=DEV)), "invalid id: zero row"


def test_grouped_large_table_keeps_table_kernel():
    # more than 512 pairs: the table kernel runs even without table outputs
    T, topk, E, N, K = 80, 8, 64, 24, 128
    x = si.normal_bf16((T, K), 1.0, 9500, DEV)
    W = si.normal_bf16((E, N, K), 0.02, 9501, DEV)
    ids = si.routing_table(T, E, topk, 9502)
    announce("grouped 640 pairs without table outputs")
    out, d = run_grouped_fused(x, W, ids)
    assert d[sg.SG_KERNEL_MOE_TABLE] == 1 and d[sg.SG_KERNEL_GROUPED] == 1
    ref, A = orc().grouped(bits(x), bits(W), ids.numpy())
    check_f32(out, ref, A, "grouped 640 pairs")


def test_grouped_no_tokens():
    E, N, K = 16, 32, 64
    x = torch.empty((0, K), dtype=torch.bfloat16, device=DEV)
    W = si.normal_bf16((E, N, K), 0.02, 9200, DEV)
    ids = torch.empty((0, 8), dtype=torch.int32)
    announce("grouped T=0")
    before = sg.skinny_gemm_get_counters()
    out, off, _, inv = run_grouped(x, W, ids)
    d = counters_delta(before, sg.skinny_gemm_get_counters())
    assert d[sg.SG_KERNEL_GROUPED] == 0
    assert torch.equal(off.cpu(), torch.zeros(E + 1, dtype=torch.int32)) and int(inv.item()) == 0


@pytest.fixture(scope="module")
def experts_full():
    """E=384 experts of N=2048 x K=7168 bf16 ~ N(0, 0.02^2) (11.3 GB), drawn on the device."""
    announce("generating the 384-expert weight set on the device")
    W = si.normal_bf16((384, 2048, 7168), 0.02, 5000 + si.TAG_W + 100, DEV)
    torch.cuda.synchronize()
    yield W
    del W
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [1, 16, 64])
def test_grouped_full_size(experts_full, T):
    E, N, K, topk = 384, 2048, 7168, 8
    W = experts_full
    x = si.normal_bf16((T, K), 1.0, 5000 + si.TAG_X + T, DEV)
    ids = si.routing_table(T, E, topk, 5000 + si.TAG_ROUTING + T)
    announce(f"grouped full T={T}")
    out, off, pairs, inv = run_grouped(x, W, ids)
    check_table(ids, E, off, pairs, inv)
    a, b = run_grouped(x, W, ids)[0], out
    assert torch.equal(a, b), "repeat runs bitwise identical"
    assert torch.equal(run_grouped_fused(x, W, ids)[0], out), "fused table path, same bits"
    # sampled outputs: a spread of pairs, 96 rows each (including the last row)
    rng = np.random.default_rng(T)
    P = T * topk
    sel_pairs = sorted(set(rng.choice(P, size=min(P, 12), replace=False).tolist()) | {P - 1})
    rows = np.array(sorted(set(rng.choice(N, size=95, replace=False).tolist()) | {N - 1}))
    xb = bits(x)
    for p in sel_pairs:
        t, j = divmod(p, topk)
        e = int(ids[t, j])
        We = bits(W[e, torch.as_tensor(rows, device=DEV)])
        y, A = orc().projection(xb[t:t + 1], We)
        check_f32(out[t, j, torch.as_tensor(rows, device=DEV)], y[0], A[0], f"grouped T={T} pair {p}")
