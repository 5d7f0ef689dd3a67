"""GPU parity of the router top-k (expert selection upstream of the grouped
projection), through the C ABI: selected ids bit-exact against the oracle's
ranking of the very same fp32 scores, and the router scores themselves
against the oracle projection."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
import skinny_gemm_projection_amd as sg
from gpu_common import DEV, announce, bits, check_f32, counters_delta, orc

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def scores_of(kind, T, E, seed):
    g = torch.Generator().manual_seed(seed)
    if kind == "normal":
        s = torch.randn((T, E), generator=g)
    elif kind == "ties":  # few distinct values: the lower-id rule decides most ranks
        s = torch.randint(-3, 4, (T, E), generator=g).float()
    else:  # NaN, +-inf and ties together
        s = torch.randint(-2, 3, (T, E), generator=g).float()
        u = torch.rand((T, E), generator=g)
        s[u < 0.2] = float("nan")
        s[(u >= 0.2) & (u < 0.3)] = float("-inf")
        s[(u >= 0.3) & (u < 0.35)] = float("inf")
    return s.contiguous()


def run_topk(s, k):
    T, _ = s.shape
    ids = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    top = torch.full((T, k), -7.0, device=DEV)
    before = sg.skinny_gemm_get_counters()
    sg.skinny_gemm_router_topk(s.to(DEV), k, topk_ids=ids, topk_scores=top)
    torch.cuda.synchronize()
    d = counters_delta(before, sg.skinny_gemm_get_counters())
    assert d[sg.SG_KERNEL_ROUTER_TOPK] == (1 if T > 0 else 0)
    return ids.cpu().numpy(), top.cpu().numpy()


@pytest.mark.parametrize("kind", ["normal", "ties", "special"])
@pytest.mark.parametrize("T,E,k", [(1, 384, 8), (16, 384, 8), (64, 384, 8), (200, 384, 8),
                                   (7, 17, 17), (5, 64, 1), (3, 1000, 32), (2, 4096, 32),
                                   (9, 65, 5), (4, 1, 1)])
def test_topk_bit_exact(kind, T, E, k):
    announce(f"router topk {kind} T={T} E={E} k={k}")
    s = scores_of(kind, T, E, 100 * T + E + k)
    ids, top = run_topk(s, k)
    ref_ids, ref_top = orc().router_topk(s.numpy(), k)
    assert np.array_equal(ids, ref_ids), "selected expert ids, bit-exact"
    assert np.array_equal(top.view(np.uint32), ref_top.view(np.uint32)), "selected scores, bitwise"


def test_topk_empty_and_rejected():
    announce("router topk T=0 and rejected sizes")
    s = torch.empty((0, 384), device=DEV)
    ids = sg.skinny_gemm_router_topk(s, 8)
    assert ids.shape == (0, 8)
    good = torch.zeros((4, 40), device=DEV)
    for E, k in [(40, 41), (40, 33), (40, 0)]:
        with pytest.raises(sg.SkinnyGemmError) as e:
            sg.skinny_gemm_router_topk(good[:, :E].contiguous(), k)
        assert e.value.status == 2
    with pytest.raises(sg.SkinnyGemmError) as e:
        sg.skinny_gemm_router_topk(torch.zeros((2, 4097), device=DEV), 8)
    assert e.value.status == 2


@pytest.mark.parametrize("T", [1, 16, 64])
def test_router_end_to_end(T):
    # router scores (the planned skinny projection, N = E = 384, K = 7168), their top-8,
    # and the grouped projection those ids select, each against the oracle
    E, K, k, N = 384, 7168, 8, 256
    announce(f"router end to end T={T}")
    x = si.normal_bf16((T, K), 1.0, 9500 + T, DEV)
    Wr = si.normal_bf16((E, K), 0.02, 9501 + T, DEV)
    ids, top, scores = sg.router_topk(x, Wr, k)
    torch.cuda.synchronize()
    y, A = orc().projection(bits(x), bits(Wr))
    check_f32(scores, y, A, f"router scores T={T}")
    ref_ids, ref_top = orc().router_topk(scores.cpu().numpy(), k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids), "ids from the GPU scores, bit-exact"
    assert np.array_equal(top.cpu().numpy().view(np.uint32), ref_top.view(np.uint32))
    # the selection feeds the per-expert table and the grouped projection
    W = si.normal_bf16((E, N, K), 0.02, 9502 + T, DEV)
    out = torch.empty((T, k, N), device=DEV)
    sg.grouped_skinny_gemm(x, W, ids, out)
    torch.cuda.synchronize()
    ref, A2 = orc().grouped(bits(x), bits(W), ids.cpu().numpy())
    check_f32(out, ref, A2, f"grouped after router T={T}")
