"""GPU parity of one MoE decode step through the C ABI (skinny_moe_step): router
scores, top-k, routed-expert projection, and the shared expert's projection --
fused into the router's GEMM, on a side stream that overlaps the routing,
serial, or (up to 4 tokens) inside the routed-expert launch.

Each output of each mode is checked against the oracle: the router scores and
the shared expert against oracle_projection, the ids (bit-exact) against
oracle_router_topk of the GPU scores, the routed output against oracle_grouped
with those ids.  The side-stream step must give bitwise the same outputs as the
serial one (the same kernels and plans run either way), and the shared-in-routed
step the same ids, scores and routed outputs (its shared expert is another
kernel's sum, checked against the oracle)."""
import ctypes

import numpy as np
import pytest
import torch

import seeded_inputs as si
import skinny_gemm_projection_amd as sg
from gpu_common import DEV, announce, bits, check_f32, counters_delta, orc

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def weights(T, K, E, N, N_shared, seed):
    """x, W_router, experts, W_shared; the router and shared weights are views of one
    [E + N_shared, K] tensor, the layout every mode accepts."""
    x = si.normal_bf16((T, K), 1.0, seed, DEV)
    Wr = si.normal_bf16((E, K), 0.02, seed + 1, DEV)
    We = si.normal_bf16((E, N, K), 0.02, seed + 2, DEV)
    Ws = si.normal_bf16((N_shared, K), 0.02, seed + 3, DEV) if N_shared else None
    if Ws is not None:
        Wr, Ws = sg.concat_router_shared(Wr, Ws)
    return x, Wr, We, Ws


def check_step(res, x, Wr, We, Ws, topk, what, out_rows=None):
    ids, top, scores, out, shared = res
    xb = bits(x)
    y, A = orc().projection(xb, bits(Wr))
    check_f32(scores, y, A, f"{what}: router scores")
    ref_ids, ref_top = orc().router_topk(scores.cpu().numpy(), topk)
    assert np.array_equal(ids.cpu().numpy(), ref_ids), f"{what}: ids bit-exact"
    assert np.array_equal(top.cpu().numpy().view(np.uint32), ref_top.view(np.uint32))
    if out_rows is None:
        ref, A2 = orc().grouped(xb, bits(We), ids.cpu().numpy())
        check_f32(out, ref, A2, f"{what}: routed experts")
    else:  # sampled rows of every pair's output (the full expert set is too big to copy)
        rows = torch.as_tensor(out_rows, device=DEV)
        ids_np = ids.cpu().numpy()
        for t in range(x.shape[0]):
            for j in range(topk):
                e = int(ids_np[t, j])
                yr, Ar = orc().projection(xb[t:t + 1], bits(We[e, rows]))
                check_f32(out[t, j, rows], yr[0], Ar[0], f"{what}: routed pair ({t},{j})")
    if Ws is not None:
        ys, As = orc().projection(xb, bits(Ws))
        check_f32(shared, ys, As, f"{what}: shared expert")


@pytest.mark.parametrize("T,K,E,N,N_shared,topk", [(1, 1024, 64, 96, 160, 8),
                                                    (5, 520, 40, 33, 72, 6),
                                                    (64, 1032, 64, 40, 48, 8),
                                                    (16, 256, 17, 130, 0, 3),
                                                    (4, 520, 384, 40, 0, 8),
                                                    (2, 264, 500, 24, 32, 32),
                                                    (3, 1032, 64, 0, 48, 4),
                                                    (4, 520, 40, 33, 72, 6),
                                                    (4, 7168, 256, 64, 2048, 8),
                                                    (3, 4104, 100, 200, 7, 4),
                                                    (1, 1024, 16, 8, 3000, 4)])
def test_step_small(T, K, E, N, N_shared, topk):
    x, Wr, We, Ws = weights(T, K, E, N, N_shared, 7000 + T)
    res = {}
    for mode in sg.MOE_STEP_MODES:
        announce(f"moe step small {mode} T={T} K={K} E={E} N={N} Ns={N_shared} k={topk}")
        before = sg.skinny_gemm_get_counters()
        res[mode] = sg.skinny_moe_step(x, Wr, We, Ws, topk, mode=mode)
        torch.cuda.synchronize()
        d = counters_delta(before, sg.skinny_gemm_get_counters())
        # the step asks for no table output: up to 512 pairs the grouped launch builds
        # its table itself (no table kernel); up to 4 tokens (E <= 512) it also ranks
        # the scores itself (no top-k kernel)
        route_fused = 1 <= T <= 4 and E <= 512 and N > 0
        assert d[sg.SG_KERNEL_ROUTER_TOPK] == (0 if route_fused else 1)
        assert d[sg.SG_KERNEL_MOE_TABLE] == (0 if T * topk <= 512 else 1)
        assert d[sg.SG_KERNEL_GROUPED] == (1 if N > 0 else 0)
        projections = sum(d[k] for k in (sg.SG_KERNEL_GEMV, sg.SG_KERNEL_SPLITK_VALU,
                                         sg.SG_KERNEL_SPLITK_MFMA))
        in_routed = mode == "shared_in_routed" and route_fused
        one = mode == "fused" or N_shared == 0 or in_routed
        assert projections == (1 if one else 2), (mode, d)
        check_step(res[mode], x, Wr, We, Ws, topk, f"{mode} T={T}")
    for a, b in zip(res["side_stream"], res["serial"]):
        assert torch.equal(a, b), "side-stream and serial steps bitwise identical"
    for a, b in zip(res["shared_in_routed"][:4], res["serial"][:4]):
        assert torch.equal(a, b), "shared-in-routed: ids, scores, routed outputs as serial"


@pytest.mark.parametrize("T", [7, 3, 1])
def test_step_integer_bit_exact(T):
    # integer inputs: every partial sum is exact in fp32, so every output is bit-exact;
    # T <= 4 takes the launch that ranks the scores itself
    K, E, N, Ns, topk = 264, 24, 50, 70, 5
    announce(f"moe step integer inputs T={T}")
    x = si.integer_bf16((T, K), -4, 4, 7101, DEV)
    Wr = si.integer_bf16((E, K), -4, 4, 7102, DEV)
    We = si.integer_bf16((E, N, K), -4, 4, 7103, DEV)
    Ws = si.integer_bf16((Ns, K), -4, 4, 7104, DEV)
    Wr, Ws = sg.concat_router_shared(Wr, Ws)
    xb = bits(x)
    y, _ = orc().projection(xb, bits(Wr))
    ref_ids, _ = orc().router_topk(y.astype(np.float32), topk)  # heavy ties: the id rule decides
    ref, _ = orc().grouped(xb, bits(We), ref_ids)
    ys, _ = orc().projection(xb, bits(Ws))
    for mode in sg.MOE_STEP_MODES:
        ids, top, scores, out, shared = sg.skinny_moe_step(x, Wr, We, Ws, topk, mode=mode)
        torch.cuda.synchronize()
        assert np.array_equal(scores.cpu().numpy().astype(np.float64), y), mode
        assert np.array_equal(ids.cpu().numpy(), ref_ids), mode
        assert np.array_equal(out.cpu().numpy().astype(np.float64), ref), mode
        assert np.array_equal(shared.cpu().numpy().astype(np.float64), ys), mode


def raw_step(x, Wr, We, topk, T=None, ws_bytes=None, flags=0):
    """skinny_moe_step through ctypes with chosen sizes; returns (status, outputs)."""
    T = x.shape[0] if T is None else T
    E, N, K = We.shape
    ids = torch.full((max(T, 1), topk), -5, dtype=torch.int32, device=DEV)
    scores = torch.full((max(T, 1), E), -5.0, device=DEV)
    out = torch.full((max(T, 1), topk, N), -5.0, device=DEV)
    need = sg.skinny_moe_step_workspace(min(T, 64), K, E, topk, N, 0)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
    step = sg.SgMoeStep(x.data_ptr(), Wr.data_ptr(), We.data_ptr(), None, scores.data_ptr(),
                        ids.data_ptr(), None, out.data_ptr(), None, T, K, E, topk, N, 0, flags)
    lib = sg._c()
    st = lib.skinny_moe_step(ctypes.byref(step), ws.data_ptr(),
                             need if ws_bytes is None else ws_bytes,
                             torch.cuda.current_stream().cuda_stream, None, None, None)
    torch.cuda.synchronize()
    return st, (ids, scores, out)


def test_step_rejections_launch_nothing():
    announce("moe step rejected calls")
    x, Wr, We, _ = weights(65, 64, 16, 24, 0, 7200)
    cases = [(dict(T=65), 3),                        # batch above the decode path
             (dict(T=4, ws_bytes=16), 5),            # workspace too small
             (dict(T=4, flags=4), 2),                # unknown mode flag
             (dict(T=4, flags=3), 2)]                # two placements of the shared expert
    for kw, status in cases:
        before = sg.skinny_gemm_get_counters()
        st, outs = raw_step(x, Wr, We, 4, **kw)
        assert st == status, (kw, st)
        assert counters_delta(before, sg.skinny_gemm_get_counters()) == [0] * sg.SG_NUM_COUNTERS
        for t in outs:
            assert bool((t == -5).all()), "a rejected call leaves its outputs alone"
    st, _ = raw_step(x, Wr, We, 17)  # topk > E
    assert st == 2
    assert sg.skinny_moe_step_workspace(4, 64, 16, 17, 24, 0) == 0
    # T = 0: nothing to do, nothing launched
    before = sg.skinny_gemm_get_counters()
    st, _ = raw_step(x, Wr, We, 4, T=0)
    assert st == 0
    assert counters_delta(before, sg.skinny_gemm_get_counters()) == [0] * sg.SG_NUM_COUNTERS


@pytest.mark.parametrize("T", [1, 16])
def test_step_side_stream_under_random_delays(T):
    # Timing hazards of the two streams: random GPU sleeps on the caller's stream
    # before the step (the fork waits for them) and on the side stream (the shared
    # expert then starts anywhere from the router projection to the end of the
    # routed experts), and x overwritten on the caller's stream right after the
    # call (the join must hold that write back until the shared expert has read
    # x).  Every run must equal the serial step bit for bit; the serial step is
    # checked against the oracle.  T = 1 takes the launch that ranks the scores
    # itself, T = 16 the separate top-k kernel.
    K, E, N, Ns, topk = 2048, 64, 512, 2048, 8
    x, Wr, We, Ws = weights(T, K, E, N, Ns, 7500 + T)
    announce(f"moe step side stream under random delays T={T}: serial reference")
    ref = sg.skinny_moe_step(x, Wr, We, Ws, topk, mode="serial")
    torch.cuda.synchronize()
    check_step(ref, x, Wr, We, Ws, topk, f"serial T={T}")
    side, _, _ = sg._side_resources(x.device)
    main = torch.cuda.current_stream()
    g = torch.Generator().manual_seed(11 + T)
    for it in range(12):
        announce(f"moe step side stream T={T} iteration {it}")
        xr = x.clone()
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            torch.cuda._sleep(int(torch.randint(0, 60000, (1,), generator=g)))
        torch.cuda._sleep(int(torch.randint(0, 30000, (1,), generator=g)))
        got = sg.skinny_moe_step(xr, Wr, We, Ws, topk, mode="side_stream")
        xr.fill_(3.0)  # on the caller's stream, right after the call
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"iteration {it}: output {i} differs from the serial step"
    assert main.query()


@pytest.fixture(scope="module")
def full_set():
    """E=384 experts of N=2048 x K=7168 (11.3 GB), the router [384, 7168] and a shared
    expert [2048, 7168], drawn on the device."""
    announce("generating the 384-expert set, router and shared expert on the device")
    Wr, Ws = sg.concat_router_shared(si.normal_bf16((384, 7168), 0.02, 7301, DEV),
                                     si.normal_bf16((2048, 7168), 0.02, 7303, DEV))
    We = si.normal_bf16((384, 2048, 7168), 0.02, 7302, DEV)
    torch.cuda.synchronize()
    yield Wr, We, Ws
    del Wr, We, Ws
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [1, 16, 64])
def test_step_full_size(full_set, T):
    Wr, We, Ws = full_set
    x = si.normal_bf16((T, 7168), 1.0, 7400 + T, DEV)
    rows = np.array(sorted(set(np.random.default_rng(T).choice(2048, 23, replace=False).tolist())
                           | {0, 2047}))
    res = {}
    for mode in sg.MOE_STEP_MODES:
        announce(f"moe step full size {mode} T={T}")
        res[mode] = sg.skinny_moe_step(x, Wr, We, Ws, 8, mode=mode)
        torch.cuda.synchronize()
        check_step(res[mode], x, Wr, We, Ws, 8, f"full {mode} T={T}",
                   out_rows=rows if T <= 16 else rows[:6])
    for a, b in zip(res["side_stream"], res["serial"]):
        assert torch.equal(a, b), "side-stream and serial steps bitwise identical"
    for a, b in zip(res["shared_in_routed"][:4], res["serial"][:4]):
        assert torch.equal(a, b), "shared-in-routed: ids, scores, routed outputs as serial"
