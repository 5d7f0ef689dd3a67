"""HIP graph capture of the entry points.  The header promises that every call is
asynchronous on the caller's stream and may be captured into a HIP graph; here
each path is captured (torch.cuda.CUDAGraph on a stream of its own) and the graph
is replayed several times, with the program's own eager calls and
synchronisations between the replays.  The library's kernels are deterministic,
so every replay must reproduce the eager call bit for bit; the eager result is
checked against the fp64 oracle on sampled rows, so the replays are too.

The outputs are filled with NaN before each replay, so a replay that skipped a
kernel would leave NaN behind.
"""
import numpy as np
import pytest
import torch

import seeded_inputs as si
import skinny_gemm_projection_amd as sg
from gpu_common import DEV, announce, bits, check_f32, orc, sample_rows

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

REPLAYS = 3


def _capture_and_replay(issue, what):
    """issue() launches the calls on the current stream and returns the output
    tensors.  Returns the eager outputs after checking every replay against them."""
    eager = [t.clone() for t in issue()]
    torch.cuda.synchronize()
    gs = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=gs):
        outs = issue()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        for t in outs:
            if t.is_floating_point():
                t.fill_(float("nan"))
            else:
                t.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, ref) in enumerate(zip(outs, eager)):
            assert torch.equal(got, ref), f"{what}: replay {rep} output {i} differs from eager"
        issue()  # eager work between the replays, on the default stream
        torch.cuda.synchronize()
    del g
    return eager


def _proj_case(M, N, K, seed, force=None):
    x = si.normal_bf16((M, K), 1.0, seed, DEV)
    W = si.normal_bf16((N, K), 0.02, seed + 1, DEV)
    plan = sg.skinny_gemm_plan(M, N, K) if force is None else sg.skinny_gemm_plan_force(M, N, K, *force)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
    y32 = torch.empty((M, N), device=DEV)
    y16 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    return x, W, plan, ws, y32, y16


PROJ = [  # (M, N, K, forced plan or None): every projection kernel and reduction
    (1, 2048, 7168, None),                                  # small-matrix kernel
    (4, 4096, 7168, None),                                  # VALU team
    (4, 1000, 7168, (sg.SG_KERNEL_SPLITK_VALU, 8, 1)),      # VALU two-pass + reduction
    (12, 4096, 7168, None),                                 # matrix-core team
    (40, 1000, 7168, None),                                 # chunk kernel + tiled reduction
]


@pytest.mark.parametrize("M,N,K,force", PROJ)
def test_graph_projection_and_residual(M, N, K, force):
    x, W, plan, ws, y32, y16 = _proj_case(M, N, K, 40000 + M, force)
    announce(f"graph projection M={M} N={N} K={K} {sg.KERNEL_NAMES[plan.kernel]} "
             f"S={plan.split_k} two_pass={plan.two_pass}")
    r = si.normal_bf16((M, N), 1.0, 40100 + M, DEV)
    o16 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)

    def issue():
        sg.skinny_gemm(plan, x, W, y_f32=y32, y_bf16=y16, workspace=ws)
        sg.skinny_gemm_residual(plan, x, W, r, out_bf16=o16, workspace=ws)
        return [y32, y16, o16]

    e32, _, _ = _capture_and_replay(issue, f"projection M={M}")
    rows = sample_rows(N, 64, 40200 + M)
    ref, A = orc().projection(bits(x), bits(W)[rows])
    check_f32(e32[:, torch.as_tensor(rows, device=DEV)], ref, A, f"graph projection M={M}")


@pytest.mark.parametrize("T,tables", [(4, False), (16, True)])
def test_graph_grouped(T, tables):
    E, topk, N, K = 64, 8, 256, 2048
    announce(f"graph grouped T={T} tables={tables}")
    x = si.normal_bf16((T, K), 1.0, 41000 + T, DEV)
    W = si.normal_bf16((E, N, K), 0.02, 41001 + T, DEV)
    ids = si.routing_table(T, E, topk, 41002 + T).to(DEV)
    out = torch.empty((T, topk, N), device=DEV)
    ws = torch.empty(max(sg.grouped_skinny_gemm_workspace(T, E, topk, N, K), 256),
                     dtype=torch.uint8, device=DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV) if tables else None
    pairs = torch.empty(T * topk, dtype=torch.int32, device=DEV) if tables else None

    def issue():
        sg.grouped_skinny_gemm(x, W, ids, out, expert_offsets=off, sorted_pairs=pairs,
                               workspace=ws)
        return [out] + ([off, pairs] if tables else [])

    eager = _capture_and_replay(issue, f"grouped T={T}")
    ref, A = orc().grouped(bits(x), bits(W), ids.cpu().numpy())
    check_f32(eager[0], ref, A, f"graph grouped T={T}")


@pytest.mark.parametrize("T,mode", [(2, "fused"), (16, "fused"), (16, "serial"),
                                     (2, "side_stream"), (16, "side_stream"),
                                     (3, "shared_in_routed")])
def test_graph_moe_step(T, mode):
    E, topk, N, Ns, K = 64, 8, 256, 128, 2048
    announce(f"graph moe step T={T} mode={mode}")
    x = si.normal_bf16((T, K), 1.0, 42000 + T, DEV)
    Wr = si.normal_bf16((E, K), 0.02, 42001, DEV)
    Wsh = si.normal_bf16((Ns, K), 0.02, 42002, DEV)
    if mode == "fused":
        Wr, Wsh = sg.concat_router_shared(Wr, Wsh)
    # side_stream: the fork (event record + wait) and the join happen inside the
    # capture, so the shared expert becomes a parallel branch of the graph
    We = si.normal_bf16((E, N, K), 0.02, 42003, DEV)
    ws = torch.empty(max(sg.skinny_moe_step_workspace(T, K, E, topk, N, Ns), 256),
                     dtype=torch.uint8, device=DEV)

    def issue():
        ids, top, scores, out, shared = sg.skinny_moe_step(x, Wr, We, Wsh, topk, mode=mode,
                                                           workspace=ws)
        return [ids, top, out, shared]

    ids, _, out, shared = _capture_and_replay(issue, f"moe step T={T} {mode}")
    ref, A = orc().grouped(bits(x), bits(We), ids.cpu().numpy())
    check_f32(out, ref, A, f"graph moe step routed T={T}")
    sref, sA = orc().projection(bits(x), bits(Wsh))
    check_f32(shared, sref, sA, f"graph moe step shared T={T}")


@pytest.mark.parametrize("fmt,M,N,K", [("mxfp4", 2, 2048, 7168), ("mxfp4", 12, 1000, 4096),
                                       ("fp8", 1, 2048, 7168), ("fp8", 8, 1000, 4096)])
def test_graph_low_precision(fmt, M, N, K):
    announce(f"graph {fmt} M={M} N={N} K={K}")
    x = si.normal_bf16((M, K), 1.0, 43000 + M, DEV)
    if fmt == "mxfp4":
        codes, scales = si.mxfp4_weights(N, K, 43001 + M, DEV)
        call = sg.skinny_gemm_mxfp4
    else:
        codes, scales = si.fp8_weights(N, K, 43001 + M, DEV)
        call = sg.skinny_gemm_fp8
    y32 = torch.empty((M, N), device=DEV)
    y16 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)

    def issue():
        call(x, codes, scales, y_f32=y32, y_bf16=y16)
        return [y32, y16]

    e32, _ = _capture_and_replay(issue, f"{fmt} M={M}")
    rows = sample_rows(N, 48, 43100 + M)
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    for n in rows[:8]:
        if fmt == "mxfp4":
            ref, A = orc().projection_mxfp4(bits(x), c[n:n + 1], s[n:n + 1])
        else:
            ref, A = orc().projection_fp8(bits(x), c[n:n + 1], s[n // 128:n // 128 + 1])
        check_f32(e32[:, n:n + 1], ref, A, f"graph {fmt} row {n}")


def test_graph_router_and_prefetch():
    T, E, K, k = 16, 384, 2048, 8
    announce("graph router top-k and prefetch")
    x = si.normal_bf16((T, K), 1.0, 44000, DEV)
    Wr = si.normal_bf16((E, K), 0.02, 44001, DEV)
    Wp = si.normal_bf16((1024, 1024), 0.02, 44002, DEV)

    def issue():
        sg.skinny_gemm_prefetch(Wp)  # writes nothing; captured and replayed with the rest
        ids, top, scores = sg.router_topk(x, Wr, k)
        return [ids, top, scores]

    ids, _, scores = _capture_and_replay(issue, "router top-k")
    ref_ids = orc().router_topk(scores.cpu().numpy(), k)[0]
    assert np.array_equal(ids.cpu().numpy(), ref_ids), "top-k ids of the replayed scores"
