"""Side-stream weight prefetch: reads only the given weights, changes no
result, and stays correct under random launch timing on both streams (the
timing-dependent hazard class the pages warn about).  The projections that
follow a prefetch are checked against the fp64 oracle on sampled rows, and
bit for bit against the same projection without a prefetch."""
import pytest
import torch

import seeded_inputs as si
import skinny_gemm_projection_amd as sg
from gpu_common import DEV, announce, bits, check_f32, counters_delta, orc, sample_rows

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def check_rows(y, x, W, what, count=64, seed=0):
    rows = sample_rows(W.shape[0], count, seed)
    ref, A = orc().projection(bits(x), bits(W[torch.as_tensor(rows, device=W.device)]))
    check_f32(y[:, torch.as_tensor(rows, device=y.device)], ref, A, what)


def test_prefetch_changes_nothing():
    M, N, K = 2, 8192, 7168
    x = si.normal_bf16((M, K), 1.0, 6000, DEV)
    W = si.normal_bf16((N, K), 0.02, 6001, DEV)
    W_copy = W.clone()
    plan = sg.skinny_gemm_plan(M, N, K)
    ref = torch.empty((M, N), device=DEV)
    sg.skinny_gemm(plan, x, W, y_f32=ref)
    announce("prefetch then projection")
    before = sg.skinny_gemm_get_counters()
    sg.skinny_gemm_prefetch(W)
    y = torch.empty((M, N), device=DEV)
    sg.skinny_gemm(plan, x, W, y_f32=y)
    torch.cuda.synchronize()
    assert counters_delta(before, sg.skinny_gemm_get_counters())[sg.SG_KERNEL_PREFETCH] == 1
    assert torch.equal(y, ref)
    check_rows(y, x, W, "projection after a prefetch", 128, 6002)
    assert torch.equal(W, W_copy), "prefetch must not write"
    sg.skinny_gemm_prefetch(W, nbytes=4096 * 7 + 16)  # a partial range
    torch.cuda.synchronize()


def test_prefetch_on_side_stream_under_random_delays():
    M, N, K = 8, 4096, 7168
    x = si.normal_bf16((M, K), 1.0, 6100, DEV)
    Ws = [si.normal_bf16((N, K), 0.02, 6101 + i, DEV) for i in range(3)]
    plan = sg.skinny_gemm_plan(M, N, K)
    refs = []
    for W in Ws:
        r = torch.empty((M, N), device=DEV)
        sg.skinny_gemm(plan, x, W, y_f32=r)
        refs.append(r)
    torch.cuda.synchronize()
    for i, (W, r) in enumerate(zip(Ws, refs)):
        check_rows(r, x, W, f"projection {i} of the prefetch ring", 48, 6110 + i)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    g = torch.Generator().manual_seed(3)
    for it in range(12):
        announce(f"side-stream prefetch iteration {it}")
        outs = []
        for i, W in enumerate(Ws):
            nxt = Ws[(i + 1) % len(Ws)]
            ready = torch.cuda.Event()
            ready.record(main)
            with torch.cuda.stream(side):
                side.wait_event(ready)
                torch.cuda._sleep(int(torch.randint(0, 20000, (1,), generator=g)))
                sg.skinny_gemm_prefetch(nxt, stream=side)
            torch.cuda._sleep(int(torch.randint(0, 20000, (1,), generator=g)))
            y = torch.empty((M, N), device=DEV)
            sg.skinny_gemm(plan, x, W, y_f32=y)
            outs.append(y)
        main.wait_stream(side)
        torch.cuda.synchronize()
        for y, r in zip(outs, refs):
            assert torch.equal(y, r)


@pytest.mark.gpu
@pytest.mark.parametrize("rows,row_bytes,rows_per_iter,grid", [
    (8192, 14336, 2, 512), (8192, 14336, 1, 512), (4097, 14336, 2, 512), (33, 16, 1, 1),
    (1000, 1040, 2, 7), (300, 16384, 1, 3000), (1, 16000, 2, 2)])
def test_read_probe_reads_only(rows, row_bytes, rows_per_iter, grid):
    """The read probe launches once, returns SG_OK and writes nothing: the matrix it
    reads is unchanged and the launch counters do not move."""
    announce(f"read probe rows={rows} row_bytes={row_bytes} R={rows_per_iter} grid={grid}")
    W = torch.randint(0, 256, (rows, row_bytes), dtype=torch.uint8, device=DEV)
    before_w = W.clone()
    before = sg.skinny_gemm_get_counters()
    sg.skinny_gemm_read_probe(W, rows_per_iter, grid)
    torch.cuda.synchronize()
    assert torch.equal(W, before_w)
    assert sg.skinny_gemm_get_counters() == before
