"""C-ABI boundary checks that need no GPU: the library loads, exports every
function include/skinny_gemm.h declares, plans shapes as documented, and
rejects bad calls before touching the device.

Calls with made-up device pointers only run on a host without a GPU: there
any accidental launch fails harmlessly instead of reading a stray address.
"""
import ctypes
import json
import os
import re
import subprocess
import sys

import pytest
import torch

import skinny_gemm_projection_amd as sg
from skinny_gemm_projection_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "skinny_gemm.h")

no_gpu_only = pytest.mark.skipif(torch.cuda.is_available(),
                                 reason="fake device pointers are only passed on a host without a GPU")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s+(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if not n.startswith("SG_")))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("skinny_gemm_plan", "skinny_gemm_plan_force", "skinny_gemm", "skinny_gemm_residual",
                 "grouped_skinny_gemm_workspace", "grouped_skinny_gemm", "skinny_gemm_prefetch",
                 "skinny_gemm_status_str", "skinny_gemm_get_counters", "skinny_gemm_reset_counters"):
        assert want in names, want


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(sg.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", sg.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, f"{name} missing from the dynamic symbol table"


def test_binding_constants_match_the_header():
    text = open(HEADER).read()
    consts = {n: int(v) for n, v in re.findall(r"^\s*(SG_KERNEL_\w+) = (\d+)", text, flags=re.M)}
    consts.update({n: int(v) for n, v in
                   re.findall(r"^#define (SG_(?:MOE_STEP_\w+|NUM_COUNTERS)) (\d+)$", text,
                              flags=re.M)})
    assert "SG_MOE_STEP_SHARED_IN_ROUTED" in consts and "SG_KERNEL_FP8" in consts
    for name, value in consts.items():
        assert getattr(_lib, name) == value, name


def test_python_binding_has_the_same_names():
    for name in declared_functions():
        assert callable(getattr(sg, name)), name


def test_status_strings():
    for code, name in _lib.STATUS_NAMES.items():
        assert sg.skinny_gemm_status_str(code).startswith(name)
    assert "unknown" in sg.skinny_gemm_status_str(99)


# ------------------------------------------------------------------ planner


def test_plan_kernel_by_batch():
    for M in range(1, 65):
        p = sg.skinny_gemm_plan(M, 4096, 7168)
        # the team kernel's 256 workgroups fill the GPU at N = 4096: matrix cores from M = 3
        want = sg.SG_KERNEL_GEMV if M <= 2 else sg.SG_KERNEL_SPLITK_MFMA
        assert p.kernel == want, (M, p)
        assert (p.M, p.N, p.K) == (M, 4096, 7168)
    # past K = 8192 (more than 8 rounds a wave: the team kernel's loop form) and below
    # K = 4096 (the streaming kernel ahead) from M = 6
    for K in (16384, 2048):
        for M in range(3, 9):
            p = sg.skinny_gemm_plan(M, 4096, K)
            want = sg.SG_KERNEL_SPLITK_VALU if M < 6 else sg.SG_KERNEL_SPLITK_MFMA
            assert p.kernel == want, (M, K, p)


def test_plan_kernel_by_batch_few_rows():
    # N/16 workgroups do not fill the GPU: the vector-ALU kernel up to M = 7
    for M in range(3, 9):
        p = sg.skinny_gemm_plan(M, 1024, 7168)
        want = sg.SG_KERNEL_SPLITK_VALU if M < 8 else sg.SG_KERNEL_SPLITK_MFMA
        assert p.kernel == want, (M, p)


def test_plan_team_or_chunk_by_width():
    # 8..16 rows on matrix cores: the team kernel (16-row tiles, one pass) while N/16 tiles
    # fill the CUs (two tiles a wave from N = 8161 and M = 12, so its grid is N/32, unless
    # K is a multiple of 4096); the chunk kernel (128/256-row tiles, second pass) below
    # that width and from 17 rows
    for M, N, K, team, grid in [(8, 4096, 7168, True, 256), (16, 4096, 7168, True, 256),
                                (8, 8192, 7168, True, 512), (11, 8192, 7168, True, 512),
                                (12, 8192, 7168, True, 256), (16, 8192, 7168, True, 256),
                                (16, 7168, 7168, True, 448), (16, 8160, 7168, True, 510),
                                (16, 8161, 7168, True, 256), (16, 16384, 7168, True, 512),
                                (16, 8192, 8192, True, 512), (12, 8192, 4096, True, 512),
                                (16, 8192, 6144, True, 256), (16, 2048, 7168, False, None),
                                (17, 4096, 7168, False, None)]:
        p = sg.skinny_gemm_plan(M, N, K)
        assert p.kernel == sg.SG_KERNEL_SPLITK_MFMA, (M, N, K, p)
        assert (p.tile_n == 16 and not p.two_pass) == team, (M, N, K, p)
        if team:
            assert p.grid == grid, (M, N, K, p)


def test_plan_rejects():
    cases = [((65, 16, 16), 3), ((1000, 16, 16), 3), ((-1, 16, 16), 2), ((1, -1, 16), 2),
             ((1, 16, -8), 2), ((1, (1 << 20) + 1, 16), 2), ((1, 16, 12), 4), ((1, 16, 7), 4)]
    for (M, N, K), code in cases:
        with pytest.raises(sg.SkinnyGemmError) as e:
            sg.skinny_gemm_plan(M, N, K)
        assert e.value.status == code, (M, N, K, e.value.status)


def test_plan_empty_problems():
    for M, N, K in [(0, 16, 16), (4, 0, 16), (0, 0, 0)]:
        p = sg.skinny_gemm_plan(M, N, K)
        assert p.kernel == sg.SG_KERNEL_NONE and p.workspace_bytes == 0
    p = sg.skinny_gemm_plan(3, 16, 0)  # K = 0: the empty sum, still written
    assert p.kernel == sg.SG_KERNEL_SPLITK_VALU and p.k_chunk == 0


@pytest.mark.parametrize("N,K", [(1024, 1024), (8192, 7168), (4096, 7168), (7168, 8192),
                                 (2048, 7168), (384, 7168), (100, 136), (33, 8), (4096, 16384)])
def test_plan_invariants(N, K):
    for M in range(1, 65):
        p = sg.skinny_gemm_plan(M, N, K)
        S, c = p.split_k, p.k_chunk
        assert S >= 1 and c % 8 == 0
        assert c == 64 * -(-K // (64 * S)), "chunk is ceil(K / S) rounded up to a multiple of 64"
        assert (S - 1) * c < K or K == 0, "no empty chunk in an automatic plan"
        if p.two_pass:
            assert S > 1
            assert p.workspace_bytes >= S * M * N * 4 and p.workspace_bytes % 256 == 0
        else:
            assert p.workspace_bytes == 0
        if p.kernel == sg.SG_KERNEL_SPLITK_VALU and S in (1, 2, 4) and K <= 8192:
            assert not p.two_pass, "VALU splits of 1, 2, 4 waves reduce inside the workgroup"
        if p.kernel in (sg.SG_KERNEL_GEMV, sg.SG_KERNEL_SPLITK_VALU):
            nch = -(-c // 512)
            cap = 16 if M <= 2 else 8 if M <= 4 else 4 if M <= 8 else 2
            assert nch <= cap, (M, N, K, p)
        if p.kernel == sg.SG_KERNEL_SPLITK_MFMA and p.tile_n != 16:
            assert p.tile_n in (128, 256)
            tiles = -(-N // p.tile_n)
            assert p.grid == -(-tiles // 8) * 8 * S, "column tiles padded to the 8 XCDs"
        assert p.grid >= 1
        assert sg.skinny_gemm_plan(M, N, K).as_dict() == p.as_dict(), "deterministic"


def test_plan_small_matrix_kernel_has_no_split_up_to_8192():
    for K in (1024, 7168, 8192):
        for M in (1, 2):
            assert sg.skinny_gemm_plan(M, 8192, K).split_k == 1


def test_plan_force():
    G, V, F = sg.SG_KERNEL_GEMV, sg.SG_KERNEL_SPLITK_VALU, sg.SG_KERNEL_SPLITK_MFMA
    p = sg.skinny_gemm_plan_force(8, 4096, 7168, F, 2)
    assert p.kernel == F and p.split_k == 2 and p.k_chunk == 3584
    p = sg.skinny_gemm_plan_force(1, 4096, 7168, V, 14)
    assert p.kernel == V and p.k_chunk == 512
    p = sg.skinny_gemm_plan_force(4, 4096, 7168, F, 3)
    assert p.k_chunk == 2432 and 2 * 2432 < 7168 <= 3 * 2432
    p = sg.skinny_gemm_plan_force(5, 1000, 2056, V, 2)
    assert p.k_chunk == 1088 and not p.two_pass and p.workspace_bytes == 0
    p = sg.skinny_gemm_plan_force(5, 1000, 2056, V, 2, two_pass=1)
    assert p.two_pass and p.workspace_bytes >= 2 * 5 * 1000 * 4
    p = sg.skinny_gemm_plan_force(12, 4096, 7168, V, 0)
    assert p.split_k == 8 and not p.two_pass, "M >= 9 splits 8 ways inside a 512-thread workgroup"
    p = sg.skinny_gemm_plan_force(4, 4096, 7168, V, 3)
    assert p.two_pass, "a 3-way split has no in-workgroup form"
    p = sg.skinny_gemm_plan_force(16, 4096, 7168, F, 1)
    assert not p.two_pass and p.workspace_bytes == 0
    p = sg.skinny_gemm_plan(64, 4096, 7168)
    assert p.split_k == 8 and p.two_pass and p.grid == 32 * 8 and p.tile_n == 128
    p = sg.skinny_gemm_plan_force(32, 4096, 7168, F, 5, tile_n=128)
    assert p.two_pass and p.grid == 32 * 5 and p.tile_n == 128
    p = sg.skinny_gemm_plan_force(32, 4096, 7168, F, 16, tile_n=256)
    assert p.two_pass and p.grid == 16 * 16 and p.tile_n == 256
    p = sg.skinny_gemm_plan_force(64, 7168, 8192, F, 0, tile_n=256)
    assert p.tile_n == 256 and p.grid == 32 * p.split_k, "28 tiles padded to 32"
    p = sg.skinny_gemm_plan_force(20, 4096, 7168, F, 4, tile_n=16)
    assert not p.two_pass and p.tile_n == 16, "tile_n 16 asks for the team kernel"
    p = sg.skinny_gemm_plan_force(64, 4096, 7168, F, 4, 0)
    assert not p.two_pass and p.tile_n == 16 and p.grid == 256, "team kernel"
    p = sg.skinny_gemm_plan_force(64, 4096, 7168, F, 2)
    assert p.two_pass and p.tile_n in (128, 256), "x is staged in phases: any chunk fits"
    for args in [(3, 64, 64, G, 1), (16, 64, 64, V, 1), (4, 4096, 7168, F, 65),
                 (4, 4096, 7168, 9, 1), (8, 4096, 7168, V, 1), (8, 4096, 7168, V, 2),
                 (4, 4096, 7168, V, 3, 0), (16, 4096, 7168, F, 3, 0), (3, 4096, 7168, V, 8, 0),
                 (16, 4096, 7168, F, 16, 0), (16, 4096, 7168, F, 8, 1, 64),
                 (16, 4096, 7168, F, 8, 1, 16)]:
        with pytest.raises(sg.SkinnyGemmError) as e:
            sg.skinny_gemm_plan_force(*args)
        assert e.value.status == 6, args


def test_grouped_workspace_size():
    assert sg.grouped_skinny_gemm_workspace(64, 384, 8, 2048, 7168) >= 4 * (3 * 384 + 512 + 3)
    assert sg.grouped_skinny_gemm_workspace(257, 384, 8, 2048, 7168) == 0
    assert sg.grouped_skinny_gemm_workspace(4, 384, 8, 2048, 8200) == 0


# ------------------------------------------------------------------ host-rejected calls


def _raw():
    return _lib.load()


@no_gpu_only
def test_projection_errors_return_before_launch():
    c = _raw()
    sg.skinny_gemm_reset_counters()
    p = sg.skinny_gemm_plan_force(16, 4096, 7168, sg.SG_KERNEL_SPLITK_MFMA, 4, 1)  # two-pass
    assert p.two_pass and p.workspace_bytes > 0
    bp = ctypes.byref(p)
    A = 0x10000  # aligned, never dereferenced
    ws = p.workspace_bytes
    assert c.skinny_gemm(None, A, A, A, None, A, ws, None) == 1
    assert c.skinny_gemm(bp, None, A, A, None, A, ws, None) == 1
    assert c.skinny_gemm(bp, A, A, None, None, A, ws, None) == 1
    assert c.skinny_gemm(bp, A + 8, A, A, None, A, ws, None) == 4
    assert c.skinny_gemm(bp, A, A, A + 4, None, A, ws, None) == 4
    assert c.skinny_gemm(bp, A, A, A, None, None, ws, None) == 5
    assert c.skinny_gemm(bp, A, A, A, None, A, ws - 1, None) == 5
    assert c.skinny_gemm(bp, A, A, A, None, A + 8, ws, None) == 4
    bad = _lib.SgPlan.from_buffer_copy(p)
    bad.grid += 1
    assert c.skinny_gemm(ctypes.byref(bad), A, A, A, None, A, ws, None) == 6
    bad = _lib.SgPlan.from_buffer_copy(p)
    bad.N = 4097
    assert c.skinny_gemm(ctypes.byref(bad), A, A, A, None, A, ws, None) == 6
    assert c.skinny_gemm_residual(bp, A, A, None, A, None, A, ws, None) == 1
    assert c.skinny_gemm_residual(bp, A, A, A, None, None, A, ws, None) == 1
    assert c.skinny_gemm_residual(bp, A, A, A + 2, A, None, A, ws, None) == 4
    assert sum(sg.skinny_gemm_get_counters()) == 0, "nothing may launch on a rejected call"


@no_gpu_only
def test_empty_projection_launches_nothing():
    c = _raw()
    sg.skinny_gemm_reset_counters()
    p = sg.skinny_gemm_plan(0, 4096, 7168)
    assert c.skinny_gemm(ctypes.byref(p), None, None, None, None, None, 0, None) == 0
    assert sum(sg.skinny_gemm_get_counters()) == 0


@no_gpu_only
def test_grouped_and_prefetch_errors_return_before_launch():
    c = _raw()
    sg.skinny_gemm_reset_counters()
    A = 0x10000
    ws = sg.grouped_skinny_gemm_workspace(4, 384, 8, 2048, 7168)
    args = dict(x=A, T=4, W=A, E=384, N=2048, K=7168, ids=A, topk=8, out=A, off=None, sp=None,
                inv=None, ws=A, wsb=ws)

    def call(**kw):
        a = dict(args, **kw)
        return c.grouped_skinny_gemm(a["x"], a["T"], a["W"], a["E"], a["N"], a["K"], a["ids"],
                                     a["topk"], a["out"], a["off"], a["sp"], a["inv"], a["ws"],
                                     a["wsb"], None)

    assert call(T=257) == 2
    assert call(topk=0) == 2
    assert call(E=0) == 2
    assert call(K=8200) == 2
    assert call(K=7164) == 4
    assert call(ids=None) == 1
    assert call(out=None) == 1
    assert call(x=None) == 1
    assert call(W=A + 4) == 4
    assert call(off=A + 4) == 4
    assert call(ws=None) == 5
    assert call(wsb=ws - 4) == 5
    assert c.skinny_gemm_prefetch(None, 16, None) == 1
    assert c.skinny_gemm_prefetch(A, 24, None) == 4
    assert c.skinny_gemm_prefetch(A + 8, 32, None) == 4
    assert c.skinny_gemm_prefetch(A, 0, None) == 0
    assert sum(sg.skinny_gemm_get_counters()) == 0


@no_gpu_only
def test_read_probe_errors_return_before_launch():
    c = _raw()
    A = 0x10000
    probe = c.skinny_gemm_read_probe
    assert probe(A, -1, 14336, 2, 512, None) == 2          # negative rows
    assert probe(A, 8, 8, 2, 512, None) == 2               # row shorter than one load
    assert probe(A, 8, 16400, 2, 512, None) == 2           # over 16 KB a row
    assert probe(A, 8, 14336, 3, 512, None) == 2           # 1 or 2 rows per iteration
    assert probe(A, 8, 14336, 2, 0, None) == 2             # empty grid
    assert probe(A, 8, 14344, 2, 512, None) == 4           # row_bytes % 16
    assert probe(A + 8, 8, 14336, 2, 512, None) == 4       # misaligned
    assert probe(None, 8, 14336, 2, 512, None) == 1
    assert probe(None, 0, 14336, 2, 512, None) == 0        # nothing to read


@no_gpu_only
def test_fp8_size_limits_return_before_launch():
    # status 3 (unsupported) for sizes outside the kernel's x storage, 4 for K % 16;
    # a size inside the limits gets past those checks and stops at the missing
    # output (status 1)
    c = _raw()
    sg.skinny_gemm_reset_counters()
    A = 0x10000

    def call(M, K, y=None, N=8, ws=None, ws_bytes=0):
        return c.skinny_gemm_fp8(M, N, K, A, A, A, None, y, None, ws, ws_bytes, None)

    assert call(65, 64) == 3                              # above the decode path
    assert call(12, 64) == 1 and call(64, 65536) == 1     # chunk kernel from 12 rows
    assert call(64, 1 << 20) == 3 and call(17, 1 << 20) == 3  # x chunk would not fit in LDS
    assert call(12, 1 << 20) == 1  # up to 16 rows the matrix-core kernel takes that K
    assert call(17, 7168, y=A, N=4096) == 5               # its split-K workspace is missing
    assert call(12, 7168, y=A, N=4096) == 5
    need = sg.skinny_gemm_fp8_workspace(17, 4096, 7168)
    assert call(17, 7168, y=A, N=4096, ws=A, ws_bytes=need - 256) == 5
    assert call(17, 7168, y=A, N=4096, ws=A + 8, ws_bytes=need) == 4  # misaligned workspace
    assert call(1, 32768) == 1 and call(1, 32784) == 3   # M * K <= 32768 (LDS) at M <= 2
    assert call(2, 16384) == 1 and call(2, 16400) == 3
    assert call(3, 16384) == 1 and call(3, 16400) == 3   # K <= 16384 (registers) at M = 3, 4
    assert call(4, 16384) == 1 and call(4, 16400) == 3
    assert call(5, 8208) == 1 and call(11, 1 << 20) == 1  # matrix-core kernel: any K
    assert call(1, 24) == 4
    assert call(0, 64) == 0
    assert call(4, 16384, y=A + 4) == 4  # misaligned output
    assert sum(sg.skinny_gemm_get_counters()) == 0


def test_lowp_workspace_sizes():
    # fp32 partials [S, N, 16 * ceil(M / 16)] of the low-precision chunk kernel: FP8 from
    # 8 rows (from 12 where N/32 is a whole multiple of 256, and below 12 rows only while
    # its x chunk fits in LDS), MXFP4 from 17 rows, from 12 where a wave takes two
    # tiles (N > 5888) and from 9 where its matrix-core grid is not a multiple of 256
    fp8, mx = sg.skinny_gemm_fp8_workspace, sg.skinny_gemm_mxfp4_workspace
    assert fp8(7, 4096, 7168) == 0 and fp8(8, 4096, 7168) > 0 and fp8(11, 4096, 7168) > 0
    assert fp8(11, 8192, 7168) == 0 and fp8(12, 8192, 7168) > 0 and fp8(8, 8200, 7168) > 0
    assert fp8(9, 5, 1 << 19) == 0  # the matrix-core kernel: no workspace
    assert mx(16, 4096, 7168) == 0 and mx(12, 5889, 7168) > 0 and mx(17, 4096, 7168) > 0
    assert mx(11, 8192, 7168) == 0 and mx(8, 5888, 7168) == 0 and mx(9, 5888, 7168) > 0
    for f in (fp8, mx):
        assert f(65, 4096, 7168) == 0
        assert f(17, 0, 7168) == 0
        assert f(17, 4096, 0) == 0      # K = 0: one launch, no split
        for M, N, K in ((17, 4096, 7168), (32, 8192, 7168), (64, 7168, 8192), (48, 200, 1024),
                        (12, 8192, 7168), (16, 7168, 8192)):
            b = f(M, N, K)
            mp = 16 * -(-M // 16)
            assert b % 256 == 0 and b >= 2 * N * mp * 4, (M, N, K, b)  # at least two splits
            assert (b // (N * mp * 4)) * N * mp * 4 <= b < (b // (N * mp * 4) + 1) * N * mp * 4
    assert fp8(20, 8192, 7168) == mx(20, 8192, 7168)  # one plan for both formats


@no_gpu_only
def test_mxfp4_size_limits_return_before_launch():
    # the vector kernel's team split bounds K (2 blocks of 32 a lane at M <= 2, one
    # from M = 3, at most 8 waves); the matrix-core kernel (M >= 9) takes any K
    c = _raw()
    sg.skinny_gemm_reset_counters()
    A = 0x10000

    def call(M, K):
        return c.skinny_gemm_mxfp4(M, 8, K, A, A, A, None, None, None, None, 0, None)

    assert call(65, 64) == 3
    assert call(17, 64) == 1 and call(64, 65536) == 1 and call(64, 1 << 20) == 3
    assert call(1, 32768) == 1 and call(1, 32800) == 3
    assert call(2, 32768) == 1 and call(2, 32800) == 3
    assert call(3, 16384) == 1 and call(8, 16416) == 3
    assert call(9, 1 << 20) == 1
    assert call(1, 48) == 4
    assert sum(sg.skinny_gemm_get_counters()) == 0


# plans from the C ABI in a fresh interpreter; _lib.py is loaded by path (no torch import)
_TUNE_PROBE = r"""
import ctypes, importlib.util, json, os, sys
spec = importlib.util.spec_from_file_location(
    "sg_lib", os.path.join(sys.argv[1], "skinny_gemm_projection_amd", "_lib.py"))
lib = importlib.util.module_from_spec(spec)
spec.loader.exec_module(lib)
c = lib.load()
out = []
for M, N, K in ((4, 4096, 7168), (20, 4096, 7168), (4, 2048, 7168), (5, 4096, 7168)):
    p = lib.SgPlan()
    assert c.skinny_gemm_plan(M, N, K, ctypes.byref(p)) == 0
    out.append([p.kernel, p.split_k, p.tile_n, p.two_pass])
print(json.dumps(out))
"""


def _plans_with_table(tmp_path, text):
    env = dict(os.environ)
    if text is None:
        env.pop("SKINNY_GEMM_TUNE_TABLE", None)
    else:
        f = tmp_path / "tune.txt"
        f.write_text(text)
        env["SKINNY_GEMM_TUNE_TABLE"] = str(f)
    r = subprocess.run([sys.executable, "-c", _TUNE_PROBE, ROOT], env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return json.loads(r.stdout.strip().splitlines()[-1]), r.stderr


def test_tune_table_file_overrides_the_built_in_choices(tmp_path):
    # the table is read once per process, so each case runs in a fresh interpreter
    default, err = _plans_with_table(tmp_path, None)
    assert err == ""
    tuned, err = _plans_with_table(tmp_path, """# M_lo M_hi N K kernel split tile_n
4 4 4096 7168 2 4 0      # VALU split-K, 4 chunks
20 20 4096 7168 3 16 256 # chunk kernel, 16 splits, 256-row tiles

4 4 2048 7168 1 0 0      # the small-matrix kernel cannot take 4 rows: default plan
""")
    assert err == ""
    assert tuned[0][:2] == [sg.SG_KERNEL_SPLITK_VALU, 4] and tuned[0][3] == 0
    assert tuned[0] != default[0]
    assert tuned[1] == [sg.SG_KERNEL_SPLITK_MFMA, 16, 256, 1] != default[1]
    assert tuned[2] == default[2] and tuned[3] == default[3]


@pytest.mark.parametrize("text", ["4 4 4096 7168 2 4\n",            # six fields
                                  "4 4 4096 7168 2 4 0 9\n",        # eight
                                  "4 4 4096 7168 2 4 0 x\n",        # stray text
                                  "0 4 4096 7168 2 4 0\n",          # M_lo < 1
                                  "4 65 4096 7168 2 4 0\n",         # M_hi > 64
                                  "4 4 4096 7168 9 4 0\n",          # no such kernel
                                  "4 4 4096 7168 2 4 64\n"])        # no such tile width
def test_tune_table_rejects_a_malformed_file(tmp_path, text):
    default, _ = _plans_with_table(tmp_path, None)
    plans, err = _plans_with_table(tmp_path, "20 20 4096 7168 3 16 256\n" + text)
    assert "SKINNY_GEMM_TUNE_TABLE" in err and "file ignored" in err
    assert plans == default   # the good first line is dropped with the rest


def test_tune_table_missing_file_is_ignored(tmp_path):
    default, _ = _plans_with_table(tmp_path, None)
    env = dict(os.environ, SKINNY_GEMM_TUNE_TABLE=str(tmp_path / "absent.txt"))
    r = subprocess.run([sys.executable, "-c", _TUNE_PROBE, ROOT], env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0 and "cannot open" in r.stderr
    assert json.loads(r.stdout.strip().splitlines()[-1]) == default
