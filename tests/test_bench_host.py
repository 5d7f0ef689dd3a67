"""Host logic of bench.py that runs without a GPU: the sweep journal (JSON lines,
section by section, resumable), the multi-GPU refusal and the low-precision plan
labels."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_journal_appends_sections_and_resumes(tmp_path):
    path = str(tmp_path / "sweep.jsonl")
    j = bench.SweepJournal(path)
    assert j.done == {}
    j.write("a", [{"workload": "a", "M": 1, "us": 2.0}, {"workload": "a", "M": 2, "us": 3.0}])
    j.write("b", [{"workload": "b", "M": 1, "us": 4.0}])
    # a run killed inside section c: one row written, no section marker, a cut line
    with open(path, "a") as f:
        f.write(json.dumps({"workload": "c", "M": 1, "us": 5.0}) + "\n")
        f.write('{"workload": "c", "M"')
    j2 = bench.SweepJournal(path)
    assert list(j2.done) == ["a", "b"]
    assert [r["M"] for r in j2.done["a"]] == [1, 2] and j2.done["b"][0]["us"] == 4.0
    # the file now holds the complete sections only, and c can be appended again
    with open(path) as f:
        lines = [json.loads(x) for x in f]
    assert lines[-1] == {"section_done": "b"} and len(lines) == 5
    j2.write("c", [{"workload": "c", "M": 1, "us": 5.5}])
    assert list(bench.SweepJournal(path).done) == ["a", "b", "c"]


def test_lowp_plan_labels_follow_the_library_routing():
    import skinny_gemm_projection_amd as sg
    for M in range(1, 65):
        for N in (4096, 5888, 5889, 8192):
            K = 7168
            f8 = bench.lowp_plan_label("fp8", M, N, sg.skinny_gemm_fp8_workspace(M, N, K))
            mx = bench.lowp_plan_label("mxfp4", M, N, sg.skinny_gemm_mxfp4_workspace(M, N, K))
            # the chunk kernel is exactly where a workspace is needed at these shapes
            assert f8.startswith("lowp_chunk") == (sg.skinny_gemm_fp8_workspace(M, N, K) > 0)
            assert mx.startswith("lowp_chunk") == (sg.skinny_gemm_mxfp4_workspace(M, N, K) > 0)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_headline_kernel_tags_name_built_kernels():
    """The kernel names bench.py looks for in rocprofv3 output (traffic and
    trace summaries) are instantiations the library holds, and the headline
    plan is the streaming kernel with one wave a row."""
    import shutil
    import skinny_gemm_projection_amd as sg
    from skinny_gemm_projection_amd import _lib
    nm = shutil.which("nm")
    if nm is None:
        import pytest
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-C", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    for tag in bench.GEMV_KERNEL_TAGS:
        assert f"sg::(anonymous namespace)::{tag}(" in out, tag
    for M in (1, 2):
        p = sg.skinny_gemm_plan(M, bench.N_MAIN, bench.K_MAIN)
        assert p.kernel == sg.SG_KERNEL_GEMV and p.split_k == 1 and p.tile_n == 1
