"""Host code under AddressSanitizer (CPU only, no GPU needed).

Two separate programs, since the oracle and the library are never linked
together:
  - tests/asan/oracle_checks.c with oracle/oracle.c, built by gcc with
    -fsanitize=address: every oracle function on ragged shapes with
    exact-size heap buffers;
  - tests/asan/host_checks.cpp with the library's host sources (api.cpp,
    plan.cpp, moe_step.cpp, noalloc.hip) instrumented for the host only
    (-Xarch_host before each -fsanitize=), linked with the GPU objects of the
    normal build: the planner over some 10 000 shapes, every pre-launch error
    path, and the tuned-table file parser (a valid file, an over-long line).
A report from the sanitizer, or a failed check, fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "skinny_gemm_projection_amd", "csrc")
BUILD = os.path.join(ROOT, "skinny_gemm_projection_amd", "_build")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
GPU_OBJECTS = ["rowdot", "splitk_mfma", "reduce", "moe", "router", "mxfp4", "prefetch", "fp8",
               "lowp_chunk", "probe"]
HOST_SOURCES = ["api.cpp", "plan.cpp", "moe_step.cpp", "noalloc.hip"]
ASAN_ENV = {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0:exitcode=86"}


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def _check_run(exe, env, tag):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600,
                       env=dict(os.environ, **ASAN_ENV, **env))
    assert "AddressSanitizer" not in r.stderr, r.stderr
    assert r.returncode == 0 and f"{tag}: ok" in r.stdout, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_address_sanitizer(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    _run(["gcc", "-std=c99", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "oracle"), os.path.join(ROOT, "tests", "asan", "oracle_checks.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", exe])
    _check_run(exe, {}, "oracle_checks")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_library_host_code_under_address_sanitizer(tmp_path):
    missing = [o for o in GPU_OBJECTS if not os.path.exists(os.path.join(BUILD, o + ".o"))]
    if missing:
        pytest.skip(f"build the library first (python -m skinny_gemm_projection_amd.build): "
                    f"{missing}")
    flags = ["-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fPIC",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = []
    for src in HOST_SOURCES + [os.path.join("..", "..", "tests", "asan", "host_checks.cpp")]:
        obj = str(tmp_path / (os.path.basename(src).split(".")[0] + ".o"))
        _run([HIPCC, "-c", os.path.join(CSRC, src), "-o", obj] + flags)
        objs.append(obj)
    exe = str(tmp_path / "host_checks")
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-o", exe] + objs +
         [os.path.join(BUILD, o + ".o") for o in GPU_OBJECTS])
    _check_run(exe, {}, "host_checks")
    table = tmp_path / "tune.txt"
    table.write_text("# M_lo M_hi N K kernel split tile_n\n4 4 4096 7168 2 4 0\n"
                     "20 64 4096 7168 3 16 256   # chunk kernel\n1 1 1000 1024 1 0 0\n")
    _check_run(exe, {"SKINNY_GEMM_TUNE_TABLE": str(table)}, "host_checks")
    long_line = tmp_path / "long.txt"
    long_line.write_text("4 4 4096 7168 2 4 0 " + "#" * 2000 + "\n")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600,
                       env=dict(os.environ, **ASAN_ENV, SKINNY_GEMM_TUNE_TABLE=str(long_line)))
    assert "AddressSanitizer" not in r.stderr and r.returncode == 0, r.stderr
    assert "file ignored" in r.stderr
