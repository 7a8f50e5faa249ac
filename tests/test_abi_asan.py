"""The C ABI's argument validation under AddressSanitizer, without a GPU.

libmoe4_asan.so is the library's host code built with ASan and no device code
(bit_mixture_experts_amd/build.py, build_asan). A child interpreter loads it in
place of libmoe4.so, with the ASan runtime preloaded, and runs the CPU ABI
tests: every refusal path reads the caller's descriptors and sizes, and any
out-of-bounds or use-after-free read there ends the child with an ASan
report."""
import glob
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

LIB = os.path.join(ROOT, "bit_mixture_experts_amd", "libmoe4_asan.so")


def _asan_runtime():
    pats = ["/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
            "/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"]
    for p in pats:
        hits = sorted(glob.glob(p))
        if hits:
            return hits[-1]
    return None


def test_abi_validation_runs_clean_under_asan():
    assert os.path.exists(LIB), ("libmoe4_asan.so is not built: "
                                 "__graft_entry__.build() builds it with libmoe4.so")
    runtime = _asan_runtime()
    assert runtime, "the ROCm clang ASan runtime (libclang_rt.asan-x86_64.so) is missing"
    env = dict(os.environ)
    env["MOE4_LIB_PATH"] = LIB
    # keep whatever the environment preloads, after the ASan runtime
    env["LD_PRELOAD"] = ":".join(p for p in (runtime, env.get("LD_PRELOAD", "")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:exitcode=86:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout


def test_asan_build_is_the_library_the_child_loads():
    """The override names the ASan build (its undefined ASan hooks prove it is
    instrumented), so the run above did not test libmoe4.so by accident."""
    if not os.path.exists(LIB):
        pytest.fail("libmoe4_asan.so is not built")
    r = subprocess.run(["nm", "-D", "--undefined-only", LIB], capture_output=True, text=True)
    assert r.returncode == 0 and "__asan_" in r.stdout
    probe = ("import os, bit_mixture_experts_amd.moe4 as m; "
             "print(os.path.realpath(m.LIB_PATH))")
    runtime = _asan_runtime()
    env = dict(os.environ, MOE4_LIB_PATH=LIB, ASAN_OPTIONS="detect_leaks=0",
               LD_PRELOAD=":".join(p for p in (runtime, os.environ.get("LD_PRELOAD", "")) if p))
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().endswith("libmoe4_asan.so")
