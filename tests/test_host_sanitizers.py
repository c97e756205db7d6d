"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(the pages' "Kernel contract", gate 1: sanitizers on the planning code).  The
HIP sources are compiled with the sanitizers on the host side only (the
device code is built as usual and never runs here), and linked with
tests/host/plan_fuzz.cpp, which drives the planning and
argument checks with thousands of random shapes and tile maps, valid and
invalid (no GPU is used and no kernel is launched).  Any sanitizer report, or
a broken plan invariant, fails the test.  CPU only."""
import os
import subprocess

import pytest

from audio_diffusion_transformer_amd import build as BUILD

HERE = os.path.dirname(os.path.abspath(__file__))
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (cmd[:4], r.stdout[-3000:] + r.stderr[-3000:])
    return r


@pytest.fixture(scope="module")
def fuzz_binary(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("no clang++ in /opt/rocm/llvm")
    out = tmp_path_factory.mktemp("san")
    objs = []
    for src in BUILD.hip_sources():
        obj = str(out / (os.path.basename(src) + ".o"))
        host_san = [f for s in SAN for f in ("-Xarch_host", s)]
        _run([BUILD.HIPCC, "-c", f"--offload-arch={BUILD.ARCH}", "-O1", "-g", "-std=c++17",
              "-fPIC", "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", "-I", BUILD.INCLUDE, "-I", BUILD.CSRC] + host_san +
             [src, "-o", obj])
        objs.append(obj)
    drv = str(out / "plan_fuzz.o")
    _run([CLANG, "-c", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", "-I", BUILD.INCLUDE]
         + SAN + [os.path.join(HERE, "host", "plan_fuzz.cpp"), "-o", drv])
    exe = str(out / "plan_fuzz")
    _run([CLANG] + SAN + objs + [drv, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                                 "-o", exe])
    return exe


def test_planning_under_sanitizers(fuzz_binary):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("H3_WS_GUARD", None)
    r = subprocess.run([fuzz_binary, "3000"], capture_output=True, text=True, env=env, timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    assert "0 failures" in report, report[-2000:]
    print(report.strip().splitlines()[-1])


def test_planning_under_sanitizers_with_guard_bands(fuzz_binary):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", H3_WS_GUARD="4096")
    r = subprocess.run([fuzz_binary, "1000"], capture_output=True, text=True, env=env, timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0 and "0 failures" in report, report[-4000:]
