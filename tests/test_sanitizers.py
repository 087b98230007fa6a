"""Sanitizer tier (CPU): the C oracle and the host side of libkvq's C ABI built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven over every supported format.

  - tests/sanitize/oracle_check.c includes the oracle and runs its quantizers, append / flush
    state machine, fp64 attention and byte-image packing over every format family with every
    buffer allocated to its exact size (gcc, -fsanitize=address,undefined plus float-cast and
    float-divide checks).
  - tests/sanitize/host_abi_check.cpp links kvq_host.hip (host code instrumented; the device
    code is not) with stand-ins for the kernel launchers that check, on the host, that every
    launch configuration stays inside the workspace it was sized for, over 2,000+ formats and
    a spread of batch, head, query and token counts; argument errors must launch nothing.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"


def run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, f"{' '.join(cmd[:3])}... failed ({r.returncode}):\n{out[-4000:]}"
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    run(["gcc", "-O1", "-g", "-std=c99", "-ffp-contract=off", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined,float-cast-overflow,float-divide-by-zero",
         "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "oracle"),
         os.path.join(ROOT, "tests", "sanitize", "oracle_check.c"), "-o", exe, "-lm"])
    out = run([exe])
    assert out.strip().endswith("ok")


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs hipcc")
def test_host_abi_under_address_and_ub_sanitizers(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "quantized_kv_cache_07_amd", "csrc")]
    # host code instrumented, device code not: each sanitizer option goes to the host pass only
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
              "-Xclang", "-packed-fp32-ops", *host_san, *inc]
    o1, o2 = str(tmp_path / "host.o"), str(tmp_path / "check.o")
    run([HIPCC, *common, "-c", os.path.join(ROOT, "quantized_kv_cache_07_amd", "csrc", "kvq_host.hip"),
         "-o", o1])
    run([HIPCC, *common, "-x", "hip", "-c", os.path.join(ROOT, "tests", "sanitize", "host_abi_check.cpp"),
         "-o", o2])
    exe = str(tmp_path / "host_abi_check")
    run([CLANG, "-fsanitize=address,undefined", o1, o2, "-L/opt/rocm/lib", "-lamdhip64",
         "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    out = run([exe], env=env)
    assert "ok (" in out and "runtime error" not in out, out[-2000:]
