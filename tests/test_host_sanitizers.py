"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library's sources host-only (an empty device binary embedded: no
kernel is compiled or run) together with `tests/host_abi/abi_check.cpp`,
which calls every size query, the status strings (including ints outside
the enum, through the C translation unit `tests/host_abi/status_c.c`) and
the argument-validation paths of every entry point, and runs it on the CPU.
Any sanitizer report or failed expectation fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_linear_recurrence_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host_abi")
# sanitizers for the host side of the HIP compile only
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def _tool(*cands):
    for c in cands:
        if c and os.path.exists(c):
            return c
    return None


def test_abi_host_code_under_sanitizers(tmp_path):
    hip = _tool(os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc"))
    cc = _tool("/opt/rocm/llvm/bin/clang", "/opt/rocm/lib/llvm/bin/clang")
    if hip is None or cc is None:
        pytest.skip("ROCm compilers not found")
    empty = tmp_path / "empty.gpubin"
    empty.write_bytes(b"")
    shim = tmp_path / "status_c.o"
    exe = tmp_path / "abi_check"
    inc = os.path.join(ROOT, "include")
    r = subprocess.run([cc, "-c", "-x", "c", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                        f"-I{inc}", "-o", str(shim), os.path.join(HOST, "status_c.c")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    cmd = [hip, "--offload-arch=gfx950", "--cuda-host-only", "-Xclang", "-fcuda-include-gpubinary", "-Xclang",
           str(empty), "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", *HOST_SANITIZE, f"-I{inc}", f"-I{CSRC}",
           "-o", str(exe), os.path.join(HOST, "abi_check.cpp"), os.path.join(CSRC, "rglru_scan.hip"),
           os.path.join(CSRC, "rglru_proj.hip"), os.path.join(CSRC, "delta_rule.hip"),
           os.path.join(CSRC, "delta_chunk.hip"), os.path.join(CSRC, "delta_bwd.hip"), f"-Wl,{shim}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "all passed" in r.stdout
