"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

csrc/abi.hip (argument validation, error text, dispatch) is compiled again
with the sanitizers on its host side only (each -fsanitize= behind
-Xarch_host: the device code is not instrumented), linked with the
library's other objects from the in-tree build and the checks in
tests/sanitize/abi_checks.cpp, and run on the CPU: every call is rejected
before a launch or is a size query, and several threads check that each
reads back its own error text.  A sanitizer report or a failed check fails
the test."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "activation_sparse_decode_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
ROCM = "/opt/rocm"


def tool(name):
    for cand in (shutil.which(name), os.path.join(ROCM, "bin", name),
                 os.path.join(ROCM, "llvm", "bin", name)):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.timeout(600)
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    hipcc, clang = tool("hipcc"), tool("clang++")
    objs = [o for o in glob.glob(os.path.join(BUILD, "*.hip.o")) if not o.endswith("abi.hip.o")]
    if not hipcc or not clang or not objs:
        pytest.skip("needs hipcc, clang++ and the in-tree build (_build/*.o)")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    abi_o = str(tmp_path / "abi_san.o")
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        f"-I{os.path.join(ROOT, 'include')}", *san, "-c",
                        os.path.join(CSRC, "abi.hip"), "-o", abi_o],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "abi_checks")
    # host-only link (no .hip source on this line): the sanitizer runtimes
    r = subprocess.run([clang, "-fsanitize=address,undefined", "-O1", "-g", "-std=c++17",
                        f"-I{os.path.join(ROOT, 'include')}",
                        os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp"), abi_o, *objs,
                        f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-lpthread",
                        "-o", exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "ok: 0 failure(s)" in r.stdout
