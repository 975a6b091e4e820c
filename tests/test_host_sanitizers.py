"""The C-ABI host code (validation, handle registry, status strings) built for the
host alone with AddressSanitizer and UndefinedBehaviorSanitizer, and driven through
every path that returns before a kernel launch (tests/sanitize/abi_host_check.cpp;
the launchers are test stand-ins that fail if reached). Runs on the CPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_sequence_attention_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")
# sanitizers for the host compilation only: the device compiler takes none
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]


@pytest.mark.timeout(600)
def test_abi_host_code_under_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not found")
    srcs = {
        "main": os.path.join(ROOT, "tests", "sanitize", "abi_host_check.cpp"),
        "stubs": os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
        "api": os.path.join(CSRC, "api.hip"),
    }
    objs = []
    for name, src in srcs.items():
        obj = str(tmp_path / f"{name}.o")
        cmd = [HIPCC, "-x", "hip", "--cuda-host-only", "-O1", "-g", "-std=c++17", *HOST_SAN,
               f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    exe = str(tmp_path / "abi_host_check")
    link = [CLANG, "-fsanitize=address,undefined", *objs, f"-L{ROCM}/lib", "-lamdhip64",
            f"-Wl,-rpath,{ROCM}/lib", "-o", exe]
    r = subprocess.run(link, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "ok: 0 failure(s)" in r.stdout, (r.stdout[-3000:], r.stderr[-3000:])
