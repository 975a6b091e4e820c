"""Compile the gfx950 HIP library ``libvdit_attn.so`` in-tree with hipcc."""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libvdit_attn.so")
SOURCES = ["attn_fwd.hip", "attn_resident.hip", "prepass.hip", "vsa.hip", "api.hip", "noalloc.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the softmax reads the scores with VALU, and the
    # loop-invariant q fragments and load staging then go to AGPRs instead
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


# Kernels whose registers must never spill to scratch memory: an outlined helper
# or a spill moves their score and accumulator arrays into scratch and costs an
# order of magnitude, with correct results, so the build rejects it.
NO_SCRATCH_SOURCES = ["attn_fwd.hip", "attn_resident.hip", "prepass.hip", "vsa.hip"]


def _scratch_users(asm: str) -> list[str]:
    """Kernels whose code-object metadata asks for private (scratch) memory."""
    users = []
    for block in asm.split("\n  - ")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        size = re.search(r"\.private_segment_fixed_size:\s+(\d+)", block)
        if name and size and int(size.group(1)) > 0:
            users.append(f"{name.group(1)} ({size.group(1)} bytes per lane)")
    return users


_DMA = re.compile(r"^\s*global_load_lds_dwordx4\s+(\S+),\s*(\S+)")


def _dma_hazards(asm: str) -> list[str]:
    """Direct global->LDS loads written as inline assembly bypass the compiler's
    hazard recognizer, so the build checks the form the kernels rely on: the
    global address in a VGPR pair with no SGPR base ("off"), and the load
    immediately preceded by an s_nop (the wait state after M0 is written)."""
    bad = []
    lines = asm.splitlines()
    for i, line in enumerate(lines):
        m = _DMA.match(line)
        if not m:
            continue
        addr, base = m.group(1), m.group(2)
        prev = lines[i - 1].strip() if i > 0 else ""
        if not re.fullmatch(r"v\[\d+:\d+\]", addr) or base != "off" or not prev.startswith("s_nop"):
            bad.append(f"line {i + 1}: {prev!r} / {line.strip()!r}")
    return bad


def build(verbose: bool = False) -> str:
    """Compile every source into the shared library; returns its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *srcs, "-o", tmp]
    with tempfile.TemporaryDirectory() as td:
        # device assembly of the hot kernels, compiled alongside, for the scratch check
        checks = []
        for name in NO_SCRATCH_SOURCES:
            asm = os.path.join(td, name + ".s")
            flags = [f for f in HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
            acmd = [hipcc(), *flags, "--cuda-device-only", "-S", f"-I{INCLUDE}", f"-I{CSRC}",
                    os.path.join(CSRC, name), "-o", asm]
            checks.append((asm, subprocess.Popen(acmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed ({res.returncode}) building {LIB}")
        for asm, proc in checks:
            out, err = proc.communicate()
            if proc.returncode != 0:
                sys.stderr.write(out + err)
                raise RuntimeError(f"hipcc failed ({proc.returncode}) compiling {asm} for the scratch check")
            with open(asm) as f:
                text = f.read()
            users = _scratch_users(text)
            if users:
                raise RuntimeError("kernels use scratch memory (spills or outlined helpers): " + "; ".join(users))
            hazards = _dma_hazards(text)
            if hazards:
                raise RuntimeError(f"direct loads in {os.path.basename(asm)} not in the checked form: " +
                                   "; ".join(hazards[:5]))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
