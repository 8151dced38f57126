"""Builds libwanvae.so in-tree with hipcc for gfx950.

    python -m causal_convolution_amd.build

Each HIP source is compiled separately (in parallel) and linked into one
shared library next to this file.  All device code is compiled with packed
FP32 instructions disabled (``-packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libwanvae.so")
SOURCES = ["abi.cpp", "rmsnorm_silu.hip", "conv3d_f32.hip", "conv3d_bf16.hip", "pack_weights.hip",
           "pointwise.hip", "attention.hip", "gemm_bf16.hip",
           "conv3d_narrow.hip", "stream_copy.hip", "cache_io.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++20", "-fPIC", "-fvisibility=hidden", f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"

# Per-source device flags.  conv3d_narrow.hip: the narrow conv's row loop
# (10 input rows per tile) must unroll fully so its accumulators stay in
# registers (their row index is the loop's); with the fused input norm the
# body outgrows the default limit for a requested full unroll, and the
# accumulators would go to scratch (which check_resources rejects).
EXTRA = {"conv3d_narrow.hip": ["-mllvm", "-pragma-unroll-threshold=200000"]}


def check_resources(src: str, remarks: str) -> None:
    """Fails the build if a kernel of `src` spills vector registers or uses
    scratch memory: every kernel here is meant to keep its working set in
    registers and LDS, and scratch traffic in an MFMA loop costs an order of
    magnitude.  A few scalar-register spills are tolerated (up to 64): they go
    to lanes of a vector register, not to memory (the scratch size, checked
    too, stays 0)."""
    bad, name = [], "?"
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"(ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill): (\d+)", line)
        if m and int(m.group(2)) > 0 and not (m.group(1) == "SGPRs Spill" and int(m.group(2)) <= 64):
            bad.append(f"{name}: {m.group(1)} = {m.group(2)}")
    if bad:
        raise RuntimeError(f"{src}: kernels spill or use scratch:\n" + "\n".join(bad))


def _compile(src: str, verbose: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJDIR, src + ".o")
    cmd = [HIPCC] + COMMON + DEVICE + EXTRA.get(src, []) + [RESOURCE_REMARKS, "-c", path, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + COMMON + ["-x", "hip"] + DEVICE + ["-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("is not a recognized feature for this target", "kernel-resource-usage")
    out = r.stdout + r.stderr
    msgs = "\n".join(l for l in out.splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if msgs.strip() and verbose:
        print(msgs)
    if src.endswith(".hip"):
        check_resources(src, out)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
