"""Builds libstepq.so in-tree with hipcc for gfx950.

Flags that matter for the arithmetic: -ffp-contract=off (no multiply-add fusion unless written
as fmaf), no fast-math (IEEE division, denormals kept), and packed FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``; the host pass warns that it does not
know the feature, which is harmless).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libstepq.so")
ARCH = os.environ.get("STEPQ_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++20", f"--offload-arch={ARCH}", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
]


SOURCES = ("stepq_k128_gdn.hip", "stepq_k128_kda.hip", "stepq_k64.hip", "stepq_calib.hip",
           "stepq_noalloc.hip", "stepq_api.cpp", "stepq_offline.cpp")
OBJDIR = os.path.join(HERE, "_build")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\nfailed ({res.returncode}):\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compiles every translation unit in parallel, then links libstepq.so."""
    from concurrent.futures import ThreadPoolExecutor
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJDIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    jobs = []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, src + ".o")
        jobs.append(([hipcc, *flags, *inc, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    with ThreadPoolExecutor(len(jobs)) as ex:
        outs = list(ex.map(lambda j: _run(j[0]), jobs))
    tmp = LIB + ".tmp"
    outs.append(_run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC",
                      *[o for _, o in jobs], "-o", tmp]))
    if verbose:
        for o in outs:
            if o.strip():
                print(o, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


KERNEL_SOURCES = ("stepq_k128_gdn.hip", "stepq_k128_kda.hip", "stepq_k64.hip")


def kernel_resources() -> dict:
    """Compiles the step kernels' units for the device only and returns the compiler's resource
    report per kernel: {mangled name: {"VGPRs", "ScratchSize", "Occupancy", "VGPRs Spill",
    "SGPRs Spill", "LDS Size"}} (integers)."""
    import re
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    flags = [f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory() as td:
        def one(src):
            return _run([hipcc, *flags, *inc, "--cuda-device-only", "-c",
                         "-Rpass-analysis=kernel-resource-usage", os.path.join(CSRC, src),
                         "-o", os.path.join(td, src + ".o")])
        with ThreadPoolExecutor(len(KERNEL_SOURCES)) as ex:
            text = "\n".join(ex.map(one, KERNEL_SOURCES))
    out, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(VGPRs|ScratchSize|Occupancy|VGPRs Spill|SGPRs Spill|LDS Size)"
                      r"(?: \[[^]]*\])?: (\d+)", line)
        if m and cur is not None:
            cur[m.group(1)] = int(m.group(2))
    return out


if __name__ == "__main__":
    print(build(verbose=True))
