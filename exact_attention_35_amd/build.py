"""Build libfa.so (the C-ABI library with the gfx950 kernels) in-tree with hipcc.

Every .hip file under csrc/ is compiled for gfx950 only, in parallel, then linked
into exact_attention_35_amd/libfa.so. Packed fp32 instructions are disabled for
all device code (-target-feature -packed-fp32-ops). The compiler's per-kernel resource
report (registers, spills, scratch, occupancy) is written to _build/kernel_resources.json.
"""

from __future__ import annotations

import glob
import json
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfa.so")
BUILD = os.path.join(ROOT, "_build")

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-Rpass-analysis=kernel-resource-usage",
]
REPORT = os.path.join(BUILD, "kernel_resources.json")
_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|VGPRs Spill|SGPRs Spill|ScratchSize \[bytes/lane\]|"
                     r"Occupancy \[waves/SIMD\]|LDS Size \[bytes/block\]): (\S+)")


def _resources(stderr: str) -> dict:
    """Per-kernel fields of the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for ln in stderr.splitlines():
        m = _REMARK.search(ln)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key] = int(val) if val.lstrip("-").isdigit() else val
    return out


def _compile(src: str, verbose: bool) -> tuple[str, dict]:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, f"-I{INCLUDE}", f"-I{CSRC}", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"compilation failed: {src}")
    # hipcc's host pass does not know the device-only feature: drop that one warning; the
    # resource remarks go to the report
    noise = [ln for ln in r.stderr.splitlines() if ln.strip() and "packed-fp32-ops" not in ln
             and "warning generated" not in ln and "warnings generated" not in ln
             and "kernel-resource-usage" not in ln]
    if noise and verbose:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj, _resources(r.stderr)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        done = list(ex.map(lambda s: _compile(s, verbose), srcs))
    objs = [o for o, _ in done]
    report = {}
    for _, res in done:
        report.update(res)
    with open(REPORT, "w") as f:
        json.dump(report, f, indent=1, sort_keys=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
