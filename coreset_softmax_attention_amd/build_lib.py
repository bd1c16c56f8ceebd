"""Build libcsa.so (the C-ABI library) from csrc/*.hip with hipcc for gfx950.

Usage: python -m coreset_softmax_attention_amd.build_lib   (or call build()).
Objects go to _build/ at the repository root; the library is written next to
this file, where the Python binding loads it.  The compiler's per-kernel
resource report (registers, scratch, LDS, occupancy) is kept in
_build/kernel_resources.json.
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

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcsa.so")
RESOURCES = os.path.join(BUILD, "kernel_resources.json")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libcsa)")


FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|SGPRs Spill|VGPRs Spill|"
                     r"Occupancy \[waves/SIMD\]|LDS Size \[bytes/block\]): (\S+)")
_FIELDS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch_bytes_per_lane",
           "SGPRs Spill": "sgpr_spills", "VGPRs Spill": "vgpr_spills", "Occupancy [waves/SIMD]": "waves_per_simd",
           "LDS Size [bytes/block]": "static_lds_bytes"}


def parse_resources(stderr: str) -> dict:
    """Per-kernel figures from hipcc's -Rpass-analysis=kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in stderr.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None and val.isdigit():
            cur[_FIELDS[key]] = int(val)
    return out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def compile_one(src: str):
        obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
        cmd = [cc, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{r.stdout}\n{r.stderr}")
        noise = "\n".join(l for l in r.stderr.splitlines()
                          if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l)
        if verbose and noise.strip():
            print(noise, file=sys.stderr)
        return obj, parse_resources(r.stderr)

    with ThreadPoolExecutor(jobs or min(8, os.cpu_count() or 1)) as ex:
        done = list(ex.map(compile_one, sources))
    objs = [o for o, _ in done]
    resources = {}
    for _, res in done:
        resources.update(res)
    with open(RESOURCES, "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
