"""Build libtilemix.so in-tree with hipcc for gfx950.

Every HIP/C++ source under csrc/ is compiled to an object in parallel and the
objects are linked into ``mixed_precision_amd/libtilemix.so``.  Always rebuilds
(the caller decides when); objects go to ``mixed_precision_amd/_build``.  The
compiler's per-kernel resource figures (VGPRs, spills, scratch, occupancy,
LDS) are kept in ``mixed_precision_amd/kernel_resources.json``.  The
microbenchmarks under probe/ become ``libtilemix_probe.so`` (not part of the
attention path).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import json
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtilemix.so")
PROBE_DIR = os.path.join(HERE, "probe")
PROBE_LIB = os.path.join(HERE, "libtilemix_probe.so")

ARCH = os.environ.get("TILEMIX_ARCH", "gfx950")

CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
] + os.environ.get("TILEMIX_EXTRA_FLAGS", "").split()

# flags for single sources: the 3-heads-per-item attention kernels schedule
# for instruction-level parallelism (measured faster there; slower at 2 heads)
SOURCE_FLAGS = {
    "attn_d128_qb3.hip": ["-mllvm", "--amdgpu-sched-strategy=max-ilp"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


RESOURCES = os.path.join(HERE, "kernel_resources.json")
_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|"
                     r"VGPRs Spill|SGPRs Spill|LDS Size \[bytes/block\]):\s+(\S+)")


def _resources(stderr: str):
    """Per-kernel register, spill, scratch, occupancy and LDS figures from the
    compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for key, val in _REMARK.findall(stderr):
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key.split(" [")[0]] = int(val) if val.isdigit() else val
    return out


def _compile(src: str):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + CXXFLAGS + SOURCE_FLAGS.get(os.path.basename(src), []) + \
        ["-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, _resources(r.stderr)


def _link(objs, out: str):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    probe_srcs = sorted(glob.glob(os.path.join(PROBE_DIR, "*.hip")))
    jobs = jobs or min(len(srcs) + len(probe_srcs), max(1, (os.cpu_count() or 4)), 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        probe_done = ex.map(_compile, probe_srcs)
        done = list(ex.map(_compile, srcs))
        probe_objs = [o for o, _ in probe_done]
    objs = [o for o, _ in done]
    res = {}
    for _, r in done:
        res.update(r)
    with open(RESOURCES, "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
    _link(objs, LIB)
    _link(probe_objs, PROBE_LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources (and {os.path.basename(PROBE_LIB)})", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
