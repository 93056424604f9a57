"""Builds libpkv.so for gfx950 in-tree (hipcc for the HIP sources, gcc for the C allocator).

Run as ``python -m paged_kv_cache_446_amd.build`` or through ``__graft_entry__.build()``.
"""

import concurrent.futures
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
OBJ = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(HERE, "libpkv.so")

ARCH = "gfx950"
HIP_SOURCES = ["attention.hip", "prefill.hip", "cache_ops.hip", "calibrate.hip", "api.cpp"]
C_SOURCES = ["allocator.c", "checks.c"]
# Packed fp32 instructions stay off: ordinary float code only.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Rpass-analysis=kernel-resource-usage",  # per-kernel registers, scratch, LDS (checked below)
    "-I", INCLUDE, "-I", CSRC,
]
RESOURCES = os.path.join(ROOT, "_build", "kernel_resources.json")
C_FLAGS = ["-std=c99", "-O2", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name: harmless, filtered
    out = "\n".join(ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                     r"Occupancy \[waves/SIMD\]|VGPRs Spill|LDS Size \[bytes/block\]):\s+(\S+)")


def _resources(out: str) -> dict:
    """Per-kernel resource remarks of one compile: {kernel: {field: value}}."""
    res, cur = {}, None
    for m in _REMARK.finditer(out):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = res.setdefault(val, {})
        elif cur is not None:
            cur[key.split(" [")[0]] = int(val)
    return res


# Per-source extra flags.  prefill.hip: its maxima never see a NaN (stale slots are
# removed by selection first), so the compiler may drop NaN-quieting before each max.
# The plan kernels add per-thread counts into shared counters: an atomic add whose
# address is the same for the whole wavefront is combined across the wavefront with
# DPP row operations, not with a scalar loop over the active lanes (one readlane and
# one LDS wait per lane).
ATOMIC_DPP = ["-mllvm", "-amdgpu-atomic-optimizer-strategy=DPP"]
EXTRA_FLAGS = {"prefill.hip": ["-fno-honor-nans"] + ATOMIC_DPP, "attention.hip": ATOMIC_DPP}


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        jobs.append([hipcc] + HIP_FLAGS + EXTRA_FLAGS.get(src, []) + lang +
                    ["-c", os.path.join(CSRC, src), "-o", obj])
    for src in C_SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
        jobs.append(["gcc"] + C_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    # every kernel keeps its values in registers: per-lane scratch memory (spills or a
    # private array the compiler could not promote) would add memory traffic unseen in
    # the source, so it fails the build
    resources = {}
    for o in outs:
        resources.update(_resources(o))
    with open(RESOURCES, "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    scratch = {k: v["ScratchSize"] for k, v in resources.items() if v.get("ScratchSize")}
    if scratch:
        raise RuntimeError(f"kernels using scratch memory (bytes per lane): {scratch}")
    if verbose:
        for o in outs:
            if o.strip() and "remark:" not in o:
                print(o)
    objs = [os.path.join(OBJ, os.path.splitext(s)[0] + ".o") for s in HIP_SOURCES + C_SOURCES]
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
