"""Build libpagedattn.so for gfx950 in-tree (hipcc; no JIT cache).

    python -m paged_kv_attention_amd.build

Compiles every ``csrc/*.hip`` with hipcc for gfx950, the host-only planning
code with g++, links ``paged_kv_attention_amd/libpagedattn.so`` and writes the
compiler's per-kernel resource report (VGPRs, AGPRs, LDS, scratch = spills)
to ``paged_kv_attention_amd/_build/resource_usage.txt``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpagedattn.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
    # packed FP32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Rpass-analysis=kernel-resource-usage",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC]
# The MFMA kernels take running maxima of scores that are never NaN (keys past
# the context are zero-filled or masked to -inf): without NaN semantics fmaxf
# maps to a bare v_max/v_max3 instead of quieting each operand first.
# Infinities keep their IEEE meaning (the masks rely on -inf).
FILE_FLAGS = {"prefill.hip": ["-fno-honor-nans"], "prefill16.hip": ["-fno-honor-nans"], "decode.hip": ["-fno-honor-nans"],
              "mixed.hip": ["-fno-honor-nans"]}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return r.returncode, r.stdout


def _compile_hip(src: str):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    rc, out = _run([HIPCC, *HIP_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj])
    return src, obj, rc, out


def _resource_summary(log: str) -> str:
    """Keep the per-kernel resource lines of the compiler's remarks."""
    keep = []
    for line in log.splitlines():
        if "remark:" in line and ("Function Name" in line or "VGPRs" in line or "AGPRs" in line
                                  or "ScratchSize" in line or "LDS Size" in line or "Occupancy" in line
                                  or "SGPRs:" in line):
            keep.append(re.sub(r"^.*remark: ", "", line))
    return "\n".join(keep) + "\n"


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs, logs = [], []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        for src, obj, rc, out in ex.map(_compile_hip, srcs):
            logs.append(f"== {os.path.basename(src)}\n{out}")
            if rc != 0:
                sys.stderr.write(out)
                raise RuntimeError(f"hipcc failed on {src}")
            objs.append(obj)
    host_obj = os.path.join(BUILD, "host_logic.o")
    rc, out = _run(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, "host_logic.cpp"), "-o", host_obj])
    if rc != 0:
        sys.stderr.write(out)
        raise RuntimeError("g++ failed on host_logic.cpp")
    tmp = LIB + ".tmp"
    rc, out = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, host_obj])
    if rc != 0:
        sys.stderr.write(out)
        raise RuntimeError("link of libpagedattn.so failed")
    os.replace(tmp, LIB)
    full = "\n".join(logs)
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        f.write(_resource_summary(full))
    if verbose:
        print(_resource_summary(full))
    return LIB


def resource_table(summary: str) -> str:
    """One line per kernel instantiation: VGPRs, AGPRs, scratch bytes per
    lane, LDS bytes per workgroup and waves per SIMD, from the remarks."""
    rows, cur = [], None
    for line in summary.splitlines():
        m = re.match(r"\s*Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            rows.append(cur)
            continue
        m = re.match(r"\s*(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|LDS Size \[bytes/block\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).split()[0]] = int(m.group(2))
    out = [f"{'kernel (mangled)':90s} {'VGPR':>5s} {'AGPR':>5s} {'scratch':>7s} {'LDS':>7s} {'waves/SIMD':>10s}"]
    for r in rows:
        if not r["name"].startswith("_ZN2pa"):
            continue
        out.append(f"{r['name'][:90]:90s} {r.get('VGPRs', 0):5d} {r.get('AGPRs', 0):5d} {r.get('ScratchSize', 0):7d} "
                   f"{r.get('LDS', 0):7d} {r.get('Occupancy', 0):10d}")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    lib = build(verbose="-v" in sys.argv)
    if "--table" in sys.argv:
        with open(os.path.join(BUILD, "resource_usage.txt")) as f:
            print(resource_table(f.read()), end="")
    else:
        print(lib)
