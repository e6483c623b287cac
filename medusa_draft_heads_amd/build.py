"""Builds libmedusa.so in place with hipcc for gfx950 (CDNA4)."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmedusa.so")
BUILD = os.path.join(ROOT, "_build", "libmedusa")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # keep the compiler from forming packed FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "api.cpp")]


# Per-file flags. The vocabulary GEMM keeps 128 accumulators a lane; with the
# MFMA accumulators in ordinary VGPRs the register allocator leaves them in
# place instead of copying them between register files every K step.
FILE_FLAGS = {
    "heads_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}

# Files whose staged pipelines wait for a counted number of outstanding vector
# memory operations (s_waitcnt vmcnt(n) with n the loads a stage issues). A
# register spill would add scratch loads and stores to that count, so these
# files must build without scratch: the compiler's resource remarks are read
# and any kernel with a nonzero scratch size fails the build.
NO_SCRATCH = ("heads_mfma.hip", "attention.hip")


def _scratch_kernels(remarks: str):
    bad, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            bad.append((name, int(m.group(1))))
    return bad


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    base = os.path.basename(src)
    cmd = [HIPCC] + FLAGS + FILE_FLAGS.get(base, []) + ["-c", src, "-o", obj]
    if base in NO_SCRATCH:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    if base in NO_SCRATCH:
        bad = _scratch_kernels(r.stderr)
        if bad:
            raise RuntimeError("%s: kernels with counted memory waits use scratch (spills): %s" % (base, bad))
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, sources()))
    tmp = OUT + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "-shared", "--offload-arch=" + ARCH, "-o", tmp] + objs, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
