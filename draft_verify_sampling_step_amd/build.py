"""Build the gfx950 library libdspark.so in-tree with hipcc (no JIT, no torch extension).

    python -m draft_verify_sampling_step_amd.build

compiles every csrc/*.hip to an object (in parallel) and links them into
draft_verify_sampling_step_amd/libdspark.so.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdspark.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
ARCH = os.environ.get("DSPARK_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept off (see the build notes of the design document)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", f"-I{INCLUDE}",
]


def _hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in cand or os.path.exists(cand):
            return cand
    return "hipcc"


# Per-file device code generation options.  resident.hip holds W2t in accumulation registers
# and feeds them to the matrix cores as the A operand; with the VGPR form of MFMA its
# accumulators and epilogue stay in ordinary vector registers (no copies between the files).
# loss.hip claims rows with one lane's returning atomic whose value is used an exchange
# later; the atomic optimizer would rewrite it into a wave-wide form that reads the result
# back at once, and so wait for the round trip there.
FILE_FLAGS = {"resident.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "loss.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                     if "is not a recognized feature" not in line and line.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if errs:
        print(errs, file=sys.stderr)
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    res = subprocess.run([_hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
