"""Build libdflash2.so (the C-ABI library with the gfx950 kernels) in-tree.

    python -m block_speculative_decoding_dflash2_amd.build

Compiles every csrc/*.hip for gfx950 with hipcc (cross-compiles without a
GPU) and links them into block_speculative_decoding_dflash2_amd/libdflash2.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libdflash2.so")
BUILD = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # keep hand-written float code off the packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


# Per-file flags: the selector (and the selector loss, which rescores the
# lattice) must evaluate its float32 sums exactly in the stated order (no
# fused multiply-add).
FILE_FLAGS = {"select_verify.hip": ["-ffp-contract=off"], "losses.hip": ["-ffp-contract=off"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [l for l in res.stdout.splitlines() if "packed-fp32-ops' is not a recognized" not in l]
    if res.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(BUILD, f[:-4] + ".o") for f in srcs]

    def compile_one(i):
        return _run([hipcc, *HIPCC_FLAGS, *FILE_FLAGS.get(srcs[i], []), "-c",
                     os.path.join(CSRC, srcs[i]), "-o", objs[i]])

    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        for log in ex.map(compile_one, range(len(srcs))):
            if verbose and log:
                print(log)
    tmp = OUT + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
