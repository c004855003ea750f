"""Build libspecverify.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libspecverify.so")
SOURCES = ["sv_api.hip", "sv_chain.hip", "sv_chain_small.hip", "sv_greedy.hip", "sv_tree.hip", "sv_fanout.hip", "sv_cache.hip", "sv_presto.hip", "sv_branch.hip", "sv_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # explicit fmaf where a fused multiply-add is meant; nothing else contracts
    "-ffp-contract=off",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


LIB_TIMELINE = os.path.join(HERE, "libspecverify_timeline.so")


def build(verbose: bool = False, timeline: bool = False) -> str:
    """Build the library; timeline=True builds the measurement variant with per-block wall-clock stamps
    (libspecverify_timeline.so, -DSV_TIMELINE) beside it."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    lib = LIB_TIMELINE if timeline else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, *(["-DSV_TIMELINE"] if timeline else []), "-I" + os.path.join(ROOT, "include"), *srcs,
           "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, timeline="--timeline" in sys.argv[1:]))
