"""Builds libmk.so (HIP, gfx950) in place next to this file."""
from __future__ import annotations

import json
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmk.so")
SOURCES = [os.path.join(CSRC, n) for n in ("mk_kernels.hip", "mk_allgather.hip", "mk_ring.hip", "mk_api.hip")]
HEADERS = [os.path.join(CSRC, n) for n in ("mk_internal.hpp", "mk_device.hpp", "mk_allgather.hpp", "mk_ring.hpp")] + [os.path.join(ROOT, "include", "mk.h")]

# Packed fp32 instructions are switched off for all device code.  LLVM's
# atomic optimizer is off too: every atomic here is issued by one lane, and the
# optimizer's wave-level rewrite reads each returned value back at once
# (readfirstlane), which waits for every bookkeeping round trip in turn instead
# of letting a task's atomics overlap one another and its stores.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


RESOURCES = LIB[:-3] + ".resources.json"
_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                     r"Occupancy \[waves/SIMD\]|SGPRs Spill|VGPRs Spill|LDS Size \[bytes/block\]):"
                     r"\s+(\S+)")


def _resources(stderr: str) -> dict:
    """Per-kernel register, scratch and occupancy figures from the compiler's
    resource-usage remarks (device pass only)."""
    out, cur = {}, None
    for line in stderr.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key.split(" [")[0]] = int(val)
    return out


def build(verbose: bool = False) -> str:
    """Compile every source into libmk.so; always recompiles.  The kernels'
    register and scratch use goes to libmk.resources.json next to it."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-Rpass-analysis=kernel-resource-usage",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stderr=subprocess.PIPE, text=True)
    # pass the compiler's own diagnostics through, without the remarks
    for line in res.stderr.splitlines():
        if "-Rpass-analysis=kernel-resource-usage" not in line:
            print(line, file=sys.stderr)
    if res.returncode != 0:
        raise subprocess.CalledProcessError(res.returncode, cmd)
    os.replace(tmp, LIB)
    with open(RESOURCES, "w") as f:
        json.dump(_resources(res.stderr), f, indent=1, sort_keys=True)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
