"""Build libfa.so for gfx950 with hipcc, in-tree (next to this file).

    python -m io_aware_flashattention_amd.build
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libfa.so")
OBJ = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_fwd_f32.hip", "fa_decode.hip", "fa_bwd.hip", "fa_fp8.hip"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(os.path.dirname(HERE), "include")]
# Packed-FP32 VALU forms are kept out of every device object.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]
# The attention kernels never produce or test NaN (masked scores are -inf and
# infinities stay honoured), so max() needs no NaN-quieting of its inputs.
PER_SOURCE = {"fa_fwd.hip": ["-fno-honor-nans"], "fa_decode.hip": ["-fno-honor-nans"],
              "fa_bwd.hip": ["-fno-honor-nans"]}


# Kernels whose waits count the vector-memory operations still in flight
# (s_waitcnt vmcnt(N) with N > 0, so later tiles stay in flight). Scratch
# spills are vector-memory operations too and would break those counts, so
# the build refuses any of these kernels that uses scratch.
COUNTED_WAITS = ("fwd_pp_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel", "decode_split_kernel")
USAGE = "-Rpass-analysis=kernel-resource-usage"


def scratch_users(remarks: str) -> list[str]:
    """Kernels of COUNTED_WAITS that use scratch, from the compiler's
    resource-usage remarks (a 'Function Name' line, then its 'ScratchSize')."""
    bad, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name is not None:
            if int(m.group(1)) > 0 and any(k in name for k in COUNTED_WAITS):
                bad.append(name)
            name = None
    return bad


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    extra = PER_SOURCE.get(src, [])
    cmd = [HIPCC, *COMMON, *extra, *DEVICE, USAGE, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *COMMON, "-x", "hip", *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    bad = scratch_users(r.stderr)
    if bad:
        raise RuntimeError(f"{src}: kernels with counted vmcnt waits use scratch (register spills): {bad}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
