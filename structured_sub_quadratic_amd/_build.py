"""Build the MonarchAttention HIP library in-tree for gfx950.

    python -m structured_sub_quadratic_amd._build

compiles csrc/monarch_attn.hip into structured_sub_quadratic_amd/libmonarch_attn.so
with hipcc (cross-compiles without a GPU).
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(PKG, "csrc", "monarch_attn.hip")
LIB = os.path.join(PKG, "libmonarch_attn.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-shared",
    "-fPIC",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    if verbose:
        noise = "is not a recognized feature for this target"
        for line in (res.stdout + res.stderr).splitlines():
            if noise not in line:
                print(line)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
