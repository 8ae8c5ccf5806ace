"""Build the MonarchAttention HIP library in-tree for gfx950.

    python -m structured_sub_quadratic_amd._build

compiles the translation units under csrc/ (the C ABI and one launch unit per
element type and head dimension) in parallel with hipcc (cross-compiles
without a GPU) and links structured_sub_quadratic_amd/libmonarch_attn.so.
"""

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmonarch_attn.so")
BUILD = os.path.join(PKG, "_build")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
NOISE = "is not a recognized feature for this target"


def hipcc():
    env = os.environ.get("HIPCC")
    if env:
        return env
    return "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if NOISE not in l)
    return res.returncode, out, cmd


def build(verbose=False, extra_flags=(), out=LIB):
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs, cmds = [], []
    for src in sources:
        obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        cmds.append([hipcc(), *HIPCC_FLAGS, *extra_flags, "-c", src, "-o", obj])
    workers = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(_run, cmds))
    for rc, text, cmd in results:
        if rc != 0:
            sys.stderr.write(text + "\n")
            raise RuntimeError(f"hipcc failed ({rc}): {' '.join(cmd)}")
        if verbose and text.strip():
            print(text)
    tmp = out + ".tmp"
    rc, text, cmd = _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    if rc != 0:
        sys.stderr.write(text + "\n")
        raise RuntimeError(f"link failed ({rc}): {' '.join(cmd)}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    flags = [a for a in sys.argv[1:] if a.startswith("-D")]
    outs = [a[len("--out="):] for a in sys.argv[1:] if a.startswith("--out=")]
    print(build(verbose=True, extra_flags=flags, out=outs[0] if outs else LIB))
