"""Build libpagedkv.so (HIP C++ for gfx950) in place, next to this file.

    python -m paged_kv_cache_63_amd.build

Compiles every ``csrc/*.hip`` with hipcc for gfx950 into ``_build/`` at the
repository root and links them into ``paged_kv_cache_63_amd/libpagedkv.so``.
Always recompiles (a few seconds per file).
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpagedkv.so")
OBJ_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-mcode-object-version=5",
    # no packed fp32 instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# The attention kernels never let a NaN reach a max or an exponential (masked
# scores are replaced by -inf by index before use), so they are built without
# NaN-preserving min/max semantics (no quieting instruction per operand).
PER_FILE = {
    "decode.hip": ["-fno-honor-nans"],
    "extend.hip": ["-fno-honor-nans"],
}


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *PER_FILE.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    # A kernel whose host-side stub was not emitted links fine but fails at
    # load time; refuse such a library here.
    r = subprocess.run(["nm", "-D", "--undefined-only", "-C", tmp], capture_output=True, text=True)
    missing = [l.strip() for l in r.stdout.splitlines() if "pkv::" in l]
    if missing:
        os.remove(tmp)
        raise RuntimeError("library has undefined symbols of its own:\n" + "\n".join(missing))
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
