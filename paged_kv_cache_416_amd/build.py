"""Build libpkv.so for gfx950 with hipcc (in-tree; the .so sits next to this file)."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpkv.so")

ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no implicit multiply-add fusion: every FMA is written out, so a kernel's rounding
    # does not depend on how the optimiser happened to shape its basic blocks
    "-ffp-contract=off",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
# attention_gqa.hip: uniform branches keep their if/else shape. Structurized, a uniform choice
# between two kinds of load (cached or non-temporal) gains a path through neither, and the
# compiler then counts the fewest loads on every path: its waits also wait for the next tile's
# loads, which drains the load pipeline once per tile.
SOURCE_FLAGS = {"attention_gqa.hip": ["-mllvm", "-structurizecfg-skip-uniform-regions=true"]}
SOURCES = ["errors.cpp", "validate.cpp", "sha256.cpp", "pool.cpp", "sim.cpp", "cache_ops.hip", "attention.hip", "attention_gqa.hip", "prefill.hip", "probe.hip"]


def _compile(src):
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *FLAGS, *SOURCE_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if errs.strip():
        sys.stderr.write(errs + "\n")
    return obj


def build(verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
