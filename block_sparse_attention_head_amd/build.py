"""Build libmsa.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m block_sparse_attention_head_amd.build          # build
    python -m block_sparse_attention_head_amd.build --check  # build, then list missing exports

hipcc cross-compiles for gfx950 without a GPU present.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import re
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_ROOT, "include")
BUILD_DIR = os.path.join(REPO_ROOT, "_build", "libmsa")
LIB_PATH = os.path.join(PKG_DIR, "libmsa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CXXFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    f"-I{INCLUDE}",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Per-source extra flags. The index max-pool and the selection's lane maxima
# never need NaN quieting, so their fmaxf chains compile to plain v_max_f32
# instead of canonicalise + max.
EXTRA_FLAGS = {
    "k_index_pool.hip": ["-fno-honor-nans"],
    "k_block_topk.hip": ["-fno-honor-nans"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CXXFLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; that is expected.
    noise = re.compile(r"'-packed-fp32-ops' is not a recognized feature|warnings? generated when compiling for host")
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if not noise.search(l))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if msgs.strip():
        sys.stderr.write(msgs + "\n")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link libmsa.so next to this file. Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


def declared_symbols(header: str = os.path.join(INCLUDE, "msa.h")):
    """Function names declared in the public header."""
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(msa_\w+)\s*\(", text, flags=re.M)))


def exported_symbols(lib: str = LIB_PATH):
    out = subprocess.run(["nm", "-D", "--defined-only", lib], capture_output=True, text=True, check=True).stdout
    return sorted({l.split()[-1] for l in out.splitlines() if l.strip()})


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--check", action="store_true")
    a = ap.parse_args(argv)
    build(verbose=True)
    if a.check:
        missing = sorted(set(declared_symbols()) - set(exported_symbols()))
        print("missing exports:", missing or "none")
        return 1 if missing else 0
    return 0


if __name__ == "__main__":
    sys.exit(main())
