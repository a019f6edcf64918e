"""Compile the gfx950 HIP library libtoktier.so in-tree (next to this file).

    python -m exact_bpe_tokenization_amd.build

Each .hip source is compiled separately (in parallel) with hipcc for gfx950, then linked into one
shared library.  Packed fp32 instructions are disabled (the library computes only integers).
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtoktier.so")
SOURCES = ["pretok.hip", "bpe.hip", "tiles.hip", "added.hip", "toktier.hip", "repair.hip"]
ARCH = "gfx950"


def hipcc():
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def common_flags():
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall", "-Wno-unused-function",
            "-Wno-unused-variable", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", CSRC, "-I", os.path.join(os.path.dirname(HERE), "include")]


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()

    def one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [cc] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with concurrent.futures.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
