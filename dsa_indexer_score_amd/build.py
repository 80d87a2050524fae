"""Build libdsa_indexer.so (HIP for gfx950) in-tree with hipcc."""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libdsa_indexer.so")
SOURCES = ["score_select.hip", "score_rows.hip", "screen_cert.hip", "select_few.hip",
           "pair_overlap.hip", "noalloc.hip", "indexer_api.cpp"]

# Per-file extra flags.  The scoring kernel assumes finite inputs (a documented
# precondition), so IEEE NaN quieting is switched off there: ReLU then lowers
# to a single v_max_f32 instead of a canonicalising max followed by the max.
_NO_NAN = ["-fno-honor-nans", "-Xclang", "-mno-amdgpu-ieee"]
FILE_FLAGS = {"score_select.hip": _NO_NAN, "score_rows.hip": _NO_NAN}

# Packed fp32 VALU ops are kept out of the generated code.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC]


def source_hash() -> str:
    """Hash of everything the library is compiled from: the kernel and host
    sources, the public header and the compile flags.  Built into the
    library (indexer_source_hash) so that a library built from other
    sources is refused at load time."""
    h = hashlib.sha256()
    files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h", ".cpp")))
    for path in [os.path.join(CSRC, f) for f in files] + [os.path.join(INCLUDE, "dsa_indexer.h")]:
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as fh:
            h.update(fh.read())
    flags = [f for f in HIP_FLAGS if f not in (INCLUDE, CSRC)]      # paths differ between trees
    h.update(repr((flags, sorted(FILE_FLAGS.items()))).encode())
    return h.hexdigest()[:16]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    tag = source_hash()

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *HIP_FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
            cmd.insert(-4, f'-DDSAI_SOURCE_HASH="{tag}"')
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
        if verbose:
            sys.stderr.write(res.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    res = subprocess.run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
