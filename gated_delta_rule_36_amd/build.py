"""Build the GDN-2 HIP library (libgdn2.so) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import hashlib
import json
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libgdn2.so")
BUILD = os.path.join(ROOT, "_build")
# what the last build was made from (not tracked: a built artefact, like the library)
BUILD_INFO = os.path.join(PKG, "build_info.json")

SOURCES = ["gdn2_api.cpp", "gdn2_chunk.hip", "gdn2_split.hip", "gdn2_bwd.hip", "gdn2_decode.hip",
           "gdn2_block.hip", "gdn2_noalloc.hip",
           "gdn2_fwd.hip", "gdn2_recurrent.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def source_digest() -> str:
    """Digest of the library's sources and public header (identifies a build)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    with open(os.path.join(ROOT, "include", "gdn2.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def _git(*args):
    try:
        r = subprocess.run(["git", "-C", ROOT, *args], capture_output=True, text=True, timeout=10)
    except (OSError, subprocess.SubprocessError):
        return None
    return r.stdout.strip() if r.returncode == 0 else None


def _write_build_info():
    """Record the commit the build was made from, so that a copy of the tree without its
    git metadata can still name it, together with the source digest it applies to."""
    sha = _git("rev-parse", "HEAD") or None
    status = _git("status", "--porcelain", "--untracked-files=no", "--", "gated_delta_rule_36_amd",
                  "include")
    info = {"git_sha": sha, "library_sources_committed": None if status is None else status == "",
            "source_sha256": source_digest()}
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libgdn2.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [_hipcc(), *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    _write_build_info()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
