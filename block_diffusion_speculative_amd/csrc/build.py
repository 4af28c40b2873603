"""Builds libdflash.so (gfx950) in-tree with hipcc.

    python -m block_diffusion_speculative_amd.csrc.build [--jobs N]

Every translation unit is compiled with packed-fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host passes warn
that they do not know the feature, which is harmless.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
SOURCES = ["gemm.hip", "gemm_tiled.hip", "attention.hip", "misc.hip", "sampling.hip", "tree.hip", "api.hip", "noalloc.hip"]
LIB = os.path.join(PKG, "libdflash.so")
ARCH = os.environ.get("DFLASH_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"]


def source_files():
    """Every file the library is built from: the HIP sources and headers of
    this folder and the public header."""
    names = sorted(f for f in os.listdir(HERE) if f.endswith((".hip", ".hpp")))
    return [os.path.join(HERE, f) for f in names] + [os.path.join(ROOT, "include", "dflash.h")]


def source_digest() -> str:
    """sha256 over the build flags and the name and bytes of every source
    file; the library reports the digest it was built from
    (dflash_build_id), so a stale build is detected before it is used."""
    import hashlib
    # flags without absolute paths (the tree may move between build and use)
    flags = [os.path.relpath(f, ROOT) if f.startswith(ROOT) else f for f in COMMON]
    h = hashlib.sha256(" ".join(flags).encode())
    for path in source_files():
        h.update(os.path.relpath(path, ROOT).encode())
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _compile(src: str, obj_dir: str, digest: str) -> str:
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, f'-DDFLASH_SOURCE_DIGEST="{digest}"', "-c", os.path.join(HERE, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 4, verbose: bool = False) -> str:
    obj_dir = os.path.join(PKG, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    digest = source_digest()
    with ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, digest), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    args = ap.parse_args(argv)
    build(args.jobs, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
