"""Build the gfx950 KDA library (libkda_mi355x.so) in-tree with hipcc.

Usage: python -m kimi_delta_attention_03_amd.build [--jobs N]
Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled (see the flags below), then linked into one shared
library next to this file.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB_NAME = "libkda_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["kda_api.cpp", "kda_stage12.hip", "kda_stage34.hip", "kda_varlen.hip", "kda_layer.hip",
           "kda_decode.hip", "kda_bwd.hip", "kda_validate.hip",
           "kda_noalloc.hip", "kda_gemm.hip"]
LIBS = ["-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # no v_pk_{add,mul,fma}_f32 selection (device feature; host pass warns and ignores it)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the KDA library)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if msg.strip():
        sys.stderr.write(msg + "\n")
    return obj


def _write_build_info():
    """Record which sources the library was built from (commit, dirty flag, source hash)
    next to it, so that measurements made from a copy of the tree without git can
    name their provenance."""
    import hashlib
    import json
    import time
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        h.update(name.encode())
        h.update(open(os.path.join(CSRC, name), "rb").read())
    for name in sorted(os.listdir(INCLUDE)):
        h.update(open(os.path.join(INCLUDE, name), "rb").read())
    commit, dirty = None, None
    try:
        root = os.path.dirname(HERE)
        r = subprocess.run(["git", "-C", root, "rev-parse", "--short=12", "HEAD"], capture_output=True, text=True,
                           timeout=10)
        commit = r.stdout.strip() or None
        r = subprocess.run(["git", "-C", root, "status", "--porcelain", "--", "kimi_delta_attention_03_amd/csrc",
                            "include"], capture_output=True, text=True, timeout=10)
        dirty = bool(r.stdout.strip())
    except Exception:
        pass
    info = {"commit": commit, "sources_dirty": dirty, "sources_sha256_16": h.hexdigest()[:16],
            "built_utc": time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime()), "arch": ARCH}
    with open(os.path.join(HERE, "_build_info.json"), "w") as f:
        json.dump(info, f)


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source and link the library; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, *LIBS, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    _write_build_info()
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args()
    build(args.jobs, verbose=True)
