"""Build libpagedattn.so for gfx950 with hipcc (in-tree, no JIT cache).

Usage: python -m paged_mqa_gqa_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(HERE, "lib")
LIB_NAME = "libpagedattn.so"
SOURCES = ["api.hip", "kv_append.hip", "decode_attn.hip", "splitk_reduce.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build)")
    return path


def _compile(src: str, obj: str) -> tuple[str, int, str]:
    cmd = [hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (p.stdout + p.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    return src, p.returncode, err


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    obj_dir = os.path.join(OUT_DIR, "obj")
    os.makedirs(obj_dir, exist_ok=True)
    objs = [os.path.join(obj_dir, s.replace(".hip", ".o")) for s in SOURCES]
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES, objs))
    failed = [(s, e) for s, rc, e in results if rc != 0]
    for s, rc, e in results:
        if verbose and e.strip():
            print(f"[{s}]\n{e}", file=sys.stderr)
    if failed:
        msg = "\n".join(f"--- {s} ---\n{e}" for s, e in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = os.path.join(OUT_DIR, LIB_NAME + ".tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stdout}\n{p.stderr}")
    final = os.path.join(OUT_DIR, LIB_NAME)
    os.replace(tmp, final)
    return final


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose))
