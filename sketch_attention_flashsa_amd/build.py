"""Build libsketchattn.so in-tree with hipcc for gfx950.

    python -m sketch_attention_flashsa_amd.build [-j N] [--diag]

Every HIP source under csrc/ is compiled to an object in parallel, then the
objects are linked into ``sketch_attention_flashsa_amd/libsketchattn.so``.
Cross-compiles without a GPU.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsketchattn.so")
ARCH = os.environ.get("SA_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU instructions are disabled for every HIP translation unit.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         f"-I{INCLUDE}", f"-I{CSRC}"]


# The sources a kernel's measurements depend on (its own file and the headers
# it includes); a measurement stays valid while these are unchanged.
KERNEL_SOURCES = {
    "sa_bf16_stream_kernel": ("sa_bf16_stream.hip", "sa_device.h", "sa_internal.h"),
}


def sources_hash(files=None) -> str:
    """First 16 hex digits of the sha256 over the given csrc files (default:
    every csrc/*.hip and *.h), in name order: tags measurements taken on one
    version of the kernels."""
    import hashlib
    h = hashlib.sha256()
    names = sorted(files) if files is not None else sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h")))
    for f in names:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, extra: list[str], out_dir: str = BUILD) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int = 8, extra: list[str] | None = None, verbose: bool = False,
          out_dir: str = BUILD, lib: str = LIB) -> str:
    """Compile every csrc/*.hip with ``extra`` flags into ``out_dir`` and link
    ``lib`` (default: the in-tree libsketchattn.so); return its path."""
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    extra = list(extra or [])
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, out_dir), srcs))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


DIAG = os.path.join(PKG, "diag")


def build_diag(verbose: bool = False) -> list[str]:
    """Compile the stand-alone measurement programs under diag/ (each .hip
    into an executable of the same name beside it); return their paths."""
    outs = []
    for src in sorted(glob.glob(os.path.join(DIAG, "*.hip"))):
        exe = src[:-4]
        cmd = [_hipcc(), *[f for f in FLAGS if f != "-fPIC"], src, "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        outs.append(exe)
        if verbose:
            print(f"built {exe}")
    return outs


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=8)
    ap.add_argument("--diag", action="store_true", help="also build the measurement programs under diag/")
    args = ap.parse_args()
    build(jobs=args.j, verbose=True)
    if args.diag:
        build_diag(verbose=True)
