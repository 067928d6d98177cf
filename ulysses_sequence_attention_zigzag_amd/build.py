"""Builds libusp.so (HIP C++ for gfx950) in-tree.

    python -m ulysses_sequence_attention_zigzag_amd.build

Each source is compiled by hipcc into _build/ (in parallel), then linked into
ulysses_sequence_attention_zigzag_amd/libusp.so.  Always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libusp.so")
SOURCES = ["api.cpp", "plan.cpp", "plan_dev.hip", "timing.cpp", "permute.hip", "lse_merge.hip", "attn_fwd.hip", "attn_bwd.hip",
           "attn_bwd_dq.hip", "decode.hip", "noalloc.hip"]
# per-source flags: the dQ kernel is built with VGPR-form MFMAs
SOURCE_FLAGS = {"attn_bwd_dq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{ROOT}/include",
]


def _compile(src: str, extra, csrc: str, build_dir: str) -> str:
    obj = os.path.join(build_dir, src + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC] + COMMON + SOURCE_FLAGS.get(src, []) + list(extra) + lang + ["-c", os.path.join(csrc, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(extra=(), verbose: bool = False, csrc: str = CSRC, out: str = LIB) -> str:
    """Compiles every source of `csrc` and links `out` (libusp.so); returns its path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    build_dir = BUILD if out == LIB else os.path.join(os.path.dirname(out), "_build")
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, csrc, build_dir), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # every symbol of the library's own namespace must be defined in it (a
    # kernel whose host stub the compiler failed to emit shows up here
    # instead of at load time)
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines() if "_ZN3usp" in l]
    if nm.returncode != 0 or missing:
        raise RuntimeError(f"link of {out} left undefined library symbols: {missing[:5]} {nm.stderr}")
    shutil.move(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(sys.argv[1:], verbose=True)
