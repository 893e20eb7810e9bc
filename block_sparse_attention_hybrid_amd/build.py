"""Builds libsparse_attn.so (gfx950 kernels + C ABI) in the package directory.

    python -m block_sparse_attention_hybrid_amd.build [--verbose]

Every source is compiled by hipcc for gfx950 with packed-fp32 instructions
disabled, then linked into one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsparse_attn.so")
# sha256 of the sources, headers and flags the library was built from, written
# beside it by build(); the binding rebuilds when it no longer matches
STAMP = LIB + ".sha256"
ARCH = "gfx950"

# -amdgpu-mfma-vgpr-form: matrix-core accumulators live in VGPRs, which lets
# the attention kernel load its K/V operands straight into AGPRs instead of
# shuttling the output accumulator between the two register files
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def sources():
    names = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    return [os.path.join(CSRC, f) for f in names]


def source_digest() -> str:
    """sha256 over every source and header of the library and the flags."""
    h = hashlib.sha256(" ".join(COMMON).encode())
    names = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp", ".h")))
    for path in [os.path.join(CSRC, f) for f in names] + [os.path.join(INCLUDE, "sparse_attn.h")]:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def is_current() -> bool:
    """True when the built library exists and was built from the present sources."""
    if not (os.path.exists(LIB) and os.path.exists(STAMP)):
        return False
    with open(STAMP) as f:
        return f.read().strip() == source_digest()


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [_hipcc(), "-c", src, "-o", obj] + COMMON
    if src.endswith(".cpp"):
        cmd = [_hipcc(), "-x", "hip", "-c", src, "-o", obj] + COMMON
    if verbose:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{r.stderr}")
    if verbose:
        sys.stderr.write(r.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    digest = source_digest()
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    with open(STAMP + ".tmp", "w") as f:
        f.write(digest + "\n")
    os.replace(STAMP + ".tmp", STAMP)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
