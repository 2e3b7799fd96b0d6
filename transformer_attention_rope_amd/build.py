"""Builds libnc_attn.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m transformer_attention_rope_amd.build      # or: python transformer_attention_rope_amd/build.py

Every source is compiled each time (seconds per file); objects go to
``_build/`` at the repository root and the shared library is written next to
this file, where the Python binding loads it.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libnc_attn.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["abi.cpp", "rope.hip", "attn_fwd.hip", "attn_decode.hip", "attn_bwd.hip", "noalloc.hip",
           "qkv.hip"]

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 (v_pk_*_f32) instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the HIP library)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature name: harmless
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


# The kernels keep every value in registers: no scratch (spill) memory. Besides
# the cost, the attention tile loops wait for their LDS copies with a hand-
# counted vmcnt that assumes the only vector-memory operations of a tile are
# the copies and loads the code issues itself; spill traffic would add others.
# The compiler's resource-usage remarks give each kernel's scratch bytes.
REMARKS = ["-Rpass-analysis=kernel-resource-usage"]


def scratch_kernels(remarks: str):
    """(kernel, scratch bytes per lane) for every kernel with scratch."""
    bad, cur = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and cur is not None and int(m.group(1)) > 0:
            bad.append((cur, int(m.group(1))))
    return bad


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip", *REMARKS] if src.endswith(".hip") else []
        cmds.append([cc, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 4)) as ex:
        for src, err in zip(SOURCES, ex.map(_run, cmds)):
            bad = scratch_kernels(err)
            if bad:
                raise RuntimeError(f"{src}: kernels with scratch (register spills): {bad}")
            if verbose:
                rest = "\n".join(l for l in err.splitlines() if "kernel-resource-usage" not in l)
                if rest.strip():
                    print(rest, file=sys.stderr)
    tmp = OUT + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
