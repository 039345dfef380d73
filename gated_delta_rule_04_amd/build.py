"""Build libgdn.so (the HIP kernels and the C-ABI) in-tree for gfx950.

    python -m gated_delta_rule_04_amd.build

Each translation unit is compiled with hipcc for gfx950 only; packed-fp32
instructions are disabled (-packed-fp32-ops) for every device compile.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = ["gdn_api.cpp", "gdn_decode.hip", "gdn_chunk.hip", "gdn_backward.hip", "gdn_bwd_chunk.hip",
           "gdn_epilogue.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags():
    return ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # keep register arrays (prefetch buffers) in registers, never in spare LDS
            "-mllvm", "-disable-promote-alloca-to-lds",
            "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source and link libgdn.so; returns its path."""
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="gdn_build_")
    try:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"]
            cmd = [cc] + compile_flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
            while len([p for _, p in procs if p.poll() is None]) >= jobs:
                procs[0][1].wait()
        errs = []
        for src, p in procs:
            out, _ = p.communicate()
            text = out.decode(errors="replace")
            # hipcc's host pass does not know the packed-fp32 target feature: harmless
            text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
            if p.returncode != 0:
                errs.append("%s:\n%s" % (src, text))
            elif verbose and text.strip():
                print(text)
        if errs:
            raise RuntimeError("HIP build failed:\n" + "\n".join(errs))
        out_tmp = LIB + ".tmp%d" % os.getpid()
        cmd = [cc, "-shared", "--offload-arch=" + ARCH, "-fPIC", "-o", out_tmp] + objs
        subprocess.run(cmd, check=True)
        os.replace(out_tmp, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
