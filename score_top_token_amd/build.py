"""Builds the HIP library liblightning_indexer.so in-tree for gfx950.

Each source is compiled by hipcc in parallel, then linked into one shared
object next to this file.  Packed fp32 instructions are disabled for all device
code (`-Xclang -target-feature -Xclang -packed-fp32-ops`).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblightning_indexer.so")
SOURCES = ["li_prefill_bf16.hip", "li_prefill_fp16.hip", "li_prefill_fp8.hip", "li_host.cpp",
           "li_metadata.hip", "li_prefill.hip", "li_decode.hip", "li_gather.hip", "li_grad.hip"]
ARCH = os.environ.get("LI_OFFLOAD_ARCH", "gfx950")


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


# The backward kernel keeps more accumulators than fit the VGPRs: its MFMA
# results stay free to live in the accumulation registers.
AGPR_SOURCES = {"li_grad.hip"}


def _flags(src=""):
    f = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-x", "hip",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    if src not in AGPR_SOURCES:
        # MFMA results straight into VGPRs, where the epilogue reads them
        f += ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    return f + ["-Wall", "-Wno-unused-function", "-I", os.path.join(HERE, "..", "include")]


def build(verbose: bool = False, jobs: int = 8) -> str:
    hipcc = _hipcc()
    tmpdir = tempfile.mkdtemp(prefix="li_build_")
    try:
        objs = []

        def compile_one(src):
            obj = os.path.join(tmpdir, src + ".o")
            cmd = [hipcc, *_flags(src), "-c", os.path.join(CSRC, src), "-o", obj]
            res = subprocess.run(cmd, capture_output=True, text=True)
            out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                            if "packed-fp32-ops" not in l)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{out}")
            if verbose and out.strip():
                print(out, file=sys.stderr)
            return obj

        with cf.ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES))) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        tmp_lib = LIB + ".tmp"
        cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp_lib, *objs]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
        os.replace(tmp_lib, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
