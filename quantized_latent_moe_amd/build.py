"""Compile the gfx950 HIP library (liblatmoe.so) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblatmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 anywhere in the device code.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA results in ordinary VGPRs (no v_accvgpr_read per folded value)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-result",
]


# Extra flags of single sources.  gateup.hip: LLVM's max-ILP machine scheduler
# interleaves the Q3_K gate/up kernel's fold with its MFMAs better (gate/up
# about 1.5% faster at 5268 and 21000 tokens); the other kernels gain nothing
# from it (down is slightly slower).
SOURCE_FLAGS = {"gateup.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def compile_flags(source: str) -> list:
    """The flags one source's object is compiled with."""
    return [f for f in FLAGS if f != "-shared"] + SOURCE_FLAGS.get(os.path.basename(source), [])


def build(verbose: bool = False) -> str:
    """Compile every source to an object with its flags, in parallel, then
    link the shared library."""
    tmpdir = tempfile.mkdtemp(prefix="latmoe_build_")
    try:
        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [HIPCC, *compile_flags(src), "-I", os.path.join(HERE, "..", "include"), "-c", "-o", obj, src]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.check_call(cmd)
            return obj

        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            objs = list(ex.map(compile_one, sources()))
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
