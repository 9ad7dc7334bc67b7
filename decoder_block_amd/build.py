"""Build libllama_layer.so (gfx950) in-tree with hipcc.

    python -m decoder_block_amd.build            # compile everything
    python -m decoder_block_amd.build --host-asan  # host-only ASan/UBSan test build of the host runtime

Objects go to decoder_block_amd/_build/, the library to decoder_block_amd/lib/.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libllama_layer.so")

ARCH = "gfx950"
SOURCES = ["llama_layer.cpp", "gemm.hip", "norm.hip", "attn_prefill.hip", "attn_decode.hip", "misc.hip",
           "scratch.hip"]
# MFMA results in VGPRs (not AGPRs): the attention kernels rescale their output
# accumulators with VALU ops, which cannot read AGPRs.
EXTRA = {"attn_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "attn_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 VALU forms on this hardware
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + err)
    return err


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *FLAGS, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        msg = _run(cmd)
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
        return obj

    n = jobs or min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(n) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def build_host_asan() -> str:
    """Host runtime + stub kernels under ASan/UBSan (CPU only; no device code)."""
    out = os.path.join(BUILD, "host_asan")
    os.makedirs(out, exist_ok=True)
    exe = os.path.join(out, "host_check")
    srcs = [os.path.join(CSRC, "llama_layer.cpp"), os.path.join(ROOT, "tests", "host", "host_check.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           *srcs, "-o", exe, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    _run(cmd)
    return exe


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--host-asan", action="store_true")
    ap.add_argument("-v", action="store_true")
    args = ap.parse_args()
    print(build_host_asan() if args.host_asan else build(verbose=args.v))
