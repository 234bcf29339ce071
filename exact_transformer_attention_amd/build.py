"""Build libattn.so (all HIP kernels and the C-ABI host code) for gfx950 with hipcc.

Usage: python -m exact_transformer_attention_amd.build  [--jobs N]
The library is written next to this file so that it travels with the source tree.
"""

import argparse
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattn.so")

SOURCES = ["api.cpp", "fwd_f32.hip", "fwd_bf16.hip", "fwd_fp8.hip", "decode.hip", "bwd_bf16.hip"]
# Per-source extra flags.  The attention kernels keep MFMA accumulators in VGPRs (their
# softmax reads every accumulator with VALU instructions; AGPR-form accumulators cost a
# copy per element per block).
EXTRA_FLAGS = {"fwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
               "decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
               "bwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
               "fwd_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; libattn needs the ROCm toolchain")
    return h


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON_FLAGS + EXTRA_FLAGS.get(src, [])
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    return obj


def build(verbose=False, jobs=4):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    build(verbose=a.verbose, jobs=a.jobs)


if __name__ == "__main__":
    sys.exit(main())
