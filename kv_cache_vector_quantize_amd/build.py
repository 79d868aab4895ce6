"""Build libtq.so in-tree with hipcc for gfx950.

``python -m kv_cache_vector_quantize_amd.build`` (or ``build()``) compiles
every ``csrc/*.hip`` translation unit and links them into
``kv_cache_vector_quantize_amd/libtq.so``.  It always rebuilds.
"""

import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtq.so")
ARCH = os.environ.get("TQ_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 VALU instructions (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# The decode kernels (decode_g*.hip) never operate on a NaN: tokens past the
# context are masked before their stored bytes are used as numbers, and the
# inputs are finite.  Without NaNs the IEEE mode's quieting of signalling
# NaNs is unnecessary, and with it off the compiler drops the canonicalising
# v_max (max(x, x)) it otherwise puts before every fmaxf of the online
# softmax: about 17 of the ~290 vector instructions per 32-token block.
NO_NAN_FLAGS = ["-fno-honor-nans", "-mno-amdgpu-ieee"]


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    extra = NO_NAN_FLAGS if os.path.basename(src).startswith("decode_g") else []
    cmd = [HIPCC, *COMMON_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    if verbose:
        for _, err in results:
            if err.strip():
                print(err, file=sys.stderr)
    _link([o for o, _ in results], LIB)
    return LIB


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


if __name__ == "__main__":
    print(build(verbose=True))
