"""Build libmi355attn.so (gfx950) in-tree with hipcc.

Every HIP source under csrc/ is compiled for gfx950 only, with packed-FP32
instructions disabled on the device pass, and linked into one shared library
next to this file.  Run ``python -m transformer_attention_attn_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmi355attn.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-fvisibility=hidden"]
# The flash kernels take row maxima of scores that are never NaN; without NaN
# semantics fmax needs no quieting (v_max3 instead of two canonicalizing v_max).
# Only that file: host-side validation must keep its NaN checks.
EXTRA = {"flash_attn.hip": ["-fno-honor-nans"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    extra = EXTRA.get(os.path.basename(src), [])
    r = subprocess.run([HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj], capture_output=True, text=True)
    msgs = [l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l]
    if r.returncode:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 4)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
