"""Build libctconv.so (HIP, gfx950) in-tree with hipcc.

    python -m vision_upsampler_decoders_amd.build            # every source
    python -m vision_upsampler_decoders_amd.build --changed  # sources newer than their objects

Every HIP source is compiled for gfx950 only, with packed-fp32 VALU forms
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops), then linked into
one shared library next to this file.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libctconv.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]

SOURCES = ["ctconv_api.hip", "prepack.hip", "gather.hip", "pointwise.hip", "stream.hip",
           "depthwise.hip", "polyphase.hip", "polyrw.hip", "noalloc.hip", "clock.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass does not know the packed-fp32 feature flag; drop that noise
    noise = ("packed-fp32-ops", "not a recognized feature", "warning generated")
    errs = [l for l in r.stderr.splitlines() if l.strip() and not any(n in l for n in noise)]
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")
    return obj


def _stale(src: str) -> bool:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    deps = [os.path.join(CSRC, src), os.path.join(CSRC, "ctconv_internal.h"),
            os.path.join(CSRC, "mfma_common.h"), os.path.join(INCLUDE, "ctconv.h")]
    return any(os.path.getmtime(d) > t for d in deps)


def build(jobs: int = 8, changed_only: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    todo = [s for s in SOURCES if _stale(s)] if changed_only else list(SOURCES)
    if todo:
        with cf.ThreadPoolExecutor(max_workers=min(jobs, len(todo))) as ex:
            list(ex.map(_compile, todo))
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(changed_only="--changed" in sys.argv[1:]))
