"""Sanitizer tier (CPU only): the oracle and the library's host-side code
under AddressSanitizer and UndefinedBehaviorSanitizer.

* The oracle (plain C) is built with gcc and driven by
  tests/native/oracle_san.c over 300 seeded small shapes (1-D and 2-D,
  stride, padding, output_padding, dilation, groups, empty batches), the
  per-point evaluators against the full result, and the iSTFT pieces.
* The library's host code (shape rules, packed sizes, every route planner,
  workspace and stream sizes, argument validation) is built with the
  sanitizers on the host side only (device code is compiled unoptimised and
  never run) and driven by tests/native/abi_san.cpp: 20000 seeded shapes
  through the queries and every entry point with arguments its validation
  rejects before any device call.  No GPU is used.

The library build is cached under vision_upsampler_decoders_amd/_build/san,
keyed by the sources' contents."""

import hashlib
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "vision_upsampler_decoders_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
SAN_DIR = os.path.join(ROOT, "vision_upsampler_decoders_amd", "_build", "san")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-3000:] + r.stderr[-3000:]
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", *SAN, os.path.join(ROOT, "oracle", "ctconv_oracle.c"),
          os.path.join(ROOT, "tests", "native", "oracle_san.c"), "-o", exe, "-lm"])
    r = _run([exe], env=ENV, timeout=600)
    assert r.stdout.startswith("ok "), r.stdout


def _library():
    h = hashlib.sha256()
    for f in SOURCES + ["ctconv_internal.h", "mfma_common.h"]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    with open(os.path.join(INCLUDE, "ctconv.h"), "rb") as fh:
        h.update(fh.read())
    key = h.hexdigest()[:16]
    lib = os.path.join(SAN_DIR, "libctconv_san.so")
    stamp = os.path.join(SAN_DIR, "stamp")
    if os.path.exists(lib) and os.path.exists(stamp) and open(stamp).read() == key:
        return lib
    os.makedirs(SAN_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(SAN_DIR, src.replace(".hip", ".o"))
        # sanitizers on the host side only; device code unoptimised (never run)
        _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
              "-Xarch_host", SAN[0], "-Xarch_host", SAN[1], "-Xarch_host", SAN[2],
              "-Xarch_device", "-O0", "-Xarch_device", "-g0",
              "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    _run([CLANGXX, *SAN, "-shared", "-fPIC", *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", lib])
    with open(stamp, "w") as f:
        f.write(key)
    return lib


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                    reason="hipcc / clang++ not available")
def test_library_host_code_under_sanitizers(tmp_path):
    lib = _library()
    exe = str(tmp_path / "abi_san")
    _run([CLANGXX, "-O1", "-g", "-std=c++17", *SAN, "-I", INCLUDE,
          os.path.join(ROOT, "tests", "native", "abi_san.cpp"), lib,
          "-Wl,-rpath," + os.path.dirname(lib), "-o", exe])
    r = _run([exe], env=ENV, timeout=600)
    assert r.stdout.startswith("ok "), r.stdout
