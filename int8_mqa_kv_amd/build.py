"""Build libmqa_kv.so, the HIP library for gfx950 (MI355X).

    python -m int8_mqa_kv_amd.build

Each ``csrc/*.hip`` file is compiled by hipcc for ``--offload-arch=gfx950``
and linked into ``libmqa_kv.so`` beside this file.  Packed-fp32 instructions
are disabled (``-packed-fp32-ops``); the build then checks the device assembly
and refuses a library that contains any packed-fp32 arithmetic.
"""
import concurrent.futures
import glob
import os
import re
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmqa_kv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
PACKED_FP32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"command failed: {' '.join(cmd)}")
    return r


def _compile(src, objdir, verbose):
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    _run([HIPCC, *FLAGS, "-c", src, "-o", obj], verbose)
    asm = os.path.join(objdir, os.path.basename(src) + ".s")
    _run([HIPCC, *FLAGS, "--cuda-device-only", "-S", src, "-o", asm], verbose)
    text = open(asm).read()
    bad = sorted(set(m.group(0) for m in PACKED_FP32.finditer(text)))
    if bad:
        raise RuntimeError(f"{src}: packed-fp32 instructions in device code: {bad}")
    return obj


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with tempfile.TemporaryDirectory(prefix="mqa_build_") as objdir:
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            objs = list(ex.map(lambda s: _compile(s, objdir, verbose), srcs))
        tmp = LIB + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
