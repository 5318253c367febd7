"""Build libmqa_kv.so, the HIP library for gfx950 (MI355X).

    python -m int8_mqa_kv_amd.build

Each ``csrc/*.hip`` file is compiled by hipcc for ``--offload-arch=gfx950``
and linked into ``libmqa_kv.so`` beside this file.  Packed-fp32 instructions
are disabled (``-packed-fp32-ops``); the build then checks the device assembly
and refuses a library that contains any packed-fp32 arithmetic, or a kernel
that keeps anything in per-lane scratch memory (arrays the compiler could not
hold in registers: every kernel here is meant to live in registers and LDS).
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
KERNEL_META = re.compile(r"\.name:\s+(\S+)")
SCRATCH = re.compile(r"\.private_segment_fixed_size:\s+(\d+)")


def _scratch_kernels(text):
    """(kernel, bytes) for every kernel of an assembly file with a private segment."""
    out = []
    for block in text.split("  - .agpr_count:")[1:]:
        name, size = KERNEL_META.search(block), SCRATCH.search(block)
        if name and size and int(size.group(1)) > 0:
            out.append((name.group(1), int(size.group(1))))
    return out


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
    scratch = _scratch_kernels(text)
    if scratch:
        raise RuntimeError(f"{src}: kernels using scratch memory: {scratch}")
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
