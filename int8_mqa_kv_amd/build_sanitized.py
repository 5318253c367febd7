"""Build libmqa_kv_san.so: the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer, for CPU-only checks of the host paths (argument
checks, launch planning, the page table, the prefix cache's tree, LRU list,
hash index and arena bookkeeping).

    python int8_mqa_kv_amd/build_sanitized.py

Every ``csrc/*.hip`` file is compiled as for the GPU build, with
``-fsanitize=address`` and ``-fsanitize=undefined`` applied to the host
compilation only (the device code is built as usual and never sanitized),
then linked by clang++ against the HIP runtime.  Load it
through the binding with ``MQA_KV_LIB=<path>`` in a process that preloads the
ASan runtime (``tests/test_host_sanitizers.py`` does this).  Never for a GPU.
"""
import concurrent.futures
import glob
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmqa_kv_san.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
COMPILE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]


def asan_runtime() -> str:
    """Path of clang's shared ASan runtime (preloaded by the sanitizer run)."""
    hits = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under the ROCm LLVM")
    return hits[-1]


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with tempfile.TemporaryDirectory(prefix="mqa_san_") as tmp:
        def one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [HIPCC, *COMPILE, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True, stderr=subprocess.DEVNULL if not verbose else None)
            return obj
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            objs = list(ex.map(one, srcs))
        link = [CLANGXX, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libasan",
                *objs, "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
                "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", LIB + ".tmp"]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
        os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
