"""The pins are strong enough: plant plausible mistakes in a copy of the
oracle's C source (on the CPU, in a temporary directory), build each mutant,
and check that at least one pin fails for every one of them.
"""
import ctypes
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (what the mistake is, text in oracle.c, replacement)
MUTANTS = [
    ("softmax scale dropped", "sigma[j] = dot * softmax_scale;", "sigma[j] = dot;"),
    ("window one key too wide", "lo = p - (int64_t)window + 1;", "lo = p - (int64_t)window;"),
    ("window one key too narrow", "lo = p - (int64_t)window + 1;", "lo = p - (int64_t)window + 2;"),
    ("query does not see its own key", "int64_t hi = p + 1; /* exclusive */",
     "int64_t hi = p; /* exclusive */"),
    ("keys used as values", "double v = (double)vs[r] * (double)vc[r * (int64_t)d + c];",
     "double v = (double)ks[r] * (double)kc[r * (int64_t)d + c];"),
    ("first token's key scale for every key",
     "double k = (double)ks[r] * (double)kc[r * (int64_t)d + c];",
     "double k = (double)ks[0] * (double)kc[r * (int64_t)d + c];"),
    ("query channels reversed", "dot += q[c] * k;", "dot += q[d - 1 - c] * k;"),
    ("exp2 instead of exp", "sigma[j] = exp(sigma[j] - m);", "sigma[j] = exp2(sigma[j] - m);"),
    ("output not normalised", "for (int32_t c = 0; c < d; ++c) out[c] /= z;",
     "for (int32_t c = 0; c < d; ++c) out[c] /= 1.0;"),
    ("quantiser divides by 128", "volatile float s = a / 127.0f;",
     "volatile float s = a / 128.0f;"),
    ("quantiser rounds half away from zero", "float n = nearbyintf(r);",
     "float n = roundf(r);"),
    ("quantiser truncates", "float n = nearbyintf(r);", "float n = truncf(r);"),
    ("quantiser multiplies by a reciprocal of the scale", "volatile float r = row[c] / sv;",
     "volatile float r = row[c] * (1.0f / sv);"),
    ("quantiser multiplies by 127 / max", "volatile float r = row[c] / sv;",
     "volatile float r = row[c] * (127.0f / a);"),
    ("dequantiser drops the scale",
     "(double)scales[t] * (double)codes[t * (int64_t)d + c];",
     "(double)codes[t * (int64_t)d + c];"),
    ("byte formula drops the factor 2", "return 2 * num_layers", "return 1 * num_layers"),
]

PIN_TESTS = [getattr(pins, n) for n in dir(pins)
             if n.startswith("test_") and not n.startswith("test_bruteforce_tiny")]


def _run_pins():
    failed = []
    for t in PIN_TESTS:
        try:
            t()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed.append(t.__name__)
    for seed in range(4):
        try:
            pins.test_bruteforce_tiny(seed)
        except Exception:  # noqa: BLE001
            failed.append(f"test_bruteforce_tiny[{seed}]")
    return failed


@pytest.mark.parametrize("what,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(what, old, new, monkeypatch):
    src = open(SRC).read()
    assert old in src, f"mutation anchor for '{what}' no longer in oracle.c"
    tmp = tempfile.mkdtemp(prefix="oracle_mutant_")
    try:
        path = os.path.join(tmp, "oracle.c")
        open(path, "w").write(src.replace(old, new))
        lib_path = os.path.join(tmp, "liboracle.so")
        subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                        path, "-o", lib_path, "-lm"], check=True)
        real = oracle._load()
        lib = ctypes.CDLL(lib_path)
        for name in ("oracle_quantize_rows", "oracle_dequantize_rows", "oracle_attend",
                     "oracle_kv_bytes_per_token", "oracle_num_threads"):
            getattr(lib, name).argtypes = getattr(real, name).argtypes
            getattr(lib, name).restype = getattr(real, name).restype
        monkeypatch.setattr(oracle, "_lib", lib)
        failed = _run_pins()
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    assert failed, f"no pin catches the planted mistake: {what}"


def test_unmutated_source_passes_all_pins():
    assert _run_pins() == []
