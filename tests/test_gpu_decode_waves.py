"""Both decode workgroup shapes -- eight wavefronts (one workgroup per CU) and
four (two per CU) -- forced in turn through the same workloads, against the
oracle, and the other plans mqa_decode_tuning allows (8-, 16- and 32-row
blocks, workgroup targets from 64 to 1024).  Which plan a launch takes by
default is a planner choice (tested on the CPU); each must compute the same
attention within the usual tolerance.
"""
import pytest

import int8_mqa_kv_amd as mk
import synth
from tests.test_gpu_decode import _run_case
from tests.test_gpu_decode_step import check_step

pytestmark = pytest.mark.gpu


@pytest.fixture(params=[4, 8], ids=["waves4", "waves8"])
def waves(request):
    mk.decode_tuning(waves=request.param)
    try:
        yield request.param
    finally:
        mk.decode_tuning()


WORKLOADS = {
    # 96 row-block items over one shared slot, 16k tokens each
    "three_layers_one_slot": lambda: synth.case3(),
    # 130 ragged sequences: kept whole with eight wavefronts, three chunks with four
    "ragged_130": lambda: synth.custom_decode(
        22, 130, 32, 128, "bf16", [1 + (37 * i * i + 11 * i) % 1500 for i in range(130)], 1, 0, 0),
    # windowed layer, contexts from 1 to 12345 tokens, permuted pool
    "window_ragged": lambda: synth.custom_decode(
        9, 6, 32, 128, "bf16", [6000, 1, 7, 4096, 4097, 12345], 1, 1024, permuted_pool=3000),
    # 48 heads (a 32-row and a 16-row block), two layers
    "heads48": lambda: synth.custom_decode(
        6, 5, 48, 128, "bf16", [1, 64, 65, 129, 700], 2, 0, permuted_pool=200),
    # head_dim 64, 16 heads, three layers, window 100
    "d64": lambda: synth.custom_decode(7, 2, 16, 64, "bf16", [33, 1234], 3, 100, 0),
}


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_decode_shape(waves, name):
    _run_case(WORKLOADS[name]())


def test_step_shape(waves):
    """The fused step (current token stored, then attention) in both shapes."""
    check_step(synth.case3())
    w = synth.custom_decode(40, 5, 32, 128, "bf16", [1, 16, 17, 1500, 3001], 4, 0,
                            permuted_pool=800)
    check_step(w, [0, 0, 0, 0], [0, 1024, 1, 300])


# Plans the planner does not pick by itself but mqa_decode_tuning allows:
# 8-row blocks, and workgroup targets far below and above one per CU (fewer,
# longer chunks; several rounds of workgroups).
TUNINGS = [dict(rows=8), dict(rows=16), dict(rows=32), dict(target_wgs=64), dict(target_wgs=1024),
           dict(waves=4, rows=8)]


@pytest.fixture(params=TUNINGS, ids=["-".join(f"{k}{v}" for k, v in t.items()) for t in TUNINGS])
def tuning(request):
    mk.decode_tuning(**request.param)
    try:
        yield request.param
    finally:
        mk.decode_tuning()


@pytest.mark.parametrize("name", ["window_ragged", "heads48", "d64"])
def test_decode_tuned_plan(tuning, name):
    _run_case(WORKLOADS[name]())
