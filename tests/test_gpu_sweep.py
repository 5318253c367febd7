"""Seeded sweeps of decode and append shapes against the oracle.

Each case draws its shape from its own seed: batch, query heads, head_dim,
query dtype, contexts (from 1 token to ~20k, page edges included), layers
and a window per layer (global, 1, 16, 17, 300 or 1024 tokens), so that the
planner's choices (rows per block, four or eight wavefronts, chunks per item)
and the masked and slow softmax paths meet in combinations the hand-written
cases do not cover.  Tolerance as everywhere: max |gpu - oracle| <= 2e-3 and
relative L2 <= 1e-3.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import GpuCase, OracleKV, assert_parity, log, q_tensor

pytestmark = pytest.mark.gpu

WINDOWS = [0, 0, 1, 16, 17, 300, 1024]
ROW_KEY_BUDGET = 40_000_000  # oracle work per case (query rows x keys)


def _decode_shape(seed):
    g = np.random.default_rng(7000 + seed)
    d = int(g.choice([64, 128], p=[0.25, 0.75]))
    hq = int(g.choice([8, 16, 32, 48]))
    qd = str(g.choice(["bf16", "f32"], p=[0.75, 0.25]))
    layers = int(g.integers(1, 5))
    windows = [int(g.choice(WINDOWS)) for _ in range(layers)]
    batch = int(g.integers(1, 21))
    long_ = g.random(batch) < 0.3
    ctx = np.where(long_, g.integers(1, 20001, batch), g.integers(1, 1100, batch))
    ctx[g.random(batch) < 0.15] = int(g.choice([1, 15, 16, 17, 32, 33, 1024, 1025]))
    # keep the oracle's work bounded: shorten the longest contexts first
    while layers * hq * int(ctx.sum()) > ROW_KEY_BUDGET:
        i = int(np.argmax(ctx))
        ctx[i] = max(1, ctx[i] // 2)
    return d, hq, qd, layers, windows, batch, [int(c) for c in ctx]


@pytest.mark.parametrize("seed", range(12))
def test_decode_sweep(seed):
    d, hq, qd, layers, windows, batch, ctx = _decode_shape(seed)
    pages = sum(synth.pages_for(c) for c in ctx)
    w = synth.custom_decode(200 + seed, batch, hq, d, qd, ctx, layers, 0,
                            permuted_pool=pages + 97 if seed % 2 else 0)
    log(f"decode sweep {seed}: B={batch} Hq={hq} d={d} q={qd} windows={windows} "
        f"ctx max {max(ctx)} sum {sum(ctx)}")
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    ls = [0] * layers
    out = g.decode(q, ls, windows)
    want = oracle.decode(q64, w.context_lens, ls, windows, OracleKV(w))
    assert_parity(out.cpu().numpy(), want, f"decode sweep {seed}")


def _append_shape(seed):
    g = np.random.default_rng(8000 + seed)
    batch = int(g.integers(1, 7))
    prefix = [int(x) for x in g.integers(0, 5001, batch)]
    q_lens = [int(x) for x in g.integers(1, 71, batch)]
    # a global slot shared by up to two layers, and local slots
    nloc = int(g.integers(0, 3))
    windows = [int(g.choice([1, 100, 1024])) for _ in range(nloc)]
    nglob = int(g.integers(1, 3))
    layer_window = windows + [0] * nglob
    layer_slot = list(range(nloc)) + [nloc] * nglob
    return batch, prefix, q_lens, layer_window, layer_slot


@pytest.mark.parametrize("seed", range(6))
def test_append_sweep(seed):
    batch, prefix, q_lens, layer_window, layer_slot = _append_shape(seed)
    w = synth.custom_append(300 + seed, prefix, q_lens, 32, 128, layer_window, layer_slot)
    log(f"append sweep {seed}: B={batch} prefix={prefix} q_lens={q_lens} windows={layer_window} "
        f"slots={layer_slot}")
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    out = g.append(q)
    want = oracle.append(q64, w.context_lens, w.cu_q_lens, w.layer_slot, w.layer_window,
                         OracleKV(w))
    assert_parity(out.cpu().numpy(), want, f"append sweep {seed}")
