"""mqa_append_attn on the GPU against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import GpuCase, OracleKV, assert_parity, assert_parity_peaked, log, q_tensor

pytestmark = pytest.mark.gpu


def _run(w, seqs=None):
    log(f"append case {w.case}: {w.name} B={w.batch} Hq={w.num_q_heads} d={w.head_dim} "
        f"L={w.num_layers} qlens={w.q_lens[:6].tolist()} maxctx={w.max_context}")
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    out = g.append(q)
    want = oracle.append(q64, w.context_lens, w.cu_q_lens, w.layer_slot, w.layer_window,
                         OracleKV(w), seqs=seqs)
    assert_parity(out.cpu().numpy(), want, f"append case {w.case}")
    return g, q, out


EDGE = [
    # (seed, prefixes, q_lens, hq, d, windows, slots)
    (40, [0, 5, 40], [1, 3, 5], 8, 64, [0], [0]),
    (41, [100, 17, 2000], [64, 1, 13], 32, 128, [1024, 0], [0, 1]),
    (42, [3000, 1023, 1024, 1025], [64, 64, 64, 64], 32, 128, [1024] * 2 + [0] + [0], [0, 1, 2, 2]),
    (43, [50, 600], [7, 9], 32, 128, [1, 16, 17], [0, 1, 2]),
    (44, [300, 40], [33, 2], 48, 128, [0, 8], [0, 0]),
]


@pytest.mark.parametrize("case", EDGE, ids=[f"edge{c[0]}" for c in EDGE])
def test_append_edges(case):
    seed, prefix, qlens, hq, d, wins, slots = case
    w = synth.custom_append(seed, prefix, qlens, hq, d, wins, slots)
    _run(w)


def test_append_fp32_q():
    w = synth.custom_append(45, [200, 31], [5, 16], 32, 128, [0, 64], [0, 1], q_dtype="f32")
    _run(w)


def test_append_one_token_matches_decode():
    w = synth.custom_append(46, [500, 77, 4000], [1, 1, 1], 32, 128, [0, 1024], [0, 1])
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    app = g.append(q).cpu().numpy()
    dec = g.decode(q).cpu().numpy()          # [L, total_q = B, Hq, D] is decode's layout
    # The two kernels split the keys differently, so the fp16 P operand is
    # rounded against different running maxima: each side is within 2^-12 of
    # |out| of the exact result (both are checked against the oracle elsewhere).
    np.testing.assert_allclose(app, dec, rtol=0, atol=1e-3)
    want = oracle.decode(q64, w.context_lens, w.layer_slot, w.layer_window, OracleKV(w))
    assert_parity(app, want, "append q_len=1")
    assert_parity(dec, want, "decode of the same rows")


def test_case4_hybrid_turn_sampled():
    """The full hybrid turn (256 sequences, 12 layers) on the GPU; the oracle
    checks every output of a sample of sequences (shortest, longest, median
    and a few random ones)."""
    w = synth.case4()
    order = np.argsort(w.context_lens)
    seqs = sorted(set([int(order[0]), int(order[-1]), int(order[len(order) // 2]), 7, 101, 200]))
    _run(w, seqs=seqs)


def test_append_peaked_softmax():
    """q scaled by 16 (exact in bf16): concentrated weights over a causal chunk."""
    w = synth.custom_append(47, [900, 3000], [64, 17], 32, 128, [1024, 0], [0, 1])
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    q, q64 = q * 16, q64 * 16
    out = g.append(q)
    want = oracle.append(q64, w.context_lens, w.cu_q_lens, w.layer_slot, w.layer_window,
                         OracleKV(w))
    assert_parity_peaked(out.cpu().numpy(), want, w, "append, peaked softmax")
