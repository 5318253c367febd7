"""mqa_append_attn on the GPU against the oracle."""
import time

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import (MAX_ABS, REL_L2, GpuCase, OracleKV, assert_parity, log, outlier_q,
                            q_tensor, with_v_gain)

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
    # The two kernels split the keys differently: the same terms summed in
    # another order and against other running maxima.
    diff = float(np.abs(app - dec).max())
    log(f"  append q_len=1 vs decode: max |diff| {diff:.2e}")
    assert diff <= 1e-4
    want = oracle.decode(q64, w.context_lens, w.layer_slot, w.layer_window, OracleKV(w))
    assert_parity(app, want, "append q_len=1")
    assert_parity(dec, want, "decode of the same rows")


@pytest.mark.timeout(1200)
def test_case4_hybrid_turn_full():
    """The full hybrid turn (256 sequences x 64 appended tokens, 12 layers, 11
    slots) on the GPU against the oracle on every output row: about 6.6e12
    fp64 flop on the host cores, taken 16 sequences at a time (each a
    sub-problem of its own) with the maximum error and the L2 sums gathered
    over the whole output."""
    w = synth.case4()
    log(f"append case 4: B={w.batch} L={w.num_layers} total_q={int(w.cu_q_lens[-1])}")
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    got_all = g.append(q).cpu().numpy()
    kv = OracleKV(w)
    cu, ctx = w.cu_q_lens.astype(np.int64), w.context_lens.astype(np.int64)
    max_abs, sq_diff, sq_ref, t0 = 0.0, 0.0, 0.0, time.time()
    for c0 in range(0, w.batch, 16):
        seqs = list(range(c0, min(w.batch, c0 + 16)))
        rows = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in seqs])
        cu_sub = np.concatenate([[0], np.cumsum([cu[b + 1] - cu[b] for b in seqs])])
        want = oracle.append(q64[:, rows], ctx[seqs], cu_sub, w.layer_slot, w.layer_window,
                             lambda s_, i: kv(s_, seqs[i]))
        got = got_all[:, rows].astype(np.float64)
        assert np.all(np.isfinite(got)), f"sequences {seqs[0]}..{seqs[-1]}: non-finite output"
        d = got - want
        max_abs = max(max_abs, float(np.abs(d).max()))
        sq_diff += float(np.sum(d * d))
        sq_ref += float(np.sum(want * want))
        for b in seqs:
            for s_ in range(w.num_slots):
                kv.cache.pop((s_, b), None)
        log(f"  sequences {seqs[0]}..{seqs[-1]}: max_abs so far {max_abs:.3e} "
            f"({time.time() - t0:.0f} s)")
    rel = (sq_diff / sq_ref) ** 0.5
    log(f"  parity append case 4 (whole output): max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= MAX_ABS and rel <= REL_L2


def test_append_peaked_softmax():
    """q scaled by 16 (exact in bf16): concentrated weights over a causal chunk."""
    w = synth.custom_append(47, [900, 3000], [64, 17], 32, 128, [1024, 0], [0, 1])
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    q, q64 = q * 16, q64 * 16
    out = g.append(q)
    want = oracle.append(q64, w.context_lens, w.cu_q_lens, w.layer_slot, w.layer_window,
                         OracleKV(w))
    assert_parity(out.cpu().numpy(), want, "append, peaked softmax")


@pytest.mark.parametrize("gain", [64, 512])
def test_append_outlier_query_channels(gain):
    """Append rows whose four outlier q channels are 64 or 512 times the rest."""
    w = synth.custom_append(48, [900, 3000], [64, 17], 32, 128, [1024, 0], [0, 1])
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    q, q64 = outlier_q(q, q64, gain, 700 + gain)
    out = g.append(q)
    want = oracle.append(q64, w.context_lens, w.cu_q_lens, w.layer_slot, w.layer_window,
                         OracleKV(w))
    assert_parity(out.cpu().numpy(), want, f"append, outlier q x{gain}")


def test_append_v_scales_over_many_octaves():
    """Append over V rows that are zero, then 2^-80 of the usual size, then
    growing by powers of two (see with_v_gain)."""
    _run(with_v_gain(synth.custom_append(49, [20, 900, 3000], [30, 64, 17], 32, 128, [1024, 0],
                                         [0, 1])))


@pytest.mark.parametrize("prefix", [16000, 32000])
def test_append_long_global_prefix(prefix):
    """A chunk over a long cached prefix on a global layer: every wavefront
    walks the whole prefix in one workgroup (no split), so its accumulators
    sum over 500-1000 blocks; the output, an average over that many keys, is
    small, which makes the relative bound the tight one."""
    w = synth.custom_append(50 + prefix // 16000, [prefix], [16], 32, 128, [0], [0])
    _run(w)
