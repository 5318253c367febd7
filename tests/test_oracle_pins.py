"""Pins of the oracle to facts the pages and mathematics fix (CPU only).

Each test would fail for a plausible slip in the oracle: a dropped softmax
scale, a wrong window bound, keys and values swapped, the wrong token's scale,
a wrong rounding rule or divisor in the quantiser, a wrong position for the
query of an append chunk.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from tests import bruteforce

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(seed, n, d, scale=1.0):
    return (np.random.default_rng(seed).standard_normal((n, d)) * scale).astype(np.float32)


# --------------------------------------------------------------------------
# KV byte formula: page 4's worked examples
# --------------------------------------------------------------------------
def _to_bytes(value, unit):
    return value * {"KiB": 1024, "MB": 1e6, "GB": 1e9}[unit]


def test_kv_bytes_worked_examples():
    g = json.load(open(os.path.join(GOLDEN, "kv_bytes_worked_examples.json")))
    for e in g["per_token"]:
        got = oracle.kv_bytes_per_token(e["layers"], e["kv_heads"], e["head_dim"],
                                        e["dtype_bytes"])
        want = _to_bytes(e["printed"], e["unit"])
        assert abs(got - want) <= e["rel_tol"] * want, e["what"]
    for e in g["per_context"]:
        got = oracle.kv_bytes_per_token(e["layers"], e["kv_heads"], e["head_dim"],
                                        e["dtype_bytes"]) * e["tokens"]
        want = _to_bytes(e["printed"], e["unit"])
        assert abs(got - want) <= e["rel_tol"] * want, e["what"]
    for e in g["ratios"]:
        a = oracle.kv_bytes_per_token(e["num"]["layers"], e["num"]["kv_heads"],
                                      e["num"]["head_dim"], e["num"]["dtype_bytes"])
        b = oracle.kv_bytes_per_token(e["den"]["layers"], e["den"]["kv_heads"],
                                      e["den"]["head_dim"], e["den"]["dtype_bytes"])
        assert abs(a / b - e["printed"]) <= e["rel_tol"] * e["printed"] + 1e-12, e["what"]


def test_kv_bytes_exact_values():
    # 36 x 8 x 64 x 2 x 2 = 73,728 exactly; one int8 MQA head at d=128 is 256 B.
    assert oracle.kv_bytes_per_token(36, 8, 64, 2) == 73728
    assert oracle.kv_bytes_per_token(1, 1, 128, 1) == 256


# --------------------------------------------------------------------------
# Quantiser
# --------------------------------------------------------------------------
def test_quantiser_golden_ties():
    g = json.load(open(os.path.join(GOLDEN, "quantiser_ties.json")))
    for row in g["rows"]:
        x = np.array([row["x"]], dtype=np.float32)
        codes, scales = oracle.quantize(x)
        assert scales[0] == np.float32(row["scale"])
        assert codes[0].tolist() == row["codes"]


def _bits_to_f32(hexes):
    return np.array([int(h, 16) for h in hexes], dtype=np.uint32).view(np.float32)


def test_quantiser_near_ties_fix_the_division():
    """Near ties of x / s derived with exact rationals (make_quantiser_near_ties.py):
    the codes of fl32(x / s) differ there from those of x * fl32(1 / s) and of
    x * fl32(127 / a), so only a quantiser that divides passes."""
    g = json.load(open(os.path.join(GOLDEN, "quantiser_near_ties.json")))
    assert len(g["rows"]) >= 4
    n_rec = n_inv = 0
    for row in g["rows"]:
        x = _bits_to_f32(row["x_bits"])[None, :]
        codes, scales = oracle.quantize(x)
        assert scales.view(np.uint32)[0] == int(row["scale_bits"], 16)
        assert codes[0].tolist() == row["codes"]
        n_rec += sum(a != b for a, b in zip(row["codes"], row["codes_if_reciprocal"]))
        n_inv += sum(a != b for a, b in zip(row["codes"], row["codes_if_inverse_scale"]))
    # the file really separates the three forms
    assert n_rec > 0 and n_inv > 0


def test_bf16_bit_patterns():
    """bfloat16 is the top half of an fp32 pattern: fixed values of the format."""
    bits = np.array([0x3F80, 0xC040, 0x0001, 0x7F7F, 0x8000, 0x4049, 0x0080], dtype=np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    want = [1.0, -3.0, 2.0 ** -133, (2.0 - 2.0 ** -7) * 2.0 ** 127, -0.0,
            3.140625, 2.0 ** -126]
    assert got.dtype == np.float64
    for g_, w_ in zip(got.tolist(), want):
        assert g_ == w_ and math.copysign(1, g_) == math.copysign(1, w_)


def test_quantiser_error_bound_and_range():
    x = _rows(1, 4000, 128) * np.float32(3.0)
    codes, s = oracle.quantize(x)
    s64 = s.astype(np.float64)[:, None]
    err = np.abs(x.astype(np.float64) - s64 * codes)
    # rint contributes half a step; the fp32 division x/s at most 128 ulp-units
    assert np.all(err <= s64 * (0.5 + 128 * 2.0 ** -24) * (1 + 1e-12))
    assert codes.min() >= -127 and codes.max() <= 127
    # the element of largest magnitude always maps to +-127
    idx = np.abs(x).argmax(axis=1)
    big = codes[np.arange(x.shape[0]), idx]
    assert np.all(np.abs(big) == 127)
    assert np.all(np.sign(big) == np.sign(x[np.arange(x.shape[0]), idx]))
    # the scale is max|x| / 127 rounded once to fp32
    a = np.abs(x).max(axis=1)
    assert np.all(np.abs(s.astype(np.float64) * 127 - a) <= a * 2.0 ** -24)


def test_quantiser_symmetries():
    x = _rows(2, 500, 64)
    c, s = oracle.quantize(x)
    cn, sn = oracle.quantize(-x)
    assert np.array_equal(cn, -c) and np.array_equal(sn, s)
    c4, s4 = oracle.quantize(x * np.float32(4.0))      # power of two: exact
    assert np.array_equal(c4, c) and np.array_equal(s4, s * np.float32(4.0))
    z, sz = oracle.quantize(np.zeros((3, 64), np.float32))
    assert not z.any() and not sz.any()


def test_dequantize_exact():
    x = _rows(3, 300, 128)
    c, s = oracle.quantize(x)
    d = oracle.dequantize(c, s)
    for t in range(0, 300, 37):
        for ch in range(0, 128, 11):
            # Python ints and floats: exact product as a rational, compared exactly
            assert d[t, ch] == float(s[t]) * int(c[t, ch])


# --------------------------------------------------------------------------
# Attention: closed forms
# --------------------------------------------------------------------------
def _single_history(n, d, seed, kscale=1.0):
    kc, ks = oracle.quantize(_rows(seed, n, d, kscale))
    vc, vs = oracle.quantize(_rows(seed + 1, n, d))
    return kc, ks, vc, vs


def test_identical_keys_give_mean_of_values():
    d, n = 64, 50
    k = np.tile(_rows(5, 1, d), (n, 1))
    kc, ks = oracle.quantize(k)
    vc, vs = oracle.quantize(_rows(6, n, d))
    q = _rows(7, 3, d)
    for w in (0, 1, 7, 50):
        p = n - 1
        out = oracle.attend(q, np.full(3, p), np.full(3, w), 0, kc, ks, vc, vs, 0.125)
        lo = 0 if w == 0 else max(0, p - w + 1)
        mean = oracle.dequantize(vc, vs)[lo:p + 1].mean(axis=0)
        np.testing.assert_allclose(out, np.tile(mean, (3, 1)), rtol=1e-12, atol=1e-13)


def test_single_key_returns_its_value():
    d = 128
    kc, ks, vc, vs = _single_history(1, d, 8)
    q = _rows(9, 4, d) * np.float32(50)
    out = oracle.attend(q, np.zeros(4), np.zeros(4), 0, kc, ks, vc, vs, 1 / math.sqrt(d))
    assert np.array_equal(out, np.tile(oracle.dequantize(vc, vs)[0], (4, 1)))


def test_two_keys_logistic_weights():
    """q = e_0; key 0 is the zero row, key 1 has khat_0 = 8 ln 3 (up to the fp32
    scale), so with d = 64 the score gap is ln 3 and the weights are 1/4 and
    3/4.  A missing or wrong 1/sqrt(d), swapped keys or swapped K/V fail."""
    d = 64
    k = np.zeros((2, d), np.float32)
    k[1, 0] = np.float32(8 * math.log(3))
    kc, ks = oracle.quantize(k)
    v = np.zeros((2, d), np.float32)
    v[0, :] = 127.0                          # scale exactly 1: vhat = 127
    v[1, :] = -127.0
    v[1, 5] = 0.0
    vc, vs = oracle.quantize(v)
    q = np.zeros((1, d), np.float32)
    q[0, 0] = 1.0
    out = oracle.attend(q, [1], [0], 0, kc, ks, vc, vs, 1 / math.sqrt(d))
    want = 0.25 * 127.0 + 0.75 * -127.0
    np.testing.assert_allclose(out[0, 0], want, rtol=1e-6)
    np.testing.assert_allclose(out[0, 5], 0.25 * 127.0, rtol=1e-6)
    # the same query one step earlier sees only key 0
    out0 = oracle.attend(q, [0], [0], 0, kc, ks, vc, vs, 1 / math.sqrt(d))
    assert out0[0, 0] == 127.0


def test_huge_scores_select_the_argmax_key():
    """Scores of order 1e4: the softmax is one-hot on the largest score.  The
    oracle must take the maximum out before exponentiating (exp of such
    scores overflows fp64, giving inf/inf) and return that key's value."""
    d, n = 64, 40
    kc, ks = oracle.quantize(_rows(12, n, d))
    vc, vs = oracle.quantize(_rows(13, n, d))
    q = _rows(14, 3, d) * np.float32(2000)
    out = oracle.attend(q, np.full(3, n - 1), np.zeros(3), 0, kc, ks, vc, vs, 1 / math.sqrt(d))
    assert np.all(np.isfinite(out))
    scores = q.astype(np.float64) @ oracle.dequantize(kc, ks).T / math.sqrt(d)
    assert scores.max() > 1000
    vh = oracle.dequantize(vc, vs)
    for r in range(3):
        top2 = np.sort(scores[r])[-2:]
        assert top2[1] - top2[0] > 40  # the runner-up weighs less than e^-40
        np.testing.assert_allclose(out[r], vh[int(np.argmax(scores[r]))], rtol=0, atol=1e-15)


def test_constant_values_pass_through():
    d, n = 128, 300
    kc, ks, _, _ = _single_history(n, d, 10)
    vc = np.full((n, d), 127, np.int8)
    vs = np.full(n, 0.5, np.float32)
    q = _rows(11, 5, d) * np.float32(4)
    out = oracle.attend(q, np.full(5, n - 1), np.array([0, 1, 3, 1024, 299]), 0,
                        kc, ks, vc, vs, 1 / math.sqrt(d))
    np.testing.assert_allclose(out, 63.5, rtol=1e-13)


def test_window_one_returns_own_value():
    d, n = 64, 40
    kc, ks, vc, vs = _single_history(n, d, 12)
    q = _rows(13, n, d)
    out = oracle.attend(q, np.arange(n), np.ones(n), 0, kc, ks, vc, vs, 0.125)
    assert np.array_equal(out, oracle.dequantize(vc, vs))


def test_keys_outside_window_do_not_matter():
    d, n, w = 128, 200, 17
    kc, ks, vc, vs = _single_history(n, d, 14)
    q = _rows(15, 6, d)
    pos = np.array([199, 150, 100, 16, 17, 5])
    out = oracle.attend(q, pos, np.full(6, w), 0, kc, ks, vc, vs, 1 / math.sqrt(d))
    kc2, vc2 = kc.copy(), vc.copy()
    ks2, vs2 = ks.copy(), vs.copy()
    for r, p in enumerate(pos):
        lo = max(0, p - w + 1)
        # poison everything before lo and after p for this query only
        kc3, vc3, ks3, vs3 = kc2.copy(), vc2.copy(), ks2.copy(), vs2.copy()
        kc3[:lo] = 99; vc3[:lo] = -99; ks3[:lo] = np.nan; vs3[:lo] = np.nan
        kc3[p + 1:] = 99; ks3[p + 1:] = np.inf; vs3[p + 1:] = np.nan
        o = oracle.attend(q[r:r + 1], [p], [w], 0, kc3, ks3, vc3, vs3, 1 / math.sqrt(d))
        assert np.array_equal(o[0], out[r])
    # window >= context is the same as global
    g = oracle.attend(q, pos, np.zeros(6), 0, kc, ks, vc, vs, 1 / math.sqrt(d))
    big = oracle.attend(q, pos, np.full(6, 10_000), 0, kc, ks, vc, vs, 1 / math.sqrt(d))
    assert np.array_equal(g, big)


def test_value_scaling_by_power_of_two_is_exact():
    d, n = 64, 120
    kc, ks, vc, vs = _single_history(n, d, 16)
    q = _rows(17, 4, d)
    pos = np.array([119, 60, 7, 0])
    a = oracle.attend(q, pos, np.zeros(4), 0, kc, ks, vc, vs, 0.125)
    b = oracle.attend(q, pos, np.zeros(4), 0, kc, ks, vc, vs * np.float32(8), 0.125)
    assert np.array_equal(b, a * 8)


def test_key_permutation_invariance_global():
    d, n = 128, 97
    kc, ks, vc, vs = _single_history(n, d, 18)
    q = _rows(19, 8, d)
    a = oracle.attend(q, np.full(8, n - 1), np.zeros(8), 0, kc, ks, vc, vs, 0.088)
    perm = np.random.default_rng(20).permutation(n)
    b = oracle.attend(q, np.full(8, n - 1), np.zeros(8), 0, kc[perm], ks[perm],
                      vc[perm], vs[perm], 0.088)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_history_offset_is_positional():
    """Storing only the tail of the history (key_start > 0) gives the same
    result as storing it all, and a window reaching before the stored part is
    refused."""
    d, n, w = 64, 300, 64
    kc, ks, vc, vs = _single_history(n, d, 21)
    q = _rows(22, 3, d)
    pos = np.array([299, 250, 200])
    full = oracle.attend(q, pos, np.full(3, w), 0, kc, ks, vc, vs, 0.125)
    start = 137
    part = oracle.attend(q, pos, np.full(3, w), start, kc[start:], ks[start:],
                         vc[start:], vs[start:], 0.125)
    assert np.array_equal(full, part)
    with pytest.raises(ValueError):
        oracle.attend(q, pos, np.full(3, 0), start, kc[start:], ks[start:],
                      vc[start:], vs[start:], 0.125)


# --------------------------------------------------------------------------
# Brute force on tiny inputs (explicit mask matrix, no max shift, fsum)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(12))
def test_bruteforce_tiny(seed):
    g = np.random.default_rng(100 + seed)
    d = int(g.choice([2, 4, 8]))
    n = int(g.integers(1, 7))
    heads = int(g.integers(1, 4))
    kc, ks, vc, vs = _single_history(n, d, 200 + seed)
    q = _rows(300 + seed, heads * n, d)
    pos = np.repeat(np.arange(n), heads)
    win = g.integers(0, 4, size=heads * n)
    scale = 1 / math.sqrt(d)
    got = oracle.attend(q, pos, win, 0, kc, ks, vc, vs, scale)
    k_hat = ks.astype(np.float64)[:, None] * kc
    v_hat = vs.astype(np.float64)[:, None] * vc
    want = bruteforce.attend(q, pos, win, np.arange(n), k_hat, v_hat, scale)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_bruteforce_medium():
    d, n = 16, 40
    kc, ks, vc, vs = _single_history(n, d, 400)
    q = _rows(401, 3 * n, d)
    pos = np.repeat(np.arange(n), 3)
    win = np.tile([0, 5, 16], n)
    got = oracle.attend(q, pos, win, 0, kc, ks, vc, vs, 0.25)
    want = bruteforce.attend(q, pos, win, np.arange(n),
                             ks.astype(np.float64)[:, None] * kc,
                             vs.astype(np.float64)[:, None] * vc, 0.25)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# Decode / append composition
# --------------------------------------------------------------------------
def _kv_table(n_slots, batch, n, d, seed):
    table = {}
    for s in range(n_slots):
        for b in range(batch):
            table[(s, b)] = (0,) + _single_history(n, d, seed + 10 * s + b)
    return lambda s, b: table[(s, b)]


def test_append_with_one_token_is_decode():
    d, hq, batch, n = 64, 4, 3, 33
    kv = _kv_table(2, batch, n, d, 500)
    ctx = np.array([33, 20, 1])
    q = _rows(501, 2 * batch * hq, d).reshape(2, batch, hq, d)
    dec = oracle.decode(q, ctx, [0, 1], [0, 8], kv)
    app = oracle.append(q, ctx, np.arange(batch + 1), [0, 1], [0, 8], kv)
    assert np.array_equal(dec, app)


def test_append_chunk_is_a_sequence_of_decodes():
    """Token t of a chunk of n on a prefix P sees exactly what a decode with
    context P + t + 1 sees."""
    d, hq, n_keys = 64, 2, 40
    kv = _kv_table(1, 1, n_keys, d, 600)
    prefix, qlen = 30, 10
    q = _rows(601, qlen * hq, d).reshape(1, qlen, hq, d)
    for w in (0, 4):
        app = oracle.append(q, [prefix + qlen], [0, qlen], [0], [w], kv)
        for t in range(qlen):
            dec = oracle.decode(q[:, t:t + 1], [prefix + t + 1], [0], [w], kv)
            assert np.array_equal(app[:, t], dec[:, 0])


def test_decode_against_bruteforce():
    d, hq, batch, n = 8, 3, 2, 6
    kv = _kv_table(1, batch, n, d, 700)
    ctx = np.array([6, 4])
    q = _rows(701, 2 * batch * hq, d).reshape(2, batch, hq, d)
    out = oracle.decode(q, ctx, [0, 0], [0, 2], kv)
    for li, w in enumerate([0, 2]):
        for b in range(batch):
            _, kc, ks, vc, vs = kv(0, b)
            want = bruteforce.attend(q[li, b], np.full(hq, ctx[b] - 1), np.full(hq, w),
                                     np.arange(n), ks.astype(np.float64)[:, None] * kc,
                                     vs.astype(np.float64)[:, None] * vc, 1 / math.sqrt(d))
            np.testing.assert_allclose(out[li, b], want, rtol=1e-12, atol=1e-13)


def test_append_against_bruteforce():
    d, hq, n = 4, 2, 6
    kv = _kv_table(1, 2, n, d, 800)
    ctx = np.array([6, 5])
    qlens = np.array([3, 4])
    cu = np.array([0, 3, 7])
    q = _rows(801, 7 * hq, d).reshape(1, 7, hq, d)
    for w in (0, 2):
        out = oracle.append(q, ctx, cu, [0], [w], kv)
        for b in range(2):
            _, kc, ks, vc, vs = kv(0, b)
            rows = q[0, cu[b]:cu[b + 1]].reshape(-1, d)
            pos = np.repeat(np.arange(ctx[b] - qlens[b], ctx[b]), hq)
            want = bruteforce.attend(rows, pos, np.full(rows.shape[0], w), np.arange(n),
                                     ks.astype(np.float64)[:, None] * kc,
                                     vs.astype(np.float64)[:, None] * vc, 0.5)
            np.testing.assert_allclose(out[0, cu[b]:cu[b + 1]].reshape(-1, d), want,
                                       rtol=1e-12, atol=1e-13)


def test_shared_slot_equals_separate_calls():
    d, hq, batch, n = 64, 4, 2, 25
    kv = _kv_table(1, batch, n, d, 900)
    ctx = np.array([25, 11])
    q = _rows(901, 3 * batch * hq, d).reshape(3, batch, hq, d)
    together = oracle.decode(q, ctx, [0, 0, 0], [0, 0, 0], kv)
    for li in range(3):
        alone = oracle.decode(q[li:li + 1], ctx, [0], [0], kv)
        assert np.array_equal(together[li], alone[0])
