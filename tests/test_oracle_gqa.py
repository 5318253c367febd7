"""Pins of the oracle's grouped-query float path (``attend_float``,
``decode_gqa``), the baseline of "Character.AI: inference optimization",
section 03 (multi-query against grouped-query attention).  CPU only.

The float path is written independently of the C int8 oracle; where both
apply (integer K/V values with unit scales) they must agree, and the closed
forms of softmax attention must hold."""
import numpy as np

import oracle


def test_float_path_equals_the_int8_oracle_on_integer_values():
    rng = np.random.default_rng(1)
    n, d, r = 300, 64, 9
    kc = rng.integers(-127, 128, (n, d)).astype(np.int8)
    vc = rng.integers(-127, 128, (n, d)).astype(np.int8)
    q = rng.standard_normal((r, d)) * 0.05
    pos = rng.integers(0, n, r)
    win = np.array([0, 1, 5, 64, 300, 0, 17, 2, 1000])
    ones = np.ones(n, np.float32)
    want = oracle.attend(q, pos, win, 0, kc, ones, vc, ones, 0.125)
    got = oracle.attend_float(q, pos, win, 0, kc.astype(np.float64), vc.astype(np.float64), 0.125)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_float_path_closed_forms():
    rng = np.random.default_rng(2)
    d = 16
    v = rng.standard_normal((5, d))
    k = np.tile(rng.standard_normal(d), (5, 1))
    q = rng.standard_normal((1, d))
    # identical keys: the mean of V
    np.testing.assert_allclose(oracle.attend_float(q, [4], [0], 0, k, v, 0.3)[0], v.mean(0),
                               rtol=1e-12)
    # a window of one: the query's own value
    np.testing.assert_allclose(oracle.attend_float(q, [2], [1], 0, rng.standard_normal((5, d)), v,
                                                   0.3)[0], v[2], rtol=1e-12)
    # two keys whose scores differ by ln 3: weights 1/4, 3/4
    k2 = np.zeros((2, d))
    k2[1, 0] = np.log(3.0)
    q2 = np.zeros((1, d))
    q2[0, 0] = 1.0
    np.testing.assert_allclose(oracle.attend_float(q2, [1], [0], 0, k2, v[:2], 1.0)[0],
                               0.25 * v[0] + 0.75 * v[1], rtol=1e-12)


def test_gqa_groups_query_heads_on_their_kv_head():
    """Query head j reads KV head j // group: with one KV head it is
    multi-query attention, and every head equals a direct call."""
    rng = np.random.default_rng(3)
    b, hq, hkv, d = 2, 8, 2, 32
    ctx = [40, 7]
    q = rng.standard_normal((b, hq, d))
    hist = {(s, h): (rng.standard_normal((40, d)), rng.standard_normal((40, d)))
            for s in range(b) for h in range(hkv)}
    out = oracle.decode_gqa(q, ctx, 16, hkv, lambda s, h: (0, *hist[(s, h)]))
    for s in range(b):
        for j in range(hq):
            k, v = hist[(s, j // (hq // hkv))]
            want = oracle.attend_float(q[s, j:j + 1], [ctx[s] - 1], [16], 0, k, v,
                                       oracle.default_scale(d))
            np.testing.assert_allclose(out[s, j], want[0], rtol=1e-12)
    one = oracle.decode_gqa(q, ctx, 0, 1, lambda s, h: (0, *hist[(s, 0)]))
    for j in range(hq):
        k, v = hist[(0, 0)]
        np.testing.assert_allclose(one[0, j], oracle.attend_float(q[0, j:j + 1], [39], [0], 0, k, v,
                                                                  oracle.default_scale(d))[0])
    assert not oracle.decode_gqa(q, [0, 0], 0, hkv, lambda s, h: (0, *hist[(s, h)])).any()
