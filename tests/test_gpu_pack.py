"""kv_pack_int8 on the GPU is bit-exact against the oracle's quantiser."""
import json
import os

import numpy as np
import pytest
import torch

import int8_mqa_kv_amd as mk
import oracle
import synth
from tests.gpu_util import log

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pack_and_read(k, v, d, src="f32", pages=None, perm_seed=0):
    """Pack rows k, v [T, d] into pages in a random order; read them back."""
    t = k.shape[0]
    n_pages = pages or (t + 15) // 16 + 3
    g = np.random.default_rng(perm_seed)
    slots = g.permutation(n_pages * 16)[:t].astype(np.int64)
    pool = mk.KVPool(n_pages, d)
    if src == "bf16":
        kb = torch.from_numpy(synth.f32_to_bf16_bits(k).view(np.int16)).cuda().view(torch.bfloat16)
        vb = torch.from_numpy(synth.f32_to_bf16_bits(v).view(np.int16)).cuda().view(torch.bfloat16)
    else:
        kb, vb = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    mk.kv_pack_int8(kb, vb, torch.from_numpy(slots).cuda(), pool)
    torch.cuda.synchronize()
    return mk.unpack_page_tokens(pool.data.cpu().numpy(), slots, d)


def _assert_bitexact(k, v, d, src="f32", seed=0):
    kc, ks, vc, vs = _pack_and_read(k, v, d, src, perm_seed=seed)
    if src == "bf16":  # the oracle quantises the exact upcast of the bf16 rows
        k = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(k))
        v = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(v))
    okc, oks = oracle.quantize(k)
    ovc, ovs = oracle.quantize(v)
    assert np.array_equal(kc, okc), f"K codes differ in {int((kc != okc).sum())} places"
    assert np.array_equal(vc, ovc), f"V codes differ in {int((vc != ovc).sum())} places"
    assert np.array_equal(ks.view(np.uint32), oks.view(np.uint32)), "K scale bits differ"
    assert np.array_equal(vs.view(np.uint32), ovs.view(np.uint32)), "V scale bits differ"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_pack_random_rows_bitexact(d, src):
    log(f"pack random rows d={d} src={src}")
    g = np.random.default_rng(11)
    t = 5000
    k = g.standard_normal((t, d), dtype=np.float32) * np.float32(2.0)
    v = g.standard_normal((t, d), dtype=np.float32)
    k[::7] *= np.float32(1e-3)
    v[::11] *= np.float32(3e4)
    _assert_bitexact(k, v, d, src, seed=d)


@pytest.mark.parametrize("d", [64, 128])
def test_pack_ties_zero_rows_and_extremes(d):
    log(f"pack ties/zeros/extremes d={d}")
    g = json.load(open(os.path.join(GOLDEN, "quantiser_ties.json")))
    rows = []
    for r in g["rows"]:
        x = np.zeros(d, np.float32)
        x[:len(r["x"])] = r["x"]
        rows.append(x)
    gen = np.random.default_rng(3)
    # constructed near-ties: x/s lands on n + 0.5 exactly or one ulp away
    for _ in range(200):
        e = int(gen.integers(-20, 20))
        s = np.float32(2.0 ** e)
        n = gen.integers(-126, 126, size=d).astype(np.float32)
        x = (n + np.float32(0.5)) * s
        x[0] = np.float32(127) * s
        bump = gen.integers(-1, 2, size=d).astype(np.int32)
        x = (x.view(np.int32) + bump).view(np.float32)
        x[0] = np.float32(127) * s
        rows.append(x)
    rows.append(np.full(d, -3.0, np.float32))          # all equal, negative
    rows.append(np.full(d, 1e-30, np.float32))         # tiny
    rows.append(np.full(d, 3e37, np.float32))          # huge
    big = np.zeros(d, np.float32)
    big[d - 1] = -1e-5
    rows.append(big)
    k = np.stack(rows)
    v = k[::-1].copy()
    _assert_bitexact(k, v, d, "f32", seed=5)


def test_pack_skips_negative_slots_and_respects_stride():
    log("pack negative slots")
    d = 128
    g = np.random.default_rng(4)
    k = g.standard_normal((32, d), dtype=np.float32)
    v = g.standard_normal((32, d), dtype=np.float32)
    pool = mk.KVPool(4, d, fill=0x5A)
    slots = np.arange(32, dtype=np.int64)
    slots[5] = -1
    slots[20] = -7
    mk.kv_pack_int8(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                    torch.from_numpy(slots).cuda(), pool)
    torch.cuda.synchronize()
    data = pool.data.cpu().numpy()
    k_off, v_off, ks_off, vs_off = mk.page_layout(d)
    assert np.all(data[0][k_off[5]] == 0x5A) and np.all(data[1][v_off[4]] == 0x5A)
    kc, ks, vc, vs = mk.unpack_page_tokens(data, np.array([0, 6, 19, 21, 31]), d)
    okc, oks = oracle.quantize(k[[0, 6, 19, 21, 31]])
    assert np.array_equal(kc, okc) and np.array_equal(ks, oks)
    # pages 2 and 3 were never addressed
    assert np.all(data[2:] == 0x5A)


@pytest.mark.parametrize("d", [64, 128])
def test_pack_near_ties_match_golden_codes(d):
    """The near-tie rows derived with exact rationals from the quantiser's
    definition (tests/golden/quantiser_near_ties.json): the kernel's codes and
    scale bits equal the file's, not only the oracle's."""
    log(f"pack near-tie golden rows d={d}")
    g = json.load(open(os.path.join(GOLDEN, "quantiser_near_ties.json")))
    rows, want, scales = [], [], []
    for r in g["rows"]:
        x = np.zeros(d, np.float32)
        vals = np.array([int(h, 16) for h in r["x_bits"]], np.uint32).view(np.float32)
        x[:len(vals)] = vals
        rows.append(x)
        c = np.zeros(d, np.int8)
        c[:len(vals)] = r["codes"]
        want.append(c)
        scales.append(int(r["scale_bits"], 16))
    k = np.stack(rows)
    v = -k[::-1].copy()
    kc, ks, vc, vs = _pack_and_read(k, v, d, "f32", perm_seed=9)
    want = np.stack(want)
    assert np.array_equal(kc, want), f"K codes differ in {int((kc != want).sum())} places"
    assert np.array_equal(vc, -want[::-1]), "V codes differ"
    assert ks.view(np.uint32).tolist() == scales
    assert vs.view(np.uint32).tolist() == scales[::-1]
