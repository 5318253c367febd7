"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import int8_mqa_kv_amd as mk

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "mqa_kv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "sizeof")))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"kv_pack_int8", "mqa_decode_attn", "mqa_append_attn"} <= set(names)
    lib = ctypes.CDLL(mk.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_version_and_sizes():
    assert mk.lib.mqa_abi_version() == 5
    assert mk.page_bytes(128) == 32 * 128 + 128 == 4224
    assert mk.page_bytes(64) == 2176
    assert mk.lib.mqa_page_bytes(96) == 0
    # page-4 formula; one int8 MQA head at d=128 is 256 code bytes per token
    assert mk.kv_bytes_per_token(36, 8, 64, 2) == 73728
    assert mk.kv_bytes_per_token(1, 1, 128, 1) == 256
    assert mk.lib.mqa_kv_bytes_per_token(-1, 1, 1, 1) == -1


@pytest.mark.parametrize("d", [64, 128])
def test_page_layout_is_a_bijection(d):
    k, v, ks, vs = mk.page_layout(d)
    allo = np.concatenate([k.ravel(), v.ravel()] +
                          [ks + b for b in range(4)] + [vs + b for b in range(4)])
    assert np.array_equal(np.sort(allo), np.arange(mk.page_bytes(d)))
    assert k.min() == 0 and k.max() == 16 * d - 1
    assert v.min() == 16 * d and v.max() == 32 * d - 1
    # lane (i, g) reads 16 consecutive bytes at 16*(16g+i) (+1024*h): token i,
    # channels g*D/4 + 16h .. +15
    for lane in (0, 5, 17, 63):
        i, g = lane % 16, lane // 16
        for h in range(d // 64):
            ch = g * (d // 4) + 16 * h + np.arange(16)
            assert np.array_equal(k[i, ch], 1024 * h + 16 * lane + np.arange(16))
    # V: lane (i, g), channel tile t: the 4 bytes of tokens 4g..4g+3, channel 16t+i
    for lane in (0, 9, 33, 62):
        i, g = lane % 16, lane // 16
        for t in range(d // 16):
            got = v[4 * g:4 * g + 4, 16 * t + i]
            base = 16 * d + 1024 * (t // 4) + 16 * lane + 4 * (t % 4)
            assert np.array_equal(got, base + np.arange(4))


def _pool(d=128, pages=10):
    return mk._Pool(0x10000, pages, d, 0)


def _call_decode(**kw):
    args = dict(q=0x1000, q_dtype=mk.MQA_BF16, out=0x2000, pool=_pool(), bt=0x3000,
                max_pages=256, ctx=0x4000, max_context=4096, batch=64, hq=32, layers=1,
                slots=1, layer_slot=[0], layer_window=[1024], scale=0.0, ws=None, ws_bytes=0)
    args.update(kw)
    ls = np.asarray(args["layer_slot"], np.int32)
    lw = np.asarray(args["layer_window"], np.int32)
    rc = mk.lib.mqa_decode_attn(args["q"], args["q_dtype"], args["out"], ctypes.byref(args["pool"]),
                                args["bt"], args["max_pages"], args["ctx"], args["max_context"],
                                args["batch"], args["hq"], args["layers"], args["slots"],
                                ls.ctypes.data, lw.ctypes.data, args["scale"], args["ws"],
                                args["ws_bytes"], None)
    return rc, mk.lib.mqa_last_error().decode()


@pytest.mark.parametrize("kw,code,text", [
    (dict(pool=mk._Pool(0x10000, 10, 96, 0)), mk.MQA_ERR_UNSUPPORTED, "head_dim"),
    (dict(pool=mk._Pool(0x10010, 10, 128, 0)), mk.MQA_ERR_INVALID, "aligned"),
    (dict(pool=mk._Pool(0x10000, 0, 128, 0)), mk.MQA_ERR_INVALID, "pages"),
    (dict(q_dtype=7), mk.MQA_ERR_UNSUPPORTED, "dtype"),
    (dict(batch=0), mk.MQA_ERR_INVALID, "batch"),
    (dict(layer_slot=[1]), mk.MQA_ERR_INVALID, "layer_slot"),
    (dict(layer_window=[-1]), mk.MQA_ERR_INVALID, "layer_window"),
    (dict(max_pages=10), mk.MQA_ERR_INVALID, "max_pages"),
    (dict(q=0), mk.MQA_ERR_INVALID, "non-NULL"),
    (dict(q=0x1002), mk.MQA_ERR_INVALID, "aligned"),
    (dict(layer_window=[0], max_context=32768, max_pages=2048, batch=16),
     mk.MQA_ERR_WORKSPACE, "workspace"),
    (dict(max_context=mk.MAX_CONTEXT + 1, max_pages=mk.MAX_CONTEXT // 16 + 1),
     mk.MQA_ERR_UNSUPPORTED, "max_context"),
    (dict(batch=1 << 24, max_pages=64, max_context=1024), mk.MQA_ERR_UNSUPPORTED,
     "launch too large"),
    (dict(scale=float("nan")), mk.MQA_ERR_INVALID, "softmax_scale"),
    (dict(scale=float("inf")), mk.MQA_ERR_INVALID, "softmax_scale"),
    (dict(scale=3e38), mk.MQA_ERR_INVALID, "softmax_scale"),
])
def test_decode_rejects_bad_arguments(kw, code, text):
    rc, msg = _call_decode(**kw)
    assert rc == code and text in msg


def test_decode_workspace_sizes():
    # short local window: one chunk per sequence, no workspace
    ws1 = mk.decode_workspace_bytes(64, 32, [0], [1024], 4096, 128)
    ws2 = mk.decode_workspace_bytes(16, 32, [0], [0], 32768, 128)
    # several chunks per sequence: an 8 MiB prefix of arrival counters, then
    # partial records (16 (row tile, channel tile) pairs x 288 fp32 each at
    # d = 128, at least two records per sequence)
    assert ws2 % 256 == 0
    assert ws2 >= (8 << 20) + 16 * 2 * 16 * 288 * 4
    assert mk.lib.mqa_decode_workspace_bytes(0, 32, 1, None, None, 4096, 128, mk.MQA_BF16) == 0
    # fp32 queries take 16-row blocks: twice the items, half the chunks each
    # here (the same 256 partial records)
    assert mk.decode_workspace_bytes(16, 32, [0], [0], 32768, 128, 'f32') == ws2
    with pytest.raises(ValueError):
        mk.decode_workspace_bytes(16, 32, [0], [0], 32768, 128, 'f16')
    assert ws1 >= 0


def test_decode_context_bound():
    """max_context is accepted up to MQA_MAX_CONTEXT (2^22 tokens), where the
    kernels' page and chunk arithmetic still fits 32 bits, and refused above.
    The chunk count per item is capped at 2048 even when the workgroup target
    asks for more, which keeps the per-chunk page ranges in the same range."""
    assert mk.MAX_CONTEXT == 1 << 22
    at = mk.decode_workspace_bytes(1, 32, [0], [0], mk.MAX_CONTEXT, 128)
    assert at > 0
    assert mk.decode_workspace_bytes(1, 32, [0], [0], mk.MAX_CONTEXT + 1, 128) == 0
    rec = 16 * 288 * 4  # one partial record: 16 (row tile, channel tile) pairs x 288 fp32
    mk.decode_tuning(target_wgs=1 << 20)
    try:
        assert mk.decode_workspace_bytes(1, 32, [0], [0], mk.MAX_CONTEXT, 128) == (8 << 20) + 2048 * rec
    finally:
        mk.decode_tuning()
    assert mk.decode_workspace_bytes(1, 32, [0], [0], mk.MAX_CONTEXT, 128) == at


def test_gqa_context_bound():
    """The grouped-query baseline takes the same bound on max_context."""
    at = mk.lib.mqa_gqa_decode_workspace_bytes(1, 32, 8, mk.MAX_CONTEXT, 0, 128)
    assert at > 0
    assert mk.lib.mqa_gqa_decode_workspace_bytes(1, 32, 8, mk.MAX_CONTEXT + 1, 0, 128) == 0
    assert "max_context" in mk.lib.mqa_last_error().decode()
    # 2^21 sequences x 8 KV heads: 2^24 workgroups of 512 work-items, past one dispatch
    assert mk.lib.mqa_gqa_decode_workspace_bytes(1 << 21, 32, 8, 1024, 0, 128) == 0
    assert "launch too large" in mk.lib.mqa_last_error().decode()


def _ws_with_waves(args, waves):
    mk.decode_tuning(waves=waves)
    try:
        return mk.decode_workspace_bytes(*args)
    finally:
        mk.decode_tuning()


def test_decode_workgroup_shape_choice():
    """Four-wavefront workgroups (two per CU) only where eight leave CUs idle
    while already splitting every item.  The choice shows in the workspace
    size: the two shapes split items into different chunk counts, so they need
    different numbers of partial records."""
    three_layers_one_slot = (32, 32, [0, 0, 0], [0, 0, 0], 16384, 128)  # 96 items x 2: 192 of 256 CUs
    ragged_130 = (130, 32, [0], [0], 1500, 128)                        # 130 items, kept whole
    local_64 = (64, 32, [0], [1024], 4096, 128)                         # 128 items x 2 chunks
    global_16 = (16, 32, [0], [0], 32768, 128)                          # 16 items x 16 chunks
    auto = mk.decode_workspace_bytes(*three_layers_one_slot)
    assert auto == _ws_with_waves(three_layers_one_slot, 4) != _ws_with_waves(three_layers_one_slot, 8)
    for args in (ragged_130, local_64, global_16):
        auto = mk.decode_workspace_bytes(*args)
        assert auto == _ws_with_waves(args, 8) != _ws_with_waves(args, 4), args
    # 96 items: 2 chunks of 8 wavefronts or 5 of 4 (partial records of 16 pairs x 288 fp32)
    rec = 16 * 288 * 4
    assert _ws_with_waves(three_layers_one_slot, 8) == (8 << 20) + 96 * 2 * rec
    assert _ws_with_waves(three_layers_one_slot, 4) == (8 << 20) + 96 * 5 * rec


@pytest.mark.parametrize("kw", [dict(waves=6), dict(waves=-4), dict(rows=24), dict(target_wgs=-1)])
def test_decode_tuning_rejects_bad_values(kw):
    before = mk.decode_workspace_bytes(32, 32, [0, 0, 0], [0, 0, 0], 16384, 128)
    with pytest.raises(mk.MQAError):
        mk.decode_tuning(**kw)
    assert mk.decode_workspace_bytes(32, 32, [0, 0, 0], [0, 0, 0], 16384, 128) == before


def test_pack_rejects_bad_arguments():
    rc = mk.lib.kv_pack_int8(0x1000, 0x2000, 5, 4, 128, 0x3000, ctypes.byref(_pool()), None)
    assert rc == mk.MQA_ERR_UNSUPPORTED
    rc = mk.lib.kv_pack_int8(0x1000, 0x2000, mk.MQA_F32, 4, 64, 0x3000, ctypes.byref(_pool()), None)
    assert rc == mk.MQA_ERR_INVALID and "row_stride" in mk.lib.mqa_last_error().decode()
    rc = mk.lib.kv_pack_int8(0x1000, 0x2000, mk.MQA_F32, 0, 128, 0x3000, ctypes.byref(_pool()), None)
    assert rc == mk.MQA_OK
    # one call packs at most MQA_PACK_MAX_TOKENS = 2^25 tokens (a launch holds 2^32 - 1
    # work-items, 64 per token)
    rc = mk.lib.kv_pack_int8(0x1000, 0x2000, mk.MQA_F32, (1 << 25) + 1, 128, 0x3000,
                             ctypes.byref(_pool()), None)
    assert rc == mk.MQA_ERR_UNSUPPORTED and "per call" in mk.lib.mqa_last_error().decode()
    rc = mk.lib.mqa_gqa_pack_bf16(0x1000, 0x2000, (1 << 22) + 1, 0x3000, 0x4000, 10, 8, 128, None)
    assert rc == mk.MQA_ERR_UNSUPPORTED and "per call" in mk.lib.mqa_last_error().decode()


def test_append_rejects_bad_arguments():
    ls = np.zeros(1, np.int32)
    lw = np.zeros(1, np.int32)
    rc = mk.lib.mqa_append_attn(0x1000, mk.MQA_BF16, 0x2000, ctypes.byref(_pool()), 0x3000, 64,
                                0x4000, None, 1024, 64, 64, 1, 32, 1, 1, ls.ctypes.data,
                                lw.ctypes.data, 0.0, None)
    assert rc == mk.MQA_ERR_INVALID and "cu_q_lens" in mk.lib.mqa_last_error().decode()
    # 2^20 sequences x 1024 tokens: 2^27 workgroups of 512 work-items, past one dispatch
    cu = 0x5000
    rc = mk.lib.mqa_append_attn(0x1000, mk.MQA_BF16, 0x2000, ctypes.byref(_pool()), 0x3000, 64,
                                0x4000, cu, 1024, 1024, 1 << 30, 1 << 20, 32, 1, 1,
                                ls.ctypes.data, lw.ctypes.data, 0.0, None)
    assert rc == mk.MQA_ERR_UNSUPPORTED and "launch too large" in mk.lib.mqa_last_error().decode()
    rc = mk.lib.mqa_append_attn(0x1000, mk.MQA_BF16, 0x2000, ctypes.byref(_pool()), 0x3000, 64,
                                0x4000, 0x5000, 1024, 64, 64, 1, 32, 1, 1, ls.ctypes.data,
                                lw.ctypes.data, float("nan"), None)
    assert rc == mk.MQA_ERR_INVALID and "softmax_scale" in mk.lib.mqa_last_error().decode()
    big = mk.MAX_CONTEXT + 1
    rc = mk.lib.mqa_append_attn(0x1000, mk.MQA_BF16, 0x2000, ctypes.byref(_pool()), 0x3000,
                                big // 16 + 1, 0x4000, 0x5000, big, 64, 64, 1, 32, 1, 1,
                                ls.ctypes.data, lw.ctypes.data, 0.0, None)
    assert rc == mk.MQA_ERR_UNSUPPORTED and "max_context" in mk.lib.mqa_last_error().decode()


def test_unpack_roundtrip_on_host():
    """The host-side reader inverts the library's layout (no GPU involved)."""
    d = 64
    k_off, v_off, ks_off, vs_off = mk.page_layout(d)
    g = np.random.default_rng(0)
    kc = g.integers(-127, 128, (16, d)).astype(np.int8)
    vc = g.integers(-127, 128, (16, d)).astype(np.int8)
    ks = g.random(16).astype(np.float32)
    vs = g.random(16).astype(np.float32)
    page = np.zeros(mk.page_bytes(d), np.uint8)
    page[k_off] = (kc.astype(np.int16) + 128).astype(np.uint8)  # codes stored as c + 128
    page[v_off] = (vc.astype(np.int16) + 128).astype(np.uint8)
    for j in range(16):
        page[ks_off[j]:ks_off[j] + 4] = np.frombuffer(ks[j].tobytes(), np.uint8)
        page[vs_off[j]:vs_off[j] + 4] = np.frombuffer(vs[j].tobytes(), np.uint8)
    pool = np.stack([np.zeros_like(page), page])
    a, b, c, e = mk.unpack_page_tokens(pool, 16 + np.arange(16), d)
    assert np.array_equal(a, kc) and np.array_equal(b, ks)
    assert np.array_equal(c, vc) and np.array_equal(e, vs)


def test_probe_rejects_bad_arguments():
    """Host-side checks of mqa_hbm_read_probe run before any launch."""
    rc = mk.lib.mqa_hbm_read_probe(0x1000, 24, 0x2000, mk.PROBE_SINK_WORDS, None)
    assert rc == mk.MQA_ERR_INVALID and "multiple of 16" in mk.lib.mqa_last_error().decode()
    rc = mk.lib.mqa_hbm_read_probe(0x1000, 0, 0x2000, mk.PROBE_SINK_WORDS, None)
    assert rc == mk.MQA_ERR_INVALID
    rc = mk.lib.mqa_hbm_read_probe(0x1000, 4096, 0x2000, mk.PROBE_SINK_WORDS - 1, None)
    assert rc == mk.MQA_ERR_INVALID and "sink_words" in mk.lib.mqa_last_error().decode()
    rc = mk.lib.mqa_hbm_read_probe(0x1008, 4096, 0x2000, mk.PROBE_SINK_WORDS, None)
    assert rc == mk.MQA_ERR_INVALID and "aligned" in mk.lib.mqa_last_error().decode()
    rc = mk.lib.mqa_hbm_read_probe(None, 4096, 0x2000, mk.PROBE_SINK_WORDS, None)
    assert rc == mk.MQA_ERR_INVALID


def test_noalloc_step_rejects_launches_beyond_its_scratch():
    """mqa_decode_step_noalloc plans on the host and refuses a launch whose
    scratch exceeds its static array before it touches the device."""
    pool = mk._Pool(0x100000, 16, 128, 0)
    ls, lw = np.zeros(1, np.int32), np.zeros(1, np.int32)
    args = (0x1000, mk.MQA_BF16, 0x2000, 0x3000, 0x4000, mk.MQA_F32, ctypes.byref(pool), 0x5000,
            1 << 14, 0x6000, 1 << 18, 256, 64, 1, 1, ls.ctypes.data, lw.ctypes.data, 0.0, None)
    assert mk.lib.mqa_decode_step_noalloc(*args) == mk.MQA_ERR_WORKSPACE
    assert "static scratch" in mk.lib.mqa_last_error().decode()
    bad = list(args)
    bad[5] = 7
    assert mk.lib.mqa_decode_step_noalloc(*bad) == mk.MQA_ERR_UNSUPPORTED


def test_header_compiles_as_c_and_cpp():
    """include/mqa_kv.h is a C header usable from C11 and C++17 callers."""
    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                       "mqa_kv.h")
    for cmd in (["gcc", "-std=c11", "-Wall", "-Wextra", "-pedantic", "-fsyntax-only", "-x", "c", hdr],
                ["g++", "-std=c++17", "-Wall", "-Wextra", "-fsyntax-only", "-x", "c++", hdr]):
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0 and not r.stderr.strip(), r.stderr
