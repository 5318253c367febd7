"""mqa_decode_attn on the GPU against the oracle (and GPU invariances).

Tolerance: max |gpu - oracle| <= 2e-3 and ||gpu - oracle||_2 / ||oracle||_2 <=
1e-3 over the whole output of each case.
"""
import numpy as np
import pytest
import torch

import int8_mqa_kv_amd as mk
import oracle
import synth
from tests.gpu_util import (GpuCase, OracleKV, assert_parity, log, outlier_q, q_tensor,
                            with_v_gain)

pytestmark = pytest.mark.gpu


def _run_case(w, seqs=None):
    log(f"decode case {w.case}: {w.name} B={w.batch} Hq={w.num_q_heads} d={w.head_dim} "
        f"L={w.num_layers} q={w.q_dtype} maxctx={w.max_context}")
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    out = g.decode(q)
    want = oracle.decode(q64, w.context_lens, w.layer_slot, w.layer_window, OracleKV(w),
                         seqs=seqs)
    got = out.cpu().numpy()
    if seqs is not None:
        got = got[:, seqs]
    return g, q, out, assert_parity(got, want, f"case {w.case}")


def test_case0_tiny_fp32_q():
    _run_case(synth.case0())


def test_case1_local_window_full_size():
    _run_case(synth.case1())


def test_case2_long_context_random_pages_outliers():
    _run_case(synth.case2())


def test_case3_three_layers_share_one_slot():
    _run_case(synth.case3())


EDGE = [
    # (seed, batch, hq, d, q dtype, contexts, layers, window, permuted pool)
    (1, 3, 8, 64, "f32", [1, 15, 16], 1, 0, 0),
    (2, 4, 32, 128, "bf16", [17, 31, 32, 33], 1, 0, 64),
    (3, 3, 32, 128, "bf16", [100, 1000, 2049], 1, 1, 0),
    (4, 3, 32, 128, "bf16", [100, 1000, 2049], 1, 37, 300),
    (5, 2, 32, 128, "bf16", [500, 3000], 1, 5000, 0),
    (6, 5, 48, 128, "bf16", [1, 64, 65, 129, 700], 2, 0, 200),
    (7, 2, 16, 64, "bf16", [33, 1234], 3, 100, 0),
    (8, 2, 32, 128, "f32", [257, 4000], 1, 0, 400),
    (9, 6, 32, 128, "bf16", [6000, 1, 7, 4096, 4097, 12345], 1, 1024, 3000),
]


@pytest.mark.parametrize("case", EDGE, ids=[f"edge{c[0]}" for c in EDGE])
def test_edge_shapes(case):
    seed, batch, hq, d, qd, ctx, layers, window, perm = case
    w = synth.custom_decode(seed, batch, hq, d, qd, ctx, layers, window, permuted_pool=perm)
    _run_case(w)


def test_mixed_windows_sharing_one_slot():
    """Layers with different windows over one slot, plus a second slot."""
    w = synth.custom_decode(20, 4, 32, 128, "bf16", [50, 1500, 3000, 2047], 4, 0,
                            permuted_pool=1000)
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    ls, lw = [0, 0, 0, 0], [0, 1024, 1, 300]
    out = g.decode(q, ls, lw)
    want = oracle.decode(q64, w.context_lens, ls, lw, OracleKV(w))
    assert_parity(out.cpu().numpy(), want, "mixed windows")


def test_softmax_scale_argument():
    w = synth.custom_decode(21, 2, 32, 128, "bf16", [300, 77], 1, 0)
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    out = g.decode(q, scale=0.05)
    want = oracle.decode(q64, w.context_lens, w.layer_slot, w.layer_window, OracleKV(w),
                         softmax_scale=0.05)
    assert_parity(out.cpu().numpy(), want, "scale 0.05")


def test_pages_outside_the_window_are_never_read():
    """Overwrite every page before the window with NaN scales: bitwise the same."""
    w = synth.case1()
    g = GpuCase(w)
    q, _ = q_tensor(w)
    before = g.decode(q).clone()
    _, _, ks_off, vs_off = mk.page_layout(w.head_dim)
    nanb = torch.tensor(np.frombuffer(np.float32(np.nan).tobytes(), np.uint8).copy()).cuda()
    pages = torch.from_numpy(w.block_table[0, :, :(4096 - 1024) // 16].reshape(-1).astype(np.int64)).cuda()
    for j in range(16):
        for b in range(4):
            g.pool.data[pages, int(ks_off[j]) + b] = nanb[b]
            g.pool.data[pages, int(vs_off[j]) + b] = nanb[b]
    after = g.decode(q)
    assert torch.equal(before, after)


def test_page_permutation_invariance_and_determinism():
    """The same logical cache through two different page placements gives
    bitwise-equal output, and a rerun is bitwise equal."""
    a = synth.custom_decode(30, 4, 32, 128, "bf16", [2000, 5000, 123, 4096], 1, 0,
                            permuted_pool=1000)
    b = synth.custom_decode(30, 4, 32, 128, "bf16", [2000, 5000, 123, 4096], 1, 0, permuted_pool=0)
    b.seed_case = a.case  # same rows, different page placement
    b.case = a.case
    ga, gb = GpuCase(a), GpuCase(b)
    assert not np.array_equal(a.block_table, b.block_table)
    q, _ = q_tensor(a)
    oa, ob, oa2 = ga.decode(q), gb.decode(q), ga.decode(q)
    assert torch.equal(oa, ob)
    assert torch.equal(oa, oa2)


def test_shared_launch_equals_separate_launches():
    w = synth.custom_decode(31, 4, 32, 128, "bf16", [3000, 100, 8000, 4500], 3, 0,
                            permuted_pool=2000)
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    together = g.decode(q).cpu().numpy()
    want = oracle.decode(q64, w.context_lens, w.layer_slot, w.layer_window, OracleKV(w))
    assert_parity(together, want, "3 layers in one launch")
    for li in range(3):
        alone = g.decode(q[li:li + 1].contiguous(), [0], [0]).cpu().numpy()
        assert_parity(alone, want[li:li + 1], f"layer {li} alone")
        # the two launches split the keys into different chunks: the same
        # terms summed in another order and against other running maxima
        # (P is carried to 2^-22, the fp32 sums hold the code bias 1152)
        diff = float(np.abs(together[li] - alone[0]).max())
        log(f"  layer {li}: shared launch vs alone max |diff| {diff:.2e}")
        assert diff <= 1e-4


def test_output_only_written_where_expected():
    """Canaries around the output stay intact."""
    w = synth.custom_decode(32, 3, 32, 128, "bf16", [700, 2500, 9000], 1, 0)
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    big = torch.full((q.numel() + 2048,), 12345.0, dtype=torch.float32, device="cuda")
    out = big[1024:1024 + q.numel()].view(tuple(q.shape))
    g.decode(q, out=out)
    assert torch.all(big[:1024] == 12345.0) and torch.all(big[-1024:] == 12345.0)
    want = oracle.decode(q64, w.context_lens, w.layer_slot, w.layer_window, OracleKV(w))
    assert_parity(out.cpu().numpy(), want, "canary case")


def test_workspace_reuse_across_calls():
    """One workspace, zero-filled once, serves many calls (case 2 splits every
    sequence across workgroups): outputs are bitwise equal and every call
    leaves the workspace as the previous one did (arrival counters back at
    zero, the same partial records)."""
    w = synth.case2()
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    first = g.decode(q).clone()
    ws1 = g._ws.clone()
    for _ in range(3):
        again = g.decode(q)
        assert torch.equal(first, again)
    assert torch.equal(g._ws, ws1)


@pytest.mark.parametrize("windows", [[0, 1024], [37, 0, 300]], ids=["global+1024", "mixed"])
def test_loose_host_context_bound(windows):
    """max_context far above every sequence's length, as a host may pass it
    without reading the lengths back (the block table is widened to match, its
    extra entries pointing at the poison page).  The page ids loaded for the
    bound are then wrong for every windowed range and loaded again, and a
    global range fills fewer chunks than the launch plans for."""
    L = len(windows)
    w = synth.custom_decode(12 + L, 5, 32, 128, "bf16", [1, 40, 1500, 5000, 9000], L, 0, 1500)
    log(f"loose bound: windows {windows}, contexts {w.context_lens.tolist()}")
    ls = [0] * L
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    extra = 2000                                  # pages beyond the longest range
    bt = np.concatenate([w.block_table, np.full(w.block_table.shape[:2] + (extra,),
                                                w.poison_page, np.int32)], axis=2)
    bound = bt.shape[2] * 16
    bt_t = torch.from_numpy(np.ascontiguousarray(bt)).cuda()
    ws = mk.decode_workspace(w.batch, w.num_q_heads, ls, windows, bound, w.head_dim,
                             q_dtype=w.q_dtype)
    out = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device="cuda")
    mk.mqa_decode_attn(q, out, g.pool, bt_t, g.context_lens, bound, ls, windows, workspace=ws)
    torch.cuda.synchronize()
    want = oracle.decode(q64, w.context_lens, ls, windows, OracleKV(w))
    assert_parity(out.cpu().numpy(), want, f"loose bound {windows}")


@pytest.mark.parametrize("window", [0, 300], ids=["global", "window300"])
def test_many_ragged_sequences(window):
    """130 sequences of ragged lengths (1 to 1500 tokens), one workgroup per
    (row block, sequence)."""
    ctx = [1 + (37 * i * i + 11 * i) % 1500 for i in range(130)]
    w = synth.custom_decode(20 + (window > 0), 130, 32, 128, "bf16", ctx, 1, window, 0)
    _run_case(w)


@pytest.mark.parametrize("window", [0, 1024], ids=["global", "window1024"])
def test_peaked_softmax(window):
    """q scaled by 16 (exact in bf16): every row's weights concentrate on a
    few keys, so the output sits near single V rows (up to |V| ~ 4.6) and any
    relative rounding of a weight shows in full; the running maximum moves in
    large steps."""
    w = synth.custom_decode(30 + (window > 0), 4, 32, 128, "bf16", [300, 1500, 4096, 9000], 1,
                            window, 2000)
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    q, q64 = q * 16, q64 * 16
    out = g.decode(q)
    want = oracle.decode(q64, w.context_lens, w.layer_slot, w.layer_window, OracleKV(w))
    assert_parity(out.cpu().numpy(), want, f"peaked softmax, window {window}")


@pytest.mark.parametrize("gain", [64, 512])
@pytest.mark.parametrize("window", [0, 1024], ids=["global", "window1024"])
def test_outlier_query_channels(gain, window):
    """bf16 q rows whose four outlier channels are 64 or 512 times the rest:
    a row's power-of-two scale is set by its outliers, so its ordinary
    elements sit far below its largest.  fp16 still holds every bf16 element
    of such a row exactly."""
    w = synth.custom_decode(60 + (window > 0), 4, 32, 128, "bf16", [300, 1500, 4096, 9000], 1,
                            window, 2000)
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    q, q64 = outlier_q(q, q64, gain, 600 + gain)
    out = g.decode(q)
    want = oracle.decode(q64, w.context_lens, w.layer_slot, w.layer_window, OracleKV(w))
    assert_parity(out.cpu().numpy(), want, f"outlier q x{gain}, window {window}")


@pytest.mark.parametrize("window", [0, 1024], ids=["global", "window1024"])
def test_v_scales_over_many_octaves(window):
    """V rows that are zero, then 2^-80 of the usual size, then growing by
    powers of two (see with_v_gain): the running V exponent starts absent,
    is clamped, and moves many times within one wavefront's keys."""
    _run_case(with_v_gain(synth.custom_decode(
        62 + (window > 0), 5, 32, 128, "bf16", [45, 300, 1500, 4096, 9000], 1, window, 2000)))


RAGGED_GLOBAL = {
    # 24 global sequences from 0 to 32768 tokens (empty, single-token, page
    # edges), permuted pool: the longest set the chunk boundaries, the
    # shorter fill fewer chunks
    "lengths_0_to_32k": lambda: synth.custom_decode(
        30, 24, 32, 128, "bf16", [0, 1, 15, 16, 17, 300, 1024, 4095, 4096, 4097, 8000, 16000, 32768,
                                  2, 33, 5000, 12000, 20000, 31000, 100, 7, 64, 65, 9999], 1, 0,
        permuted_pool=40000),
    # 100 sequences of 1 to 6000 tokens, two chunks each at most
    "batch100": lambda: synth.custom_decode(
        31, 100, 32, 128, "bf16", [1 + (53 * i * i + 7 * i) % 6000 for i in range(100)], 1, 0,
        permuted_pool=40000),
    # fp32 q, two layers on one slot (two 16-row blocks each), 40 sequences
    "f32_two_layers": lambda: synth.custom_decode(
        32, 40, 32, 128, "f32", [17 + (97 * i) % 9000 for i in range(40)], 2, 0,
        permuted_pool=30000),
}


def _run_with_empty(w):
    """Parity on the sequences with a context; zeros (the header's rule for a
    length <= 0) on the others."""
    full = [b for b in range(w.batch) if w.context_lens[b] > 0]
    empty = [b for b in range(w.batch) if w.context_lens[b] <= 0]
    _, _, out, _ = _run_case(w, seqs=full)
    if empty:
        assert torch.all(out[:, empty] == 0)


@pytest.mark.parametrize("name", list(RAGGED_GLOBAL))
def test_ragged_global_lengths(name):
    """Global groups split into chunks over sequences of very different
    lengths, empty ones included."""
    _run_with_empty(RAGGED_GLOBAL[name]())


def test_many_sequences_split():
    """200 sequences (0 to 3000 tokens), split into chunks because the
    workgroup target is raised to 1024."""
    mk.decode_tuning(target_wgs=1024)
    try:
        w = synth.custom_decode(33, 200, 32, 128, "bf16",
                                [(41 * i * i + 3 * i) % 3000 for i in range(200)], 1, 0,
                                permuted_pool=40000)
        _run_with_empty(w)
    finally:
        mk.decode_tuning()


@pytest.mark.timeout(600)
def test_decode_at_the_context_bound():
    """One sequence of MQA_MAX_CONTEXT (2^22) tokens, the largest context the
    library accepts, on a permuted pool of 262,241 pages.  The planner's own
    plan splits it into about 500 chunks; a workgroup target of 2^20 forces
    the 2048-chunk cap.  Either way the chunks' page ranges, worked out in
    32-bit arithmetic in the kernel, must tile the 262,144 pages, and the last
    arrival folds every chunk's record.  Both plans are checked against one
    oracle result."""
    w = synth.custom_decode(35, 1, 8, 64, "bf16", [mk.MAX_CONTEXT], 1, 0,
                            permuted_pool=mk.MAX_CONTEXT // 16 + 97)
    log(f"decode at the context bound: ctx {mk.MAX_CONTEXT}, Hq=8, d=64")
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    want = oracle.decode(q64, w.context_lens, w.layer_slot, w.layer_window, OracleKV(w))
    for target in (0, 1 << 20):
        mk.decode_tuning(target_wgs=target)
        try:
            log(f"  workgroup target {target or 'planner'}: workspace "
                f"{mk.decode_workspace_bytes(1, 8, [0], [0], mk.MAX_CONTEXT, 64)} bytes")
            out = g.decode(q)
        finally:
            mk.decode_tuning()
        assert_parity(out.cpu().numpy(), want, f"context bound, target {target}")


@pytest.mark.parametrize("target_wgs", [1, 8])
def test_long_range_per_wavefront(target_wgs):
    """One 32000-token global sequence split over very few workgroups, so each
    wavefront walks 60-250 blocks: the accumulators' code bias is taken out
    between groups of blocks, and the output, an average over 32000 keys,
    stays within the relative bound."""
    mk.decode_tuning(target_wgs=target_wgs)
    try:
        _run_case(synth.custom_decode(34, 1, 32, 128, "bf16", [32000], 1, 0, permuted_pool=2100))
    finally:
        mk.decode_tuning()
