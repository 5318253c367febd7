"""Host-side memory management of the paged cache, on the CPU: the KV
footprint of a layer map and the page table that recycles windowed slots.

The footprint reproduces the size arguments of "Character.AI: inference
optimization", section 03 (technique table: multi-query attention 8X smaller
than grouped-query, KV shared across layers 2-3x, 1 in 6 layers global with a
1024-token horizon, together more than 20X) on the hybrid-turn model (12
layers, 32 query heads, d=128, 5 local + 1 global per block, the two global
layers sharing one slot), and the per-token formula of "Como funciona a
inferência de IA", section "Qual é o tamanho real do cache KV?" (whose
printed figures pin it in test_oracle_pins / test_abi).

The page table is checked against a plain model of what a step may read:
after every call, the pages a (slot, sequence) holds are exactly the pages
covering its readable tokens, no page is held twice, and held + free pages
always add up to the pool.
"""
import json
import os

import numpy as np
import pytest

import int8_mqa_kv_amd as mk

HERE = os.path.dirname(os.path.abspath(__file__))

# the hybrid-turn model: 5 local (window 1024) + 1 global per 6-layer block,
# 12 layers, the two global layers (5 and 11) sharing slot 10
HYBRID_SLOT = [0, 1, 2, 3, 4, 10, 5, 6, 7, 8, 9, 10]
HYBRID_WINDOW = [1024] * 5 + [0] + [1024] * 5 + [0]
PLAIN_SLOT = list(range(12))          # every layer its own cache
PLAIN_WINDOW = [0] * 12               # every layer global


def fp(slot, window, kv_heads, code_bytes, scale_bytes, ctx, page=0, d=128):
    return mk.kv_footprint_bytes(slot, window, kv_heads, d, code_bytes, scale_bytes, ctx, page)


# ---------------------------------------------------------------- footprint
def test_footprint_reduces_to_the_per_token_formula():
    """One slot per layer, every layer global, no scales: context x
    2 x layers x kv_heads x head_dim x bytes (the Red Hat formula)."""
    for L, h, d, b, ctx in [(36, 8, 64, 2, 2048), (80, 8, 128, 2, 1000), (12, 1, 128, 1, 17)]:
        got = mk.kv_footprint_bytes(list(range(L)), [0] * L, h, d, b, 0, ctx, 0)
        assert got == ctx * mk.kv_bytes_per_token(L, h, d, b) == ctx * 2 * L * h * d * b


def test_footprint_printed_context_sizes():
    """The Red Hat page's per-context sizes for its 120B example (full
    history in half of its 36 layers) come out of the footprint too."""
    g = json.load(open(os.path.join(HERE, "golden", "kv_bytes_worked_examples.json")))
    for e in g["per_context"]:
        L = e["layers"]
        got = mk.kv_footprint_bytes(list(range(L)), [0] * L, e["kv_heads"], e["head_dim"],
                                    e["dtype_bytes"], 0, e["tokens"], 0)
        scale = {"MB": 1e6, "GB": 1e9}[e["unit"]]
        assert abs(got / scale - e["printed"]) <= e["rel_tol"] * e["printed"], e["what"]


def test_mqa_is_eight_times_smaller_than_gqa8():
    """Section 03 table, multi-query row: 8X smaller than grouped-query
    attention (8 KV heads), at any context and for either cache format."""
    for ctx in (1, 100, 4096, 30000):
        for code, scale in ((2, 0), (1, 4)):
            a = fp(HYBRID_SLOT, HYBRID_WINDOW, 8, code, scale, ctx, 16)
            b = fp(HYBRID_SLOT, HYBRID_WINDOW, 1, code, scale, ctx, 16)
            assert a == 8 * b


@pytest.mark.parametrize("share", [2, 3])
def test_sharing_across_layers_divides_by_the_group_size(share):
    """Section 03 table, shared-KV row ('2-3x'): global layers whose KV is
    shared by groups of 2 or 3 neighbours hold 2 or 3 times less."""
    L = 6
    alone = fp(list(range(L)), [0] * L, 1, 1, 4, 20000, 16)
    shared = fp([l // share for l in range(L)], [0] * L, 1, 1, 4, 20000, 16)
    assert alone == share * shared


def test_local_slot_holds_its_window_only():
    """A windowed slot keeps the tokens its window reaches: exactly W (token
    count) or the pages covering them (at most ceil(W/16) + 1 pages)."""
    per_tok = 2 * (128 + 4)
    for ctx in (1, 15, 16, 17, 1023, 1024, 1025, 1040, 1041, 5000, 5007):
        exact = fp([0], [1024], 1, 1, 4, ctx, 0)
        assert exact == min(ctx, 1024) * per_tok
        paged = fp([0], [1024], 1, 1, 4, ctx, 16)
        lo = max(0, ctx - 1024)
        assert paged == ((ctx - 1) // 16 - lo // 16 + 1) * 16 * per_tok
        assert paged <= (1024 // 16 + 1) * 16 * per_tok
    # a slot read by both a windowed and a global layer keeps everything
    assert fp([0, 0], [1024, 0], 1, 1, 4, 5000, 0) == 5000 * per_tok
    # two windows on one slot: the wider one decides
    assert fp([0, 0], [64, 1024], 1, 1, 4, 5000, 0) == 1024 * per_tok


def test_int8_cache_bytes_against_bf16():
    """Section 05 (int8 KV): 2d code bytes + 8 scale bytes per token and slot
    against 4d for bf16 -- 512/264 at d = 128."""
    a = fp(PLAIN_SLOT, PLAIN_WINDOW, 1, 2, 0, 8192, 0)
    b = fp(PLAIN_SLOT, PLAIN_WINDOW, 1, 1, 4, 8192, 0)
    assert a * 264 == b * 512


def test_combined_reduction_exceeds_20x_on_the_hybrid_model():
    """Section 03 and section 01 ('more than 20X'): grouped-query (8 KV heads)
    with every layer global and unshared, against multi-query + 1-in-6 global
    (horizon 1024) + the global pair sharing one slot, same bf16 format.  At
    the hybrid turn's median context (6000 cached + 64 new tokens) the factor
    is well above 20.  Past the window the factor is 96c / (c + 10 x 1024):
    8 for the heads, 12 layers against one global slot plus ten windows of
    1024 tokens; it passes 20 at c = 20 x 10240 / 76 (about 2,695 tokens) and
    tends to 96."""
    def ratio(ctx):
        return (fp(PLAIN_SLOT, PLAIN_WINDOW, 8, 2, 0, ctx, 0)
                / fp(HYBRID_SLOT, HYBRID_WINDOW, 1, 2, 0, ctx, 0))
    assert ratio(6064) > 20
    assert ratio(1024) == pytest.approx(8 * 12 / 11)     # every window still covers everything
    for c in (1025, 2048, 6064, 32768):
        assert ratio(c) == pytest.approx(96 * c / (c + 10240), rel=1e-12)
    assert ratio(2694) < 20 < ratio(2695)
    assert ratio(10 ** 7) == pytest.approx(96, rel=1e-2)
    # the int8 cache (this library's format, paged) multiplies it by ~1.9 more
    ours = fp(HYBRID_SLOT, HYBRID_WINDOW, 1, 1, 4, 6064, 16)
    assert fp(PLAIN_SLOT, PLAIN_WINDOW, 8, 2, 0, 6064, 0) / ours > 40


def test_footprint_rejects_bad_arguments():
    f = mk.lib.mqa_kv_footprint_bytes
    assert f(-1, None, None, 1, 128, 1, 4, 10, 16) == -1
    assert f(1, None, None, 1, 128, 1, 4, 10, 16) == -1
    s = np.array([0], np.int32)
    w = np.array([-1], np.int32)
    assert f(1, s.ctypes.data, w.ctypes.data, 1, 128, 1, 4, 10, 16) == -1
    w[0] = 0
    assert f(1, s.ctypes.data, w.ctypes.data, 1, 128, 1, 4, -5, 16) == -1
    assert f(0, None, None, 1, 128, 1, 4, 10, 16) == 0


# --------------------------------------------------------------- page table
class Model:
    """What a (slot, sequence) must hold: the pages covering the tokens its
    next step may read, given the window and the earliest query."""

    def __init__(self, windows, batch):
        self.windows, self.batch = windows, batch
        self.ctx = [0] * batch
        self.qfirst = [0] * batch

    def needed(self, slot, seq):
        c = self.ctx[seq]
        if c == 0:
            return set()
        w = self.windows[slot]
        lo = 0 if w == 0 else max(0, self.qfirst[seq] + 1 - w)
        return set(range(lo // 16, (c - 1) // 16 + 1))


def check(pt, model, num_pages, first_page, invalid):
    seen = set()
    held_total = 0
    for s in range(pt.num_slots):
        for b in range(pt.batch):
            row = pt.block_table[s, b]
            held = {i for i in range(pt.max_pages) if row[i] != invalid}
            assert held == model.needed(s, b), (s, b)
            assert pt.held_pages(b, s) == len(held)
            ids = row[row != invalid]
            assert np.all((ids >= first_page) & (ids < first_page + num_pages))
            assert not (set(ids.tolist()) & seen), "a page held twice"
            seen |= set(ids.tolist())
            held_total += len(held)
    assert held_total + pt.free_pages() == num_pages


def test_page_table_random_growth_matches_the_model():
    rng = np.random.default_rng(7)
    windows = [0, 64, 1024, 33]
    batch, max_pages, num_pages, first, invalid = 6, 300, 1400, 5, 0
    pt = mk.PageTable(first, num_pages, windows, batch, max_pages, invalid)
    model = Model(windows, batch)
    for step in range(600):
        b = int(rng.integers(batch))
        op = rng.random()
        if op < 0.03:
            pt.release(b)
            model.ctx[b] = model.qfirst[b] = 0
        else:
            c = model.ctx[b]
            grow = int(rng.choice([1, 1, 1, 7, 64, 300])) if c else int(rng.integers(1, 900))
            new = c + grow
            if new > max_pages * 16:
                continue
            try:
                pt.advance(b, new, grow)
            except mk.MQAError:
                # the pool ran short: nothing may have changed
                check(pt, model, num_pages, first, invalid)
                pt.release(b)
                model.ctx[b] = model.qfirst[b] = 0
                continue
            model.ctx[b], model.qfirst[b] = new, new - grow
        check(pt, model, num_pages, first, invalid)


def test_decode_steps_keep_a_local_slot_within_its_window():
    """Decode steps (one new token each): a slot with window W never holds
    more than ceil(W/16) + 1 pages, and recycled pages serve the global slot."""
    W = 100
    pt = mk.PageTable(0, 40, [W, 0], 1, 64, -1)
    pt.advance(0, 10, 10)
    for c in range(11, 300):
        pt.advance(0, c, 1)
        assert pt.held_pages(0, 0) <= -(-W // 16) + 1
        assert pt.held_pages(0, 1) == (c - 1) // 16 + 1
    lo = 299 - W                                   # first token the step at 299 reads
    assert pt.held_pages(0, 0) == (298 // 16) - (lo // 16) + 1
    assert pt.free_pages() == 40 - pt.held_pages(0, 0) - pt.held_pages(0, 1)


def test_exhausted_pool_changes_nothing():
    pt = mk.PageTable(0, 10, [0], 2, 20, -1)
    pt.advance(0, 100, 100)                         # 7 pages
    before = pt.block_table.copy()
    with pytest.raises(mk.MQAError):
        pt.advance(1, 64, 64)                       # 4 pages, 3 free
    assert np.array_equal(pt.block_table, before)
    assert pt.free_pages() == 3 and pt.held_pages(1, 0) == 0
    pt.advance(1, 48, 48)                           # 3 pages fit
    assert pt.free_pages() == 0


def test_freed_pages_of_a_step_serve_its_own_growth():
    """A full pool still advances when the step frees what it needs."""
    pt = mk.PageTable(0, 3, [32], 1, 20, -1)
    pt.advance(0, 48, 48)                           # pages 0..2, pool empty
    assert pt.free_pages() == 0
    pt.advance(0, 49, 1)                            # reads 17..48: frees page 0, needs page 3
    assert pt.held_pages(0, 0) == 3 and pt.free_pages() == 0


def test_page_table_argument_errors():
    with pytest.raises(mk.MQAError):
        mk.PageTable(0, 10, [0], 1, 4, invalid_page=3)     # invalid id inside the range
    with pytest.raises(mk.MQAError):
        mk.PageTable(0, 10, [-1], 1, 4)
    pt = mk.PageTable(0, 50, [0, 16], 2, 8, -1)
    with pytest.raises(mk.MQAError):
        pt.advance(2, 5, 1)                             # no such sequence
    with pytest.raises(mk.MQAError):
        pt.advance(0, 129, 1)                           # beyond max_pages * 16
    with pytest.raises(mk.MQAError):
        pt.advance(0, 5, 0)                             # no new token
    pt.advance(0, 40, 40)
    with pytest.raises(mk.MQAError):
        pt.advance(0, 39, 1)                            # shrinking
    pt.advance(0, 41, 1)
    with pytest.raises(mk.MQAError):
        pt.advance(0, 44, 10)                           # earliest query moved back
    assert pt.held_pages(0, 1) == (40 // 16) - ((41 - 16) // 16) + 1


def test_slot_mapping_follows_the_table():
    pt = mk.PageTable(3, 30, [0, 20], 2, 10, -1)
    pt.advance(1, 70, 70)
    sm = pt.slot_mapping(1, 0, 0, 70)
    row = pt.block_table[0, 1]
    assert np.array_equal(sm, row[np.arange(70) // 16].astype(np.int64) * 16 + np.arange(70) % 16)
    pt.advance(1, 71, 1)                            # slot 1 now reads 51..70
    with pytest.raises(mk.MQAError):
        pt.slot_mapping(1, 1, 0, 1)                 # token 0 of the windowed slot was recycled
    sm = pt.slot_mapping(1, 1, 70, 1)
    assert sm[0] == pt.block_table[1, 1, 4] * 16 + 6


def test_advance_all_equals_one_call_per_sequence():
    """A batch step holds the same table entries as sequence-by-sequence
    calls (which ids: the free-list order differs, as the batch frees before
    it grows), keeps every id unique, and is all or nothing when the pool runs
    short."""
    windows = [0, 48]
    a = mk.PageTable(2, 400, windows, 5, 64, -1)
    b = mk.PageTable(2, 400, windows, 5, 64, -1)
    ctx = np.array([30, 1, 100, 77, 16], np.int64)
    a.advance_all(ctx, ctx.astype(np.int32))
    for s in range(5):
        b.advance(s, int(ctx[s]), int(ctx[s]))
    rng = np.random.default_rng(3)
    for _ in range(120):
        new = rng.integers(0, 3, size=5).astype(np.int32)
        ctx = ctx + new
        a.advance_all(ctx, new)
        for s in range(5):
            if new[s]:
                b.advance(s, int(ctx[s]), int(new[s]))
        assert np.array_equal(a.block_table >= 0, b.block_table >= 0)
        ids = a.block_table[a.block_table >= 0]
        assert ids.size == np.unique(ids).size
        assert a.free_pages() == b.free_pages()
    small = mk.PageTable(0, 6, [0], 2, 20, -1)
    small.advance_all(np.array([48, 32], np.int64), np.array([48, 32], np.int32))  # 3 + 2 pages
    before = small.block_table.copy()
    with pytest.raises(mk.MQAError):
        small.advance_all(np.array([49, 49], np.int64), np.array([1, 17], np.int32))  # 2 more, 1 free
    assert np.array_equal(small.block_table, before) and small.free_pages() == 1
