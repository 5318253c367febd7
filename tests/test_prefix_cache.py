"""The cross-turn prefix cache on the CPU (host-only mode: entries written and
read with memcpy, no GPU): longest-prefix lookup over a radix tree of pages,
least-recently-used eviction of leaves, and the rule that a windowed slot
only needs the pages its window reaches ("Character.AI: inference
optimization", section 04, cache between turns; section 03, local layers).
"""
import numpy as np
import pytest

import int8_mqa_kv_amd as mk

D = 128
PB = mk.page_bytes(D)
RING = 256 * 1024


def arena_for(entries, slots):
    """Arena bytes for `entries` cached (page, slot) pairs."""
    return RING + entries * (-(-PB // 256) * 256)


def pages_for(tokens, slots, seed):
    n = len(tokens) // 16
    return np.random.default_rng(seed).integers(0, 256, (n, slots, PB), dtype=np.uint8)


def full(slots):
    return (1 << slots) - 1


def test_insert_then_read_back_is_exact():
    c = mk.PrefixCache(arena_for(30, 2), [0, 64], D, host_only=True)
    t = np.arange(200, dtype=np.int32)
    pg = pages_for(t, 2, 1)
    pres = np.full(len(pg), full(2), np.uint64)
    pres[:4] = 1                               # the windowed slot's first pages were recycled
    assert c.insert_host(t, pg, pres) == 12
    out, got = c.read_host(t, 12)
    assert np.array_equal(got, pres)
    assert np.array_equal(out[:, 0], pg[:, 0]) and np.array_equal(out[4:, 1], pg[4:, 1])
    assert not out[:4, 1].any()                # absent pages read back as zeros
    assert c.entries() == 12 + 8 and c.capacity() == 30   # one entry per cached (page, slot)


def test_longest_prefix_and_branches():
    c = mk.PrefixCache(arena_for(64, 1), [0], D, host_only=True)
    rng = np.random.default_rng(2)
    a = rng.integers(0, 50000, 200).astype(np.int32)
    c.insert_host(a, pages_for(a, 1, 3), np.full(12, 1, np.uint64))
    assert c.lookup(np.concatenate([a, [1, 2, 3]])) == 192
    assert c.lookup(a) == 192                  # (200-1)//16 = 12 pages
    assert c.lookup(a[:193]) == 192
    assert c.lookup(a[:192]) == 176            # the last token is left to compute
    assert c.lookup(a[:100]) == 96
    assert c.lookup(a[:16]) == 0
    # a dialogue that shares the first 70 tokens, then differs
    b = np.concatenate([a[:70], rng.integers(0, 50000, 130)]).astype(np.int32)
    assert c.lookup(b) == 64
    c.insert_host(b, pages_for(b, 1, 4), np.full(12, 1, np.uint64))
    assert c.entries() == 12 + 12 - 4          # the first four pages are shared
    assert c.lookup(b) == 192 and c.lookup(a) == 192


def test_same_page_under_another_prefix_does_not_match():
    c = mk.PrefixCache(arena_for(8, 1), [0], D, host_only=True)
    p1, p2, p3 = (np.full(16, v, np.int32) for v in (1, 2, 3))
    x = np.concatenate([p1, p2, [9]])
    y = np.concatenate([p3, p2, [9]])
    c.insert_host(x, pages_for(x, 1, 5), np.ones(2, np.uint64))
    assert c.lookup(x) == 32
    assert c.lookup(y) == 0


def test_lru_evicts_leaves_and_keeps_prefixes_whole():
    c = mk.PrefixCache(arena_for(10, 1), [0], D, host_only=True)
    rng = np.random.default_rng(6)
    a = rng.integers(0, 1000, 97).astype(np.int32)          # 6 pages
    b = rng.integers(1000, 2000, 97).astype(np.int32)       # 6 pages, disjoint
    c.insert_host(a, pages_for(a, 1, 7), np.ones(6, np.uint64))
    c.insert_host(b, pages_for(b, 1, 8), np.ones(6, np.uint64))
    # B needed 6 entries with 4 free: A's two last pages (its leaves) went
    assert c.entries() == 10 and c.stats()["entries_evicted"] == 2
    assert c.lookup(a) == 64 and c.lookup(b) == 96
    # every cached page still has its whole prefix: reads of each length work
    for k in range(1, 5):
        c.read_host(a, k)
    # touch A, then insert C (3 pages): B's leaves are now the oldest
    c.lookup(a)
    cc = rng.integers(2000, 3000, 49).astype(np.int32)
    c.insert_host(cc, pages_for(cc, 1, 9), np.ones(3, np.uint64))
    assert c.lookup(a) == 64 and c.lookup(b) == 48 and c.lookup(cc) == 48


def test_insert_larger_than_the_arena_stops_cleanly():
    c = mk.PrefixCache(arena_for(10, 1), [0], D, host_only=True)
    t = np.arange(16 * 15 + 1, dtype=np.int32)
    assert c.insert_host(t, pages_for(t, 1, 10), np.ones(15, np.uint64)) == 10
    assert c.lookup(t) == 160 and c.entries() == 10


def test_windowed_slot_needs_only_its_window():
    """Slot 0 global, slot 1 windowed (W = 32).  A step whose earliest query
    is token 16P reads slot 1 from 16P + 1 - 32 on."""
    c = mk.PrefixCache(arena_for(40, 2), [0, 32], D, host_only=True)
    t = np.arange(201, dtype=np.int32)                       # 12 full pages
    pres = np.full(12, 1, np.uint64)                          # global everywhere
    pres[10:] |= 2                                            # windowed: last two pages only
    c.insert_host(t, pages_for(t, 2, 11), pres)
    assert c.lookup(t) == 192                                 # P=12 reads slot 1 from page 10
    # the same history known only up to page 8 for the windowed slot
    c2 = mk.PrefixCache(arena_for(40, 2), [0, 32], D, host_only=True)
    pres2 = np.full(12, 1, np.uint64)
    pres2[6:8] |= 2
    c2.insert_host(t, pages_for(t, 2, 12), pres2)
    assert c2.lookup(t) == 128                                # P=8 reads pages 6, 7
    # a global page missing caps the match at it
    c3 = mk.PrefixCache(arena_for(40, 2), [0, 32], D, host_only=True)
    pres3 = np.full(12, 3, np.uint64)
    pres3[5] = 2
    c3.insert_host(t, pages_for(t, 2, 13), pres3)
    assert c3.lookup(t) == 80
    # a history whose windowed slot kept only page 12 (tokens 192..207):
    # restarting at token 208 needs tokens 177.. (page 11 on), and every
    # earlier boundary needs earlier pages still, so nothing matches
    c4 = mk.PrefixCache(arena_for(40, 2), [0, 32], D, host_only=True)
    t4 = np.arange(210, dtype=np.int32)
    pres4 = np.full(13, 1, np.uint64)
    pres4[12:] |= 2
    c4.insert_host(t4, pages_for(t4, 2, 15), pres4)
    assert c4.lookup(t4) == 0


def test_stats_count_asked_and_matched_tokens():
    c = mk.PrefixCache(arena_for(16, 1), [0], D, host_only=True)
    t = np.arange(100, dtype=np.int32)
    c.insert_host(t, pages_for(t, 1, 14), np.ones(6, np.uint64))
    c.lookup(t)
    c.lookup(np.arange(500, 600, dtype=np.int32))
    s = c.stats()
    assert s["lookups"] == 2 and s["tokens_asked"] == 200 and s["tokens_matched"] == 96
    assert s["entries_inserted"] == 6


def test_argument_errors():
    with pytest.raises(mk.MQAError):
        mk.PrefixCache(1000, [0], D, host_only=True)          # no room for one entry
    with pytest.raises(mk.MQAError):
        mk.PrefixCache(arena_for(4, 1), [0], 96, host_only=True)
    c = mk.PrefixCache(arena_for(4, 1), [0], D, host_only=True)
    with pytest.raises(mk.MQAError):
        c.read_host(np.arange(64, dtype=np.int32), 2)        # nothing cached
    pool = mk.KVPool.__new__(mk.KVPool)                       # never used: the call fails first
    pool._c = mk._Pool(0, 4, D, 0)
    with pytest.raises(mk.MQAError):                          # host-only: no GPU copies
        c.restore(np.arange(64, dtype=np.int32), 32, pool, np.zeros((1, 1, 4), np.int32), 0,
                  stream=0)
