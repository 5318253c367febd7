"""The cross-turn prefix cache on the GPU: offload, lookup, restore, append.

An earlier turn of each dialogue was computed into pool A: every position of
a global slot and, after a decode step, only the last pages of a windowed
slot (W = 64; the page table recycled the rest).  Its full pages are
offloaded to the host arena (mqa_prefix_cache_insert, device -> host).  The
next turn starts on another server's pool B (0xFF bytes: NaN scales), with
other page ids: the longest usable prefix is looked up, its pages restored
(mqa_prefix_cache_restore, host -> device), the rest of the dialogue packed,
and the new chunk attended with mqa_append_attn.  Checked:
  * restored pages equal the offloaded ones byte for byte;
  * the chunk's output matches the oracle over the full history (max |err|
    <= 2e-3, relative L2 <= 1e-3).
"""
import numpy as np
import pytest
import torch

import int8_mqa_kv_amd as mk
import oracle
import synth
from tests.gpu_util import assert_parity, log

pytestmark = pytest.mark.gpu

HQ, D, W = 32, 128, 64
EARLIER = [100, 230, 37, 1000]     # tokens of each dialogue's earlier turn
NEW = [20, 5, 40, 64]              # tokens of the new message


def test_offload_restore_append():
    batch = len(EARLIER)
    final = [a + b for a, b in zip(EARLIER, NEW)]
    layer_slot, layer_window = [0, 1], [0, W]
    slot_window = [0, W]
    w = synth.custom_decode(71, batch, HQ, D, "bf16", final, 2, 0)
    max_pages = -(-max(final) // 16)
    rng = np.random.default_rng(72)
    tokens = [rng.integers(0, 32000, n).astype(np.int32) for n in final]

    def pack(pool, pt, b, start, stop):
        for s in range(2):
            k, v = w.kv_rows(s, b, start, stop)
            sm = torch.from_numpy(pt.slot_mapping(b, s, start, stop - start)).cuda()
            mk.kv_pack_int8(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), sm, pool)

    # ---- the earlier turn on pool A, then offloaded
    pages_a = 2 * sum(-(-n // 16) for n in EARLIER)
    pool_a = mk.KVPool(pages_a, D)
    pt_a = mk.PageTable(0, pages_a, slot_window, batch, max_pages)
    for b, n in enumerate(EARLIER):
        pt_a.advance(b, n, n)
        pack(pool_a, pt_a, b, 0, n)
        pt_a.advance(b, n, 1)          # a decode step recycles the windowed slot's early pages
    torch.cuda.synchronize()
    cache = mk.PrefixCache(64 << 20, slot_window, D)
    for b, n in enumerate(EARLIER):
        assert cache.insert(tokens[b][:n], pool_a, pt_a.block_table, b) == n // 16
    torch.cuda.synchronize()

    # ---- the new turn on pool B
    pages_b = 2 * sum(-(-n // 16) for n in final) + 8
    pool_b = mk.KVPool(pages_b + 3, D, fill=0xFF)
    pt_b = mk.PageTable(3, pages_b, slot_window, batch, max_pages, invalid_page=0)
    matched = [cache.lookup(t) for t in tokens]
    for b, n in enumerate(EARLIER):
        # every full page of the earlier turn is usable: the windowed slot
        # still held the pages its window reaches
        assert matched[b] == (n // 16) * 16, (b, matched[b])
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    for b in range(batch):
        pt_b.advance(b, final[b], final[b] - matched[b])
    t0.record()
    for b in range(batch):
        cache.restore(tokens[b], matched[b], pool_b, pt_b.block_table, b, invalid_page=0)
    t1.record()
    torch.cuda.synchronize()
    restored = cache.stats()["entries_restored"]
    gbs = restored * mk.page_bytes(D) / (t0.elapsed_time(t1) * 1e-3) / 1e9
    log(f"prefix cache: restored {restored} pages ({restored * mk.page_bytes(D) / 1e6:.2f} MB) "
        f"at {gbs:.1f} GB/s host -> device")

    a_bytes = pool_a.data.cpu().numpy()
    b_bytes = pool_b.data.cpu().numpy()
    for b in range(batch):
        for s in range(2):
            for k in range(matched[b] // 16):
                dst = pt_b.block_table[s, b, k]
                if dst == 0:
                    continue                  # not needed by this step (outside the window)
                src = pt_a.block_table[s, b, k]
                assert src >= 0, "restored a page the earlier turn did not hold"
                assert np.array_equal(b_bytes[dst], a_bytes[src]), (b, s, k)

    # ---- the rest of the dialogue, then the new chunk's attention
    for b in range(batch):
        pack(pool_b, pt_b, b, matched[b], final[b])
    q_lens = [f - m for f, m in zip(final, matched)]
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    total_q = int(cu[-1])
    qf = rng.standard_normal((2, total_q, HQ, D)).astype(np.float32)
    bits = synth.f32_to_bf16_bits(qf)
    q = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    q64 = oracle.bf16_bits_to_f64(bits)
    out = torch.full((2, total_q, HQ, D), float("nan"), dtype=torch.float32, device="cuda")
    bt = torch.from_numpy(pt_b.block_table).cuda()
    cl = torch.tensor(final, dtype=torch.int32, device="cuda")
    mk.mqa_append_attn(q, out, pool_b, bt, cl, torch.from_numpy(cu).cuda(), max(final),
                       max(q_lens), layer_slot, layer_window)
    torch.cuda.synchronize()

    memo = {}

    def kv_source(slot, seq):
        if (slot, seq) not in memo:
            k, v = w.kv_rows(slot, seq, 0, final[seq])
            kc, ksc = oracle.quantize(k)
            vc, vsc = oracle.quantize(v)
            memo[(slot, seq)] = (0, kc, ksc, vc, vsc)
        return memo[(slot, seq)]

    want = oracle.append(q64, final, cu, layer_slot, layer_window, kv_source)
    assert_parity(out.cpu().numpy(), want, "append after restore")
    cache.close()
