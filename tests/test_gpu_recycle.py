"""Decode steps over a pool whose windowed-slot pages are recycled, on the GPU.

Four sequences grow token by token through mqa_decode_step, with one layer
reading a local slot (window 64) and one a global slot.  Before each step the
page table (mqa_page_table_advance_all, one call for the batch) frees the local pages that fell behind
the window and hands out pages for the new token; the pool is too small to
hold every page without that.  The pool starts as 0xFF bytes (NaN scales), so
a step that read a page nobody wrote would give NaN; a step that read a
recycled page now holding another sequence's tokens would give wrong values.
Every step's output is compared with the oracle over the full history
(max |err| <= 2e-3, relative L2 <= 1e-3).
"""
import numpy as np
import pytest
import torch

import int8_mqa_kv_amd as mk
import oracle
import synth
from tests.gpu_util import assert_parity, log, q_tensor

pytestmark = pytest.mark.gpu

WINDOW = 64
START = [20, 70, 130, 200]
STEPS = 60
HQ, D = 32, 128


def rows(w, slot, seq, start, stop):
    """fp32 K, V rows of positions [start, stop) (seeded per slot, sequence)."""
    return w.kv_rows(slot, seq, start, stop)


def test_decode_steps_on_recycled_pages():
    batch = len(START)
    final = [c + STEPS for c in START]
    w = synth.custom_decode(61, batch, HQ, D, "bf16", final, 2, 0)
    layer_slot, layer_window = [0, 1], [WINDOW, 0]
    max_pages = -(-max(final) // 16)
    # pages the two slots need at the end without recycling, and with it
    need_all = 2 * sum(-(-c // 16) for c in final)
    need_recycled = sum(-(-c // 16) for c in final) + batch * (-(-WINDOW // 16) + 1)
    num_pages = (need_all + need_recycled) // 2
    assert need_recycled <= num_pages < need_all
    log(f"recycle: B={batch} window={WINDOW} steps={STEPS} pool={num_pages} pages "
        f"(without recycling {need_all})")

    pool = mk.KVPool(num_pages + 1, D, fill=0xFF)        # page 0 stays poison
    pt = mk.PageTable(1, num_pages, [WINDOW, 0], batch, max_pages, invalid_page=0)
    ctx = list(START)
    # prefill: every position of both slots, coded by kv_pack_int8
    for b in range(batch):
        pt.advance(b, ctx[b], ctx[b])
        for s in range(2):
            k, v = rows(w, s, b, 0, ctx[b])
            sm = torch.from_numpy(pt.slot_mapping(b, s, 0, ctx[b])).cuda()
            mk.kv_pack_int8(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), sm, pool)
    torch.cuda.synchronize()

    q, q64 = q_tensor(w)
    ws = mk.decode_workspace(batch, HQ, layer_slot, layer_window, max(final), D, q_dtype=w.q_dtype)
    cache = {}

    def kv_source(slot, seq):
        c = ctx[seq]
        key = (slot, seq, c)
        if key not in cache:
            k, v = rows(w, slot, seq, 0, c)
            kc, ksc = oracle.quantize(k)
            vc, vsc = oracle.quantize(v)
            cache[key] = (0, kc, ksc, vc, vsc)
        return cache[key]

    recycled_any = False
    for step in range(STEPS):
        k_new = np.zeros((2, batch, D), np.float32)
        v_new = np.zeros_like(k_new)
        for b in range(batch):
            ctx[b] += 1
        pt.advance_all(ctx, [1] * batch)          # one step of the batch
        for b in range(batch):
            # fewer local pages than the history spans: some went back to the pool
            recycled_any |= pt.held_pages(b, 0) < -(-ctx[b] // 16)
            for s in range(2):
                k, v = rows(w, s, b, ctx[b] - 1, ctx[b])
                k_new[s, b], v_new[s, b] = k[0], v[0]
        bt = torch.from_numpy(pt.block_table).cuda()
        cl = torch.tensor(ctx, dtype=torch.int32, device="cuda")
        out = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device="cuda")
        mk.mqa_decode_step(q, out, torch.from_numpy(k_new).cuda(), torch.from_numpy(v_new).cuda(),
                           pool, bt, cl, max(final), layer_slot, layer_window, workspace=ws)
        torch.cuda.synchronize()
        want = oracle.decode(q64, ctx, layer_slot, layer_window, kv_source)
        assert_parity(out.cpu().numpy(), want, f"recycled step {step} ctx {ctx}")
        for b in range(batch):
            assert pt.held_pages(b, 0) <= -(-WINDOW // 16) + 1
    assert recycled_any, "no local page was ever freed"
    assert pt.free_pages() >= 0
