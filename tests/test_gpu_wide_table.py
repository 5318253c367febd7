"""Block tables wider than any context needs.

The kernels bound a context by max_context and by the table's width in
pages times 16 tokens.  At 2^27 pages per row that product no longer fits
32 bits; the bound is taken in 64 bits, so a row that wide still gives the
same result, bit for bit, as the narrow table (the launch plan depends on
max_context, not on the width).  Entries past the sequences' pages hold the
poison page: they are never loaded.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import GpuCase, OracleKV, assert_parity, log, q_tensor

pytestmark = pytest.mark.gpu

WIDE = 1 << 27  # pages per row: 2^31 tokens, past what 32-bit products hold


def _widen(g):
    bt = g.block_table
    wide = torch.full((bt.shape[0], bt.shape[1], WIDE), int(g.w.poison_page), dtype=torch.int32,
                      device=bt.device)
    wide[:, :, :bt.shape[2]] = bt
    return wide


def test_decode_with_a_wide_block_table():
    w = synth.custom_decode(36, 2, 32, 128, "bf16", [1000, 5000], 1, 0, permuted_pool=400)
    log(f"wide table decode: {WIDE} pages per row")
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    narrow = g.decode(q).clone()
    g.block_table = _widen(g)
    wide = g.decode(q)
    assert torch.equal(wide, narrow)
    want = oracle.decode(q64, w.context_lens, w.layer_slot, w.layer_window, OracleKV(w))
    assert_parity(wide.cpu().numpy(), want, "wide table decode")


def test_append_with_a_wide_block_table():
    w = synth.custom_append(37, [700, 3000], [20, 9], 32, 128, [0], [0])
    log(f"wide table append: {WIDE} pages per row")
    g = GpuCase(w)
    q, q64 = q_tensor(w)
    narrow = g.append(q).clone()
    g.block_table = _widen(g)
    wide = g.append(q)
    assert torch.equal(wide, narrow)
    want = oracle.append(q64, w.context_lens, w.cu_q_lens, w.layer_slot, w.layer_window,
                         OracleKV(w))
    assert_parity(wide.cpu().numpy(), want, "wide table append")
