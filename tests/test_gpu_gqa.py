"""The grouped-query bf16 baseline (mqa_gqa_pack_bf16 + mqa_gqa_decode_bf16)
against the oracle's float path (``oracle.decode_gqa``), on the GPU.

Shapes cover split contexts (few (sequence, KV head) items, so each context
is cut into chunks merged by the second kernel) and unsplit ones, global and
windowed layers, head_dim 128 and 64, ragged and edge contexts (0, 1, page
boundaries), and a permuted page pool.  Bar: max |err| <= 2e-3, relative L2
<= 1e-3.
"""
import numpy as np
import pytest
import torch

import int8_mqa_kv_amd as mk
import oracle
import synth
from tests.gpu_util import assert_parity, log

pytestmark = pytest.mark.gpu

CASES = [
    # (seed, batch, hq, hkv, d, contexts, window)
    (81, 4, 32, 8, 128, [1, 17, 1000, 5000], 0),
    (82, 4, 32, 8, 128, [16, 33, 1025, 3000], 1024),
    (83, 33, 32, 8, 128, [int(x) for x in np.linspace(1, 700, 33)], 0),   # 264 items: unsplit
    (84, 3, 16, 4, 64, [0, 64, 2049], 0),
    (85, 2, 8, 8, 128, [300, 77], 40),                                     # one query head per KV head
]


def bf16(rng, shape):
    bits = synth.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    return bits, oracle.bf16_bits_to_f64(bits)


def run_case(seed, batch, hq, hkv, d, ctx, window):
    rng = np.random.default_rng(seed)
    log(f"gqa case {seed}: B={batch} Hq={hq} Hkv={hkv} d={d} window={window} ctx={ctx}")
    pages = [-(-c // 16) for c in ctx]
    max_pages = max(1, max(pages))
    num_pages = sum(pages) + 1
    perm = rng.permutation(num_pages - 1) + 1          # page 0: never handed out
    bt = np.zeros((batch, max_pages), np.int32)
    k_bits, v_bits, k64, v64, sm = [], [], {}, {}, []
    at = 0
    for b, c in enumerate(ctx):
        ids = perm[at:at + pages[b]]
        at += pages[b]
        bt[b, :pages[b]] = ids
        kb, kf = bf16(rng, (c, hkv, d))
        vb, vf = bf16(rng, (c, hkv, d))
        k_bits.append(kb)
        v_bits.append(vb)
        for h in range(hkv):
            k64[(b, h)], v64[(b, h)] = kf[:, h], vf[:, h]
        pos = np.arange(c)
        sm.append(ids[pos // 16].astype(np.int64) * 16 + pos % 16)
    pool = torch.full((num_pages, mk.gqa_page_bytes(hkv, d)), 0xFF, dtype=torch.uint8,
                      device="cuda")
    if sum(ctx):
        kt = torch.from_numpy(np.concatenate(k_bits).view(np.int16)).cuda().view(torch.bfloat16)
        vt = torch.from_numpy(np.concatenate(v_bits).view(np.int16)).cuda().view(torch.bfloat16)
        mk.gqa_pack_bf16(kt, vt, torch.from_numpy(np.concatenate(sm)).cuda(), pool, hkv)
    qb, q64 = bf16(rng, (batch, hq, d))
    q = torch.from_numpy(qb.view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.full((batch, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    ws = mk.gqa_decode_workspace(batch, hq, hkv, max(ctx), window, d)
    mk.gqa_decode_bf16(q, out, pool, hkv, torch.from_numpy(bt).cuda(),
                       torch.tensor(ctx, dtype=torch.int32, device="cuda"), max(ctx), window,
                       workspace=ws)
    torch.cuda.synchronize()
    want = oracle.decode_gqa(q64, ctx, window, hkv, lambda b, h: (0, k64[(b, h)], v64[(b, h)]))
    assert_parity(out.cpu().numpy(), want, f"gqa case {seed}")


@pytest.mark.parametrize("case", CASES, ids=[f"gqa{c[0]}" for c in CASES])
def test_gqa_decode_matches_the_oracle(case):
    run_case(*case)
