"""mqa_decode_step -- the current token's store fused into decode attention --
on the GPU.

Before each step the current token's bytes in the pool are overwritten with
garbage (NaN scales), so a step that read them back instead of coding the
token itself would fail.  Checked:
  * the pool bytes the step leaves equal what kv_pack_int8 writes (bit-exact);
  * the output equals kv_pack_int8 followed by mqa_decode_attn, bit for bit;
  * the output matches the oracle (max |err| <= 2e-3, relative L2 <= 1e-3).
"""
import numpy as np
import pytest
import torch

import int8_mqa_kv_amd as mk
import oracle
import synth
from tests.gpu_util import GpuCase, OracleKV, assert_parity, log, q_tensor

pytestmark = pytest.mark.gpu


def current_rows(w, ctx, dtype=torch.float32):
    """k_new, v_new [num_slots, B, D]: each slot's row at position ctx[b]-1."""
    ks = np.zeros((w.num_slots, w.batch, w.head_dim), np.float32)
    vs = np.zeros_like(ks)
    for s in range(w.num_slots):
        for b in range(w.batch):
            c = int(ctx[b])
            if c >= 1:
                k, v = w.kv_rows(s, b, c - 1, c)
                ks[s, b], vs[s, b] = k[0], v[0]
    return (torch.from_numpy(ks).cuda().to(dtype), torch.from_numpy(vs).cuda().to(dtype))


def garble_positions(g, w, positions, slots):
    """Overwrite token `positions[b]` of every listed slot: codes 0x5A, NaN scales."""
    k_off, v_off, ks_off, vs_off = mk.page_layout(w.head_dim)
    nan = np.frombuffer(np.float32(np.nan).tobytes(), np.uint8)
    pages, offs, vals = [], [], []
    for s in slots:
        for b in range(w.batch):
            p = int(positions[b])
            if p < 0:
                continue
            page = int(w.block_table[s, b, p // 16])
            j = p % 16
            code_offs = np.concatenate([k_off[j], v_off[j]])
            pages.append(np.full(code_offs.size + 8, page))
            offs.append(np.concatenate([code_offs, ks_off[j] + np.arange(4), vs_off[j] + np.arange(4)]))
            vals.append(np.concatenate([np.full(code_offs.size, 0x5A, np.uint8), nan, nan]))
    if pages:
        pt = torch.from_numpy(np.concatenate(pages)).cuda()
        ot = torch.from_numpy(np.concatenate(offs)).cuda()
        g.pool.data[pt, ot] = torch.from_numpy(np.concatenate(vals)).cuda()
    torch.cuda.synchronize()


def run_step(g, q, k_new, v_new, ctx_t, max_context, ls, lw, ws):
    out = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device="cuda")
    mk.mqa_decode_step(q, out, k_new, v_new, g.pool, g.block_table, ctx_t, max_context, ls, lw,
                       workspace=ws)
    torch.cuda.synchronize()
    return out


def check_step(w, layer_slot=None, layer_window=None, kv_dtype=torch.float32):
    ls = w.layer_slot if layer_slot is None else layer_slot
    lw = w.layer_window if layer_window is None else layer_window
    log(f"decode_step case {w.case}: {w.name} B={w.batch} Hq={w.num_q_heads} d={w.head_dim} "
        f"L={len(ls)} slots={sorted(set(ls))} windows={sorted(set(lw))} kv={kv_dtype}")
    q, q64 = q_tensor(w)
    k_new, v_new = current_rows(w, w.context_lens, kv_dtype)
    ref = GpuCase(w)                     # every position packed by kv_pack_int8
    if kv_dtype != torch.float32:        # the current token as kv_pack_int8 codes bf16 rows
        sm = []
        for s in sorted(set(ls)):
            for b in range(w.batch):
                c = int(w.context_lens[b])
                if c >= 1:
                    sm.append((s, b, int(w.block_table[s, b, (c - 1) // 16]) * 16 + (c - 1) % 16))
        idx = torch.tensor([[s, b] for s, b, _ in sm], device="cuda")
        mk.kv_pack_int8(k_new[idx[:, 0], idx[:, 1]].contiguous(),
                        v_new[idx[:, 0], idx[:, 1]].contiguous(),
                        torch.tensor([x for _, _, x in sm], dtype=torch.int64, device="cuda"),
                        ref.pool)
    want_out = ref.decode(q, ls, lw)

    g = GpuCase(w)
    garble_positions(g, w, w.context_lens.astype(np.int64) - 1, sorted(set(ls)))
    ws = mk.decode_workspace(w.batch, w.num_q_heads, ls, lw, w.max_context, w.head_dim,
                             q_dtype=w.q_dtype)
    out = run_step(g, q, k_new, v_new, g.context_lens, w.max_context, ls, lw, ws)
    assert torch.equal(g.pool.data, ref.pool.data), "pool bytes differ from kv_pack_int8's"
    assert torch.equal(out, want_out), "output differs from kv_pack_int8 + mqa_decode_attn"
    if kv_dtype == torch.float32:
        want = oracle.decode(q64, w.context_lens, ls, lw, OracleKV(w))
        assert_parity(out.cpu().numpy(), want, f"step case {w.case}")
    return g, ws


def test_step_case0_tiny_fp32():
    check_step(synth.case0())


def test_step_case1_full_size():
    check_step(synth.case1())


def test_step_case1_bf16_rows():
    check_step(synth.case1(), kv_dtype=torch.bfloat16)


def test_step_case3_three_layers_one_writer():
    check_step(synth.case3())


def test_step_mixed_windows_on_one_slot():
    w = synth.custom_decode(40, 5, 32, 128, "bf16", [1, 16, 17, 1500, 3001], 4, 0,
                            permuted_pool=800)
    check_step(w, [0, 0, 0, 0], [0, 1024, 1, 300])


STEP_EDGE = [
    # (seed, batch, hq, d, q dtype, contexts, layers, window, permuted pool)
    (41, 6, 8, 64, "f32", [1, 2, 15, 16, 17, 33], 1, 0, 0),
    (42, 4, 48, 128, "bf16", [31, 32, 4097, 9000], 2, 0, 3000),
    (43, 3, 32, 128, "bf16", [100, 2049, 5000], 1, 37, 500),
]


@pytest.mark.parametrize("case", STEP_EDGE, ids=[f"edge{c[0]}" for c in STEP_EDGE])
def test_step_edges(case):
    seed, batch, hq, d, qd, ctx, layers, window, perm = case
    check_step(synth.custom_decode(seed, batch, hq, d, qd, ctx, layers, window,
                                   permuted_pool=perm))


def test_two_steps_in_a_row():
    """Step at ctx-1 stores token ctx-2; the next step (ctx) must read it from
    the pool and store token ctx-1.  Both outputs match the oracle and the
    final pool equals kv_pack_int8's."""
    w = synth.custom_decode(44, 4, 32, 128, "bf16", [18, 1025, 3000, 4096], 2, 0,
                            permuted_pool=2000)
    q, q64 = q_tensor(w)
    ls, lw = w.layer_slot, w.layer_window
    ref = GpuCase(w)
    g = GpuCase(w)
    ctx = w.context_lens.astype(np.int64)
    garble_positions(g, w, ctx - 2, sorted(set(ls)))
    garble_positions(g, w, ctx - 1, sorted(set(ls)))
    ws = mk.decode_workspace(w.batch, w.num_q_heads, ls, lw, w.max_context, w.head_dim,
                             q_dtype=w.q_dtype)
    okv = OracleKV(w)
    for c in (ctx - 1, ctx):
        k_new, v_new = current_rows(w, c)
        ct = torch.from_numpy(c.astype(np.int32)).cuda()
        out = run_step(g, q, k_new, v_new, ct, w.max_context, ls, lw, ws)
        want = oracle.decode(q64, c, ls, lw, okv)
        assert_parity(out.cpu().numpy(), want, f"step at ctx {c.tolist()}")
    assert torch.equal(g.pool.data, ref.pool.data)


def test_step_workspace_reuse_is_deterministic():
    """Case 2 splits every sequence across workgroups: repeated steps on one
    workspace give bitwise-equal outputs and leave the workspace unchanged."""
    w = synth.case2()
    g, ws = check_step(w)
    q, _ = q_tensor(w)
    k_new, v_new = current_rows(w, w.context_lens)
    first = run_step(g, q, k_new, v_new, g.context_lens, w.max_context, w.layer_slot,
                     w.layer_window, ws)
    ws1 = ws.clone()
    for _ in range(3):
        again = run_step(g, q, k_new, v_new, g.context_lens, w.max_context, w.layer_slot,
                         w.layer_window, ws)
        assert torch.equal(first, again)
    assert torch.equal(ws, ws1)
