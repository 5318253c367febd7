"""mqa_decode_step_noalloc -- the decode step with its scratch in the
library's static per-GPU array -- against mqa_decode_step with a caller's
workspace, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input (fewer
sequences, shorter contexts, another layer map), so the second call reuses
the array the first one left: each must store the same pool bytes and return
the same output, bit for bit, as mqa_decode_step on an identical pool, and
match the oracle.
"""
import numpy as np
import pytest
import torch

import int8_mqa_kv_amd as mk
import oracle
import synth
from tests.gpu_util import GpuCase, OracleKV, assert_parity, log, q_tensor
from tests.test_gpu_decode_step import current_rows, garble_positions

pytestmark = pytest.mark.gpu


def _one_call(w, ls, lw):
    log(f"noalloc vs step: B={w.batch} contexts {w.context_lens.tolist()} layers {ls} "
        f"windows {lw}")
    q, q64 = q_tensor(w)
    k_new, v_new = current_rows(w, w.context_lens, torch.float32)
    wsb = mk.decode_workspace_bytes(w.batch, w.num_q_heads, ls, lw, w.max_context, w.head_dim,
                                    w.q_dtype)
    assert 0 < wsb <= mk.DECODE_STATIC_SCRATCH_BYTES, wsb     # the scratch is really used
    a, b = GpuCase(w), GpuCase(w)
    slots = sorted(set(ls))
    garble_positions(a, w, w.context_lens.astype(np.int64) - 1, slots)
    garble_positions(b, w, w.context_lens.astype(np.int64) - 1, slots)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    out_a = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device="cuda")
    out_b = torch.full_like(out_a, float("nan"))
    mk.mqa_decode_step(q, out_a, k_new, v_new, a.pool, a.block_table, a.context_lens,
                       w.max_context, ls, lw, workspace=ws)
    mk.mqa_decode_step_noalloc(q, out_b, k_new, v_new, b.pool, b.block_table, b.context_lens,
                               w.max_context, ls, lw)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b), "output differs from mqa_decode_step's"
    assert torch.equal(a.pool.data, b.pool.data), "stored bytes differ from mqa_decode_step's"
    want = oracle.decode(q64, w.context_lens, ls, lw, OracleKV(w))
    assert_parity(out_b.cpu().numpy(), want, f"noalloc B={w.batch}")


def test_noalloc_matches_decode_step_twice():
    big = synth.custom_decode(70, 6, 32, 128, "bf16", [9000, 20000, 4096, 12345, 700, 16384], 3,
                              0, 5000)
    _one_call(big, [0, 0, 0], [0, 0, 0])
    small = synth.custom_decode(71, 3, 32, 128, "bf16", [5000, 2100, 6000], 2, 0, 2000)
    _one_call(small, [0, 0], [0, 1024])


def test_noalloc_rejects_launches_beyond_its_scratch():
    """A plan needing more scratch than the static array holds is refused
    before anything is enqueued (here: 256 sequences at 256k context)."""
    ls, lw = [0], [0]
    need = mk.decode_workspace_bytes(256, 64, ls, lw, 1 << 18, 128, "bf16")
    assert need > mk.DECODE_STATIC_SCRATCH_BYTES
    q = torch.zeros((1, 256, 64, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    kn = torch.zeros((1, 256, 128), dtype=torch.float32, device="cuda")
    pool = mk.KVPool(16, 128)
    bt = torch.zeros((1, 256, 1 << 14), dtype=torch.int32, device="cuda")
    cl = torch.ones(256, dtype=torch.int32, device="cuda")
    with pytest.raises(mk.MQAError, match="static scratch"):
        mk.mqa_decode_step_noalloc(q, out, kn, kn, pool, bt, cl, 1 << 18, ls, lw)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
