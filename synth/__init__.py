"""Seeded synthetic workloads for the int8 MQA KV attention path.

This module only draws random numbers and lays out page tables.  It holds none
of the method's arithmetic: no quantisation, no attention, no page-record
addressing.  Both the oracle side and the GPU side of the tests and the bench
take their inputs from here.

Workload shapes follow the five cases the path is measured on:

====  ===============================================================
 0    tiny decode: B=2, 8 query heads, d=64, contexts 100 and 37, fp32 q
 1    local sliding-window decode: B=64, 32 heads, d=128, ctx 4096, W=1024
 2    global long-context decode: B=16, ctx ~ U{8192..32768}, random pages,
      6 of 128 K channels scaled x8 before quantisation
 3    three global layers sharing one KV slot: B=32, 96 query rows, ctx 16384
 4    hybrid append turn: 256 sequences, log-normal cached prefix, 64 new
      tokens, 12 layers (5 local W=1024 + 1 global per block of 6, the two
      global layers sharing one slot)
====  ===============================================================

Seeds: ``np.random.SeedSequence(20240620, spawn_key=(case, stream, ...))`` with
PCG64.  Streams: 0 lengths, 1 page permutation, 2 outlier channels, 3 K rows,
4 V rows, 5 q, 6 poison page.  K/V rows are drawn per (slot, sequence, block of
1024 positions) so any part of any history can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

ENTROPY = 20240620
PAGE_TOKENS = 16          # tokens per KV page
KV_BLOCK = 1024           # positions per independently seeded K/V block

S_LENGTHS, S_PERM, S_OUTLIER, S_K, S_V, S_Q, S_POISON = range(7)


def rng(*spawn_key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(ENTROPY, spawn_key=tuple(int(k) for k in spawn_key))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); return the bits.

    Inputs are finite draws from N(0, 1), so no NaN handling is needed.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def pages_for(n_tokens: int) -> int:
    return -(-int(n_tokens) // PAGE_TOKENS)


@dataclasses.dataclass
class Workload:
    """One synthetic case.  Arrays are host numpy arrays."""
    case: int
    name: str
    kind: str                      # "decode" or "append"
    batch: int
    num_q_heads: int
    head_dim: int
    q_dtype: str                   # "f32" or "bf16"
    layer_slot: np.ndarray         # int32 [L]
    layer_window: np.ndarray       # int32 [L], 0 = global
    num_slots: int
    context_lens: np.ndarray       # int32 [B], keys cached incl. current/chunk
    q_lens: np.ndarray             # int32 [B] (1 per sequence for decode)
    num_pages: int                 # pool pages including the poison page
    poison_page: int
    block_table: np.ndarray        # int32 [num_slots, B, max_pages]
    slot_first_pos: np.ndarray     # int64 [num_slots, B]: first stored position
    outlier_channels: np.ndarray   # int64 [n]: K channels scaled by outlier_gain
    outlier_gain: float = 1.0
    seed_case: Optional[int] = None  # seed namespace (defaults to case)

    # ---------------------------------------------------------------- shapes
    @property
    def num_layers(self) -> int:
        return int(self.layer_slot.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[2])

    @property
    def max_context(self) -> int:
        return int(self.context_lens.max())

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max())

    @property
    def cu_q_lens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    @property
    def total_q(self) -> int:
        return int(self.q_lens.sum())

    def _sk(self) -> int:
        return self.case if self.seed_case is None else self.seed_case

    # ------------------------------------------------------------------ K/V
    def kv_rows(self, slot: int, seq: int, start: int, stop: int
                ) -> Tuple[np.ndarray, np.ndarray]:
        """fp32 K and V rows of (slot, seq) for positions [start, stop)."""
        d = self.head_dim
        n = max(0, stop - start)
        k = np.empty((n, d), dtype=np.float32)
        v = np.empty((n, d), dtype=np.float32)
        if n == 0:
            return k, v
        b0, b1 = start // KV_BLOCK, (stop - 1) // KV_BLOCK
        for blk in range(b0, b1 + 1):
            lo, hi = blk * KV_BLOCK, (blk + 1) * KV_BLOCK
            kb = rng(self._sk(), S_K, slot, seq, blk).standard_normal(
                (KV_BLOCK, d), dtype=np.float32)
            vb = rng(self._sk(), S_V, slot, seq, blk).standard_normal(
                (KV_BLOCK, d), dtype=np.float32)
            a, b = max(lo, start), min(hi, stop)
            k[a - start:b - start] = kb[a - lo:b - lo]
            v[a - start:b - start] = vb[a - lo:b - lo]
        if self.outlier_channels.size:
            k[:, self.outlier_channels] *= np.float32(self.outlier_gain)
        return k, v

    def stored_range(self, slot: int, seq: int) -> Tuple[int, int]:
        """Positions [first, ctx) held in the cache for (slot, seq)."""
        return int(self.slot_first_pos[slot, seq]), int(self.context_lens[seq])

    # -------------------------------------------------------------------- q
    def q_shape(self) -> Tuple[int, int, int, int]:
        rows = self.batch if self.kind == "decode" else self.total_q
        return (self.num_layers, rows, self.num_q_heads, self.head_dim)

    def q_f32(self) -> np.ndarray:
        """Query values as fp32 (bf16-exact when ``q_dtype == 'bf16'``)."""
        shape = self.q_shape()
        out = np.empty(shape, dtype=np.float32)
        for li in range(shape[0]):
            x = rng(self._sk(), S_Q, li).standard_normal(shape[1:], dtype=np.float32)
            if self.q_dtype == "bf16":
                x = bf16_bits_to_f32(f32_to_bf16_bits(x))
            out[li] = x
        return out

    def q_bf16_bits(self) -> np.ndarray:
        assert self.q_dtype == "bf16"
        return f32_to_bf16_bits(self.q_f32())

    # ------------------------------------------------------------ poisoning
    def poison_kv(self) -> Tuple[np.ndarray, np.ndarray]:
        """Random K/V rows for the poison page (its scales are set to NaN by
        whoever writes the pool)."""
        g = rng(self._sk(), S_POISON)
        k = g.standard_normal((PAGE_TOKENS, self.head_dim), dtype=np.float32)
        v = g.standard_normal((PAGE_TOKENS, self.head_dim), dtype=np.float32)
        return k, v

    # ------------------------------------------------------------- counting
    def attended_keys(self) -> int:
        """(slot, sequence, key) triples one call must read, each slot once.

        Decode: each slot's key range is the union over the layers sharing it.
        Append: the union over the chunk's tokens as well.
        """
        total = 0
        for s in sorted(set(int(x) for x in self.layer_slot)):
            wins = [int(self.layer_window[l]) for l in range(self.num_layers)
                    if int(self.layer_slot[l]) == s]
            for b in range(self.batch):
                ctx = int(self.context_lens[b])
                first_q = ctx - int(self.q_lens[b])
                lo = ctx
                for w in wins:
                    lo = min(lo, 0 if w == 0 else max(0, first_q - w + 1))
                total += ctx - lo
        return total


# --------------------------------------------------------------------------
# Page tables
# --------------------------------------------------------------------------
def _tables_in_order(num_slots: int, pages_needed: np.ndarray, first_page: np.ndarray,
                     max_pages: int) -> Tuple[np.ndarray, int, int]:
    """Consecutive page ids, slot-major then sequence-major."""
    nxt = 0
    bt_rows = []
    for s in range(num_slots):
        row = []
        for b in range(pages_needed.shape[1]):
            n = int(pages_needed[s, b]) - int(first_page[s, b])
            row.append(np.arange(nxt, nxt + n, dtype=np.int64))
            nxt += n
        bt_rows.append(row)
    poison = nxt
    bt = np.full((num_slots, pages_needed.shape[1], max_pages), poison, dtype=np.int32)
    for s in range(num_slots):
        for b in range(pages_needed.shape[1]):
            f = int(first_page[s, b])
            bt[s, b, f:f + bt_rows[s][b].size] = bt_rows[s][b]
    return bt, nxt + 1, poison


def _tables_permuted(case: int, num_slots: int, pages_needed: np.ndarray,
                     first_page: np.ndarray, max_pages: int, pool_pages: int
                     ) -> Tuple[np.ndarray, int, int]:
    """Each (slot, seq) gets a consecutive run of a seeded permutation of the
    pool; the poison page is one extra page after the pool."""
    perm = rng(case, S_PERM).permutation(pool_pages).astype(np.int32)
    poison = pool_pages
    bt = np.full((num_slots, pages_needed.shape[1], max_pages), poison, dtype=np.int32)
    off = 0
    for s in range(num_slots):
        for b in range(pages_needed.shape[1]):
            f, n = int(first_page[s, b]), int(pages_needed[s, b])
            cnt = n - f
            if off + cnt > pool_pages:
                raise ValueError("page pool too small")
            bt[s, b, f:n] = perm[off:off + cnt]
            off += cnt
    return bt, pool_pages + 1, poison


# --------------------------------------------------------------------------
# The five cases
# --------------------------------------------------------------------------
def _decode_case(case: int, name: str, batch: int, hq: int, d: int, q_dtype: str,
                 ctx: np.ndarray, n_layers: int, window: int, permuted_pool: int = 0,
                 outliers: int = 0, gain: float = 1.0,
                 seed_case: Optional[int] = None) -> Workload:
    sk = case if seed_case is None else seed_case
    ctx = np.asarray(ctx, dtype=np.int32)
    max_pages = pages_for(int(ctx.max()))
    need = np.array([[pages_for(c) for c in ctx]], dtype=np.int64)
    first = np.zeros_like(need)
    if permuted_pool:
        bt, num_pages, poison = _tables_permuted(sk, 1, need, first, max_pages,
                                                 permuted_pool)
    else:
        bt, num_pages, poison = _tables_in_order(1, need, first, max_pages)
    oc = (np.sort(rng(sk, S_OUTLIER).choice(d, size=outliers, replace=False))
          if outliers else np.zeros(0, dtype=np.int64))
    return Workload(
        case=case, name=name, kind="decode", batch=batch, num_q_heads=hq,
        head_dim=d, q_dtype=q_dtype,
        layer_slot=np.zeros(n_layers, dtype=np.int32),
        layer_window=np.full(n_layers, window, dtype=np.int32), num_slots=1,
        context_lens=ctx, q_lens=np.ones(batch, dtype=np.int32),
        num_pages=num_pages, poison_page=poison, block_table=bt,
        slot_first_pos=np.zeros((1, batch), dtype=np.int64),
        outlier_channels=oc.astype(np.int64), outlier_gain=gain, seed_case=seed_case)


def case0() -> Workload:
    return _decode_case(0, "tiny decode, global, d=64, fp32 q", 2, 8, 64, "f32",
                        np.array([100, 37]), 1, 0)


def case1() -> Workload:
    return _decode_case(1, "local sliding-window decode, W=1024, ctx 4096", 64, 32,
                        128, "bf16", np.full(64, 4096), 1, 1024)


def case2() -> Workload:
    ctx = rng(2, S_LENGTHS).integers(8192, 32768, size=16, endpoint=True)
    return _decode_case(2, "global long-context decode, random pages, K outliers",
                        16, 32, 128, "bf16", ctx, 1, 0, permuted_pool=40000,
                        outliers=round(0.05 * 128), gain=8.0)


def case3() -> Workload:
    return _decode_case(3, "3 global layers sharing one KV slot, ctx 16384", 32, 32,
                        128, "bf16", np.full(32, 16384), 3, 0, permuted_pool=40000)


def case4(batch: int = 256, q_len: int = 64) -> Workload:
    """Hybrid append turn after a cross-turn cache hit."""
    case = 4
    z = rng(case, S_LENGTHS).standard_normal(batch)
    prefix = np.clip(np.rint(6000.0 * np.exp(0.6 * z)), 512, 32768).astype(np.int64)
    ctx = (prefix + q_len).astype(np.int32)
    layer_window = np.array(([1024] * 5 + [0]) * 2, dtype=np.int32)
    layer_slot = np.array([0, 1, 2, 3, 4, 10, 5, 6, 7, 8, 9, 10], dtype=np.int32)
    num_slots = 11
    max_pages = pages_for(int(ctx.max()))
    need = np.zeros((num_slots, batch), dtype=np.int64)
    first = np.zeros((num_slots, batch), dtype=np.int64)
    for s in range(num_slots):
        w = int(layer_window[list(layer_slot).index(s)])
        for b in range(batch):
            need[s, b] = pages_for(int(ctx[b]))
            if w > 0:
                first[s, b] = max(0, int(prefix[b]) - w + 1) // PAGE_TOKENS
    total = int((need - first).sum())
    pool = int(np.ceil(1.25 * total))
    bt, num_pages, poison = _tables_permuted(case, num_slots, need, first, max_pages,
                                             pool)
    return Workload(
        case=case, name="hybrid append turn, 12 layers, shared global pair",
        kind="append", batch=batch, num_q_heads=32, head_dim=128, q_dtype="bf16",
        layer_slot=layer_slot, layer_window=layer_window, num_slots=num_slots,
        context_lens=ctx, q_lens=np.full(batch, q_len, dtype=np.int32),
        num_pages=num_pages, poison_page=poison, block_table=bt,
        slot_first_pos=(first * PAGE_TOKENS).astype(np.int64),
        outlier_channels=np.zeros(0, dtype=np.int64))


CASES = {0: case0, 1: case1, 2: case2, 3: case3, 4: case4}


def case(i: int) -> Workload:
    return CASES[i]()


def custom_decode(seed_case: int, batch: int, hq: int, d: int, q_dtype: str,
                  ctx: Sequence[int], n_layers: int = 1, window: int = 0,
                  permuted_pool: int = 0, outliers: int = 0,
                  gain: float = 1.0) -> Workload:
    """A decode case of any shape (edge cases and sweeps); its own seed space."""
    return _decode_case(100 + seed_case, f"custom decode {seed_case}", batch, hq, d,
                        q_dtype, np.asarray(ctx), n_layers, window,
                        permuted_pool=permuted_pool, outliers=outliers, gain=gain)


def custom_append(seed_case: int, prefix: Sequence[int], q_lens: Sequence[int],
                  hq: int, d: int, layer_window: Sequence[int],
                  layer_slot: Sequence[int], q_dtype: str = "bf16",
                  permuted: bool = True) -> Workload:
    """An append case of any shape; local slots store only what their window
    can reach, like the hybrid turn."""
    case = 100 + seed_case
    prefix = np.asarray(prefix, dtype=np.int64)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    ctx = (prefix + q_lens).astype(np.int32)
    batch = prefix.shape[0]
    layer_window = np.asarray(layer_window, dtype=np.int32)
    layer_slot = np.asarray(layer_slot, dtype=np.int32)
    num_slots = int(layer_slot.max()) + 1
    max_pages = pages_for(int(ctx.max()))
    need = np.zeros((num_slots, batch), dtype=np.int64)
    first = np.zeros((num_slots, batch), dtype=np.int64)
    for s in range(num_slots):
        wins = [int(layer_window[l]) for l in range(layer_slot.size)
                if int(layer_slot[l]) == s]
        for b in range(batch):
            need[s, b] = pages_for(int(ctx[b]))
            if wins and min(wins) > 0:
                first[s, b] = max(0, int(prefix[b]) - max(wins) + 1) // PAGE_TOKENS
    if permuted:
        total = int((need - first).sum())
        bt, num_pages, poison = _tables_permuted(case, num_slots, need, first,
                                                 max_pages, int(np.ceil(1.25 * total)) + 1)
    else:
        bt, num_pages, poison = _tables_in_order(num_slots, need, first, max_pages)
    return Workload(
        case=case, name=f"custom append {seed_case}", kind="append", batch=batch,
        num_q_heads=hq, head_dim=d, q_dtype=q_dtype, layer_slot=layer_slot,
        layer_window=layer_window, num_slots=num_slots, context_lens=ctx,
        q_lens=q_lens, num_pages=num_pages, poison_page=poison, block_table=bt,
        slot_first_pos=(first * PAGE_TOKENS).astype(np.int64),
        outlier_channels=np.zeros(0, dtype=np.int64))
