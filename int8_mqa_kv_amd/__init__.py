"""int8 multi-query KV-cache attention for AMD Instinct MI355X (gfx950).

A thin Python binding over ``libmqa_kv.so`` (C ABI in ``include/mqa_kv.h``).
Every step of the path runs in the library's HIP kernels; this module only
turns torch tensors into pointers and sizes, and torch only provides device
memory and streams.  The library must be built (``python -m
int8_mqa_kv_amd.build``); importing fails loudly when it is not.

Entry points (same names as the C ABI):
  kv_pack_int8      quantise new K/V rows to int8 + fp32 scales into pages
  mqa_decode_attn   one decode step over the paged int8 cache
  mqa_decode_step   kv_pack_int8 of the current token fused into mqa_decode_attn
  mqa_append_attn   causal attention of an appended chunk on a cached prefix
Host-side memory management (no GPU work except the prefix cache's copies):
  kv_footprint_bytes  KV bytes a sequence holds for a layer map
  PageTable           page table recycling windowed-slot pages (mqa_page_table_*)
  PrefixCache         cross-turn prefix cache in pinned host memory (mqa_prefix_cache_*)
Baseline: gqa_pack_bf16 / gqa_decode_bf16, grouped-query bf16 decode (mqa_gqa_*).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
# torch ships its own HIP runtime under the same soname as ROCm's
# (libamdhip64.so.7).  Loading torch first makes the library below bind to
# that one runtime; loading the library first would bring up a second runtime
# that sees no device once torch initialises its own.
import torch  # noqa: F401  (import order matters, see above)

__all__ = [
    "PAGE_TOKENS", "MAX_CONTEXT", "MQAError", "KVPool", "lib", "page_bytes", "kv_bytes_per_token",
    "page_layout", "kv_pack_int8", "decode_workspace_bytes", "decode_workspace",
    "mqa_decode_attn", "mqa_decode_step", "mqa_decode_step_noalloc", "DECODE_STATIC_SCRATCH_BYTES",
    "mqa_append_attn", "slot_mapping_for", "unpack_page_tokens",
    "kv_footprint_bytes", "PageTable", "PrefixCache",
    "gqa_page_bytes", "gqa_pack_bf16", "gqa_decode_workspace", "gqa_decode_bf16",
    "PROBE_SINK_WORDS", "hbm_read_probe",
]

PAGE_TOKENS = 16
MAX_CONTEXT = 1 << 22  # MQA_MAX_CONTEXT: the largest max_context decode and append accept
_HERE = os.path.dirname(os.path.abspath(__file__))
# MQA_KV_LIB selects another build of the library (the host-sanitizer build
# of the CPU checks); by default the gfx950 build beside this file.
LIB_PATH = os.environ.get("MQA_KV_LIB") or os.path.join(_HERE, "libmqa_kv.so")

MQA_OK, MQA_ERR_INVALID, MQA_ERR_UNSUPPORTED, MQA_ERR_WORKSPACE, MQA_ERR_HIP = 0, -1, -2, -3, -4
MQA_F32, MQA_BF16 = 0, 1


class MQAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


class _Pool(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("num_pages", ctypes.c_int64),
                ("head_dim", ctypes.c_int32), ("reserved", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m int8_mqa_kv_amd.build` "
                          "(hipcc, gfx950) before using the HIP path")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, p, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    f32 = ctypes.c_float
    L.mqa_abi_version.argtypes, L.mqa_abi_version.restype = [], ctypes.c_int
    L.mqa_last_error.argtypes, L.mqa_last_error.restype = [], ctypes.c_char_p
    L.mqa_page_bytes.argtypes, L.mqa_page_bytes.restype = [i32], sz
    L.mqa_kv_bytes_per_token.argtypes, L.mqa_kv_bytes_per_token.restype = [i32, i32, i32, i32], i64
    L.mqa_page_offset.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i64)]
    L.mqa_page_offset.restype = ctypes.c_int
    L.kv_pack_int8.argtypes = [p, p, ctypes.c_int, i64, i64, p, ctypes.POINTER(_Pool), p]
    L.kv_pack_int8.restype = ctypes.c_int
    L.mqa_decode_workspace_bytes.argtypes = [i32, i32, i32, p, p, i32, i32, ctypes.c_int]
    L.mqa_decode_workspace_bytes.restype = sz
    L.mqa_decode_tuning.argtypes = [i32, i32, i32]
    L.mqa_decode_tuning.restype = ctypes.c_int
    L.mqa_decode_attn.argtypes = [p, ctypes.c_int, p, ctypes.POINTER(_Pool), p, i32, p, i32, i32,
                                  i32, i32, i32, p, p, f32, p, sz, p]
    L.mqa_decode_attn.restype = ctypes.c_int
    L.mqa_decode_step.argtypes = [p, ctypes.c_int, p, p, p, ctypes.c_int, ctypes.POINTER(_Pool), p,
                                  i32, p, i32, i32, i32, i32, i32, p, p, f32, p, sz, p]
    L.mqa_decode_step.restype = ctypes.c_int
    L.mqa_decode_step_noalloc.argtypes = [p, ctypes.c_int, p, p, p, ctypes.c_int,
                                          ctypes.POINTER(_Pool), p, i32, p, i32, i32, i32, i32,
                                          i32, p, p, f32, p]
    L.mqa_decode_step_noalloc.restype = ctypes.c_int
    L.mqa_append_attn.argtypes = [p, ctypes.c_int, p, ctypes.POINTER(_Pool), p, i32, p, p, i32,
                                  i32, i32, i32, i32, i32, i32, p, p, f32, p]
    L.mqa_append_attn.restype = ctypes.c_int
    L.mqa_kv_footprint_bytes.argtypes = [i32, p, p, i32, i32, i32, i32, i64, i32]
    L.mqa_kv_footprint_bytes.restype = i64
    L.mqa_page_table_create.argtypes = [i32, i32, i32, p, i32, i32, i32, ctypes.POINTER(p)]
    L.mqa_page_table_create.restype = ctypes.c_int
    L.mqa_page_table_destroy.argtypes, L.mqa_page_table_destroy.restype = [p], ctypes.c_int
    L.mqa_page_table_advance.argtypes = [p, i32, i64, i32, p]
    L.mqa_page_table_advance.restype = ctypes.c_int
    L.mqa_page_table_advance_all.argtypes = [p, p, p, p]
    L.mqa_page_table_advance_all.restype = ctypes.c_int
    L.mqa_page_table_release.argtypes = [p, i32, p]
    L.mqa_page_table_release.restype = ctypes.c_int
    L.mqa_page_table_free_pages.argtypes, L.mqa_page_table_free_pages.restype = [p], i64
    L.mqa_page_table_held_pages.argtypes = [p, i32, i32]
    L.mqa_page_table_held_pages.restype = i64
    L.mqa_page_table_slot_mapping.argtypes = [p, i32, i32, i64, i32, p]
    L.mqa_page_table_slot_mapping.restype = ctypes.c_int
    L.mqa_prefix_cache_create.argtypes = [p, i64, i32, p, i32, i32, ctypes.POINTER(p)]
    L.mqa_prefix_cache_create.restype = ctypes.c_int
    L.mqa_prefix_cache_destroy.argtypes, L.mqa_prefix_cache_destroy.restype = [p], ctypes.c_int
    L.mqa_prefix_cache_capacity.argtypes, L.mqa_prefix_cache_capacity.restype = [p], i64
    L.mqa_prefix_cache_entries.argtypes, L.mqa_prefix_cache_entries.restype = [p], i64
    L.mqa_prefix_cache_stats.argtypes, L.mqa_prefix_cache_stats.restype = [p, p], ctypes.c_int
    L.mqa_prefix_cache_lookup.argtypes = [p, p, i64, ctypes.POINTER(i64)]
    L.mqa_prefix_cache_lookup.restype = ctypes.c_int
    L.mqa_prefix_cache_restore.argtypes = [p, p, i64, ctypes.POINTER(_Pool), p, i32, i32, i32, i32,
                                           p]
    L.mqa_prefix_cache_restore.restype = ctypes.c_int
    L.mqa_prefix_cache_insert.argtypes = [p, p, i64, ctypes.POINTER(_Pool), p, i32, i32, i32, i32,
                                          p, ctypes.POINTER(i64)]
    L.mqa_prefix_cache_insert.restype = ctypes.c_int
    L.mqa_prefix_cache_insert_host.argtypes = [p, p, i64, p, p, ctypes.POINTER(i64)]
    L.mqa_prefix_cache_insert_host.restype = ctypes.c_int
    L.mqa_prefix_cache_read_host.argtypes = [p, p, i64, p, p]
    L.mqa_prefix_cache_read_host.restype = ctypes.c_int
    L.mqa_gqa_page_bytes.argtypes, L.mqa_gqa_page_bytes.restype = [i32, i32], sz
    L.mqa_gqa_pack_bf16.argtypes = [p, p, i64, p, p, i64, i32, i32, p]
    L.mqa_gqa_pack_bf16.restype = ctypes.c_int
    L.mqa_hbm_read_probe.argtypes = [p, i64, p, i32, p]
    L.mqa_hbm_read_probe.restype = ctypes.c_int
    L.mqa_gqa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    L.mqa_gqa_decode_workspace_bytes.restype = sz
    L.mqa_gqa_decode_bf16.argtypes = [p, p, p, i64, i32, i32, p, i32, p, i32, i32, i32, i32, f32,
                                      p, sz, p]
    L.mqa_gqa_decode_bf16.restype = ctypes.c_int
    return L


lib = _load()
PREFIX_HOST_ONLY = 1


def _check(status: int) -> None:
    if status != MQA_OK:
        raise MQAError(status, lib.mqa_last_error().decode())


def page_bytes(head_dim: int) -> int:
    n = int(lib.mqa_page_bytes(head_dim))
    if n == 0:
        raise MQAError(MQA_ERR_UNSUPPORTED, f"head_dim {head_dim} unsupported")
    return n


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    return int(lib.mqa_kv_bytes_per_token(num_layers, num_kv_heads, head_dim, dtype_bytes))


def kv_footprint_bytes(layer_slot: Sequence[int], layer_window: Sequence[int], num_kv_heads: int,
                       head_dim: int, code_bytes: int, scale_bytes: int, context: int,
                       page_tokens: int = PAGE_TOKENS) -> int:
    """KV bytes one sequence holds at ``context`` tokens for a layer map
    (``mqa_kv_footprint_bytes``)."""
    n = len(layer_slot)
    ls = _host_i32(layer_slot, n, "layer_slot")
    lw = _host_i32(layer_window, n, "layer_window")
    r = int(lib.mqa_kv_footprint_bytes(n, ls.ctypes.data, lw.ctypes.data, num_kv_heads, head_dim,
                                       code_bytes, scale_bytes, int(context), page_tokens))
    if r < 0:
        raise MQAError(MQA_ERR_INVALID, "invalid footprint arguments")
    return r


class PageTable:
    """Page table with recycling of windowed slots (``mqa_page_table_*``).
    ``block_table`` is the host mirror ([num_slots, batch, max_pages] int32)
    the library writes; copy it to the device for the attention calls."""

    def __init__(self, first_page: int, num_pages: int, slot_window: Sequence[int], batch: int,
                 max_pages: int, invalid_page: int = -1):
        self.num_slots = len(slot_window)
        self.batch, self.max_pages = batch, max_pages
        sw = _host_i32(slot_window, self.num_slots, "slot_window")
        h = ctypes.c_void_p()
        _check(lib.mqa_page_table_create(first_page, num_pages, self.num_slots, sw.ctypes.data,
                                         batch, max_pages, invalid_page, ctypes.byref(h)))
        self._h = h
        self.block_table = np.full((self.num_slots, batch, max_pages), invalid_page, np.int32)

    def close(self) -> None:
        if self._h is not None and self._h.value:
            lib.mqa_page_table_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def advance(self, seq: int, context: int, new_tokens: int = 1) -> None:
        _check(lib.mqa_page_table_advance(self._h, seq, int(context), int(new_tokens),
                                          self.block_table.ctypes.data))

    def advance_all(self, context: Sequence[int], new_tokens: Sequence[int]) -> None:
        """One step of the whole batch (``new_tokens[b] = 0``: b does not step)."""
        c = np.ascontiguousarray(context, dtype=np.int64)
        n = np.ascontiguousarray(new_tokens, dtype=np.int32)
        if c.shape != (self.batch,) or n.shape != (self.batch,):
            raise ValueError(f"context and new_tokens must have {self.batch} entries")
        _check(lib.mqa_page_table_advance_all(self._h, c.ctypes.data, n.ctypes.data,
                                              self.block_table.ctypes.data))

    def release(self, seq: int) -> None:
        _check(lib.mqa_page_table_release(self._h, seq, self.block_table.ctypes.data))

    def free_pages(self) -> int:
        return int(lib.mqa_page_table_free_pages(self._h))

    def held_pages(self, seq: int, slot: int) -> int:
        return int(lib.mqa_page_table_held_pages(self._h, seq, slot))

    def slot_mapping(self, seq: int, slot: int, start: int, count: int) -> np.ndarray:
        out = np.empty(count, np.int64)
        _check(lib.mqa_page_table_slot_mapping(self._h, seq, slot, int(start), int(count),
                                               out.ctypes.data))
        return out


class PrefixCache:
    """Cross-turn prefix cache in pinned host memory (``mqa_prefix_cache_*``).

    ``arena_bytes`` of pinned host memory are allocated through torch (or, with
    ``host_only``, plain host memory: no GPU copies, for host-side use)."""

    def __init__(self, arena_bytes: int, slot_window: Sequence[int], head_dim: int,
                 host_only: bool = False):
        torch = _torch()
        self.num_slots = len(slot_window)
        self.head_dim = head_dim
        self.page_bytes = page_bytes(head_dim)
        # 256 bytes of slack so that the arena can start on a 256-byte boundary
        self.arena = torch.empty(int(arena_bytes) + 256, dtype=torch.uint8,
                                 pin_memory=not host_only)
        base = self.arena.data_ptr()
        self._off = (-base) % 256
        sw = _host_i32(slot_window, self.num_slots, "slot_window")
        h = ctypes.c_void_p()
        _check(lib.mqa_prefix_cache_create(base + self._off, int(arena_bytes), self.num_slots,
                                           sw.ctypes.data, head_dim,
                                           PREFIX_HOST_ONLY if host_only else 0, ctypes.byref(h)))
        self._h = h

    def close(self) -> None:
        if self._h is not None and self._h.value:
            lib.mqa_prefix_cache_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _tokens(tokens) -> np.ndarray:
        return np.ascontiguousarray(tokens, dtype=np.int32)

    def capacity(self) -> int:
        return int(lib.mqa_prefix_cache_capacity(self._h))

    def entries(self) -> int:
        return int(lib.mqa_prefix_cache_entries(self._h))

    def stats(self) -> dict:
        out = np.zeros(6, np.int64)
        _check(lib.mqa_prefix_cache_stats(self._h, out.ctypes.data))
        keys = ("lookups", "tokens_asked", "tokens_matched", "entries_inserted",
                "entries_evicted", "entries_restored")
        return dict(zip(keys, (int(x) for x in out)))

    def lookup(self, tokens) -> int:
        t = self._tokens(tokens)
        m = ctypes.c_int64()
        _check(lib.mqa_prefix_cache_lookup(self._h, t.ctypes.data, t.size, ctypes.byref(m)))
        return int(m.value)

    def restore(self, tokens, matched: int, pool: "KVPool", block_table_host: np.ndarray, seq: int,
                invalid_page: int = -1, stream=None) -> None:
        t = self._tokens(tokens)
        bt = np.ascontiguousarray(block_table_host, dtype=np.int32)
        _check(lib.mqa_prefix_cache_restore(self._h, t.ctypes.data, int(matched),
                                            ctypes.byref(pool.c), bt.ctypes.data, bt.shape[1], seq,
                                            bt.shape[2], invalid_page, _stream_ptr(stream)))

    def insert(self, tokens, pool: "KVPool", block_table_host: np.ndarray, seq: int,
               invalid_page: int = -1, stream=None) -> int:
        t = self._tokens(tokens)
        bt = np.ascontiguousarray(block_table_host, dtype=np.int32)
        n = ctypes.c_int64()
        _check(lib.mqa_prefix_cache_insert(self._h, t.ctypes.data, t.size, ctypes.byref(pool.c),
                                           bt.ctypes.data, bt.shape[1], seq, bt.shape[2],
                                           invalid_page, _stream_ptr(stream), ctypes.byref(n)))
        return int(n.value)

    def insert_host(self, tokens, pages: np.ndarray, present: np.ndarray) -> int:
        t = self._tokens(tokens)
        pg = np.ascontiguousarray(pages, dtype=np.uint8)
        pr = np.ascontiguousarray(present, dtype=np.uint64)
        n = ctypes.c_int64()
        _check(lib.mqa_prefix_cache_insert_host(self._h, t.ctypes.data, t.size, pg.ctypes.data,
                                                pr.ctypes.data, ctypes.byref(n)))
        return int(n.value)

    def read_host(self, tokens, pages: int):
        t = self._tokens(tokens)
        out = np.empty((pages, self.num_slots, self.page_bytes), np.uint8)
        present = np.empty(pages, np.uint64)
        _check(lib.mqa_prefix_cache_read_host(self._h, t.ctypes.data, pages, out.ctypes.data,
                                              present.ctypes.data))
        return out, present


# --------------------------------------------------------------------------
# grouped-query bf16 baseline (mqa_gqa_*)
# --------------------------------------------------------------------------
def gqa_page_bytes(num_kv_heads: int, head_dim: int) -> int:
    n = int(lib.mqa_gqa_page_bytes(num_kv_heads, head_dim))
    if n == 0:
        raise MQAError(MQA_ERR_UNSUPPORTED, f"({num_kv_heads}, {head_dim}) unsupported")
    return n


PROBE_SINK_WORDS = 4096


def hbm_read_probe(src, sink, stream=None) -> None:
    """Streaming read of the device tensor ``src`` (``mqa_hbm_read_probe``);
    ``sink`` uint32-sized (int32) [>= PROBE_SINK_WORDS] receives per-range
    XORs whose XOR is that of all 32-bit words of ``src``."""
    torch = _torch()
    if not src.is_contiguous() or not sink.is_contiguous():
        raise ValueError("src and sink must be contiguous")
    _check(lib.mqa_hbm_read_probe(_dev_ptr(src, "src"), src.numel() * src.element_size(),
                                  _dev_ptr(sink, "sink", torch.int32), int(sink.numel()),
                                  _stream_ptr(stream)))


def gqa_pack_bf16(k, v, slot_mapping, pool, num_kv_heads: int, stream=None) -> None:
    """``k, v`` bf16 [T, Hkv, D]; ``pool`` a uint8 tensor [num_pages, page_bytes]."""
    torch = _torch()
    t, h, d = (int(x) for x in k.shape)
    if h != num_kv_heads or tuple(v.shape) != (t, h, d):
        raise ValueError("k and v must be [T, num_kv_heads, D]")
    _check(lib.mqa_gqa_pack_bf16(_dev_ptr(k, "k", torch.bfloat16), _dev_ptr(v, "v", torch.bfloat16),
                                 t, _dev_ptr(slot_mapping, "slot_mapping", torch.int64),
                                 _dev_ptr(pool, "pool", torch.uint8), int(pool.shape[0]), h, d,
                                 _stream_ptr(stream)))


def gqa_decode_workspace(batch: int, num_q_heads: int, num_kv_heads: int, max_context: int,
                         window: int, head_dim: int):
    torch = _torch()
    n = int(lib.mqa_gqa_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, max_context,
                                                window, head_dim))
    return torch.empty(max(n, 256), dtype=torch.uint8, device="cuda") if n else None


def gqa_decode_bf16(q, out, pool, num_kv_heads: int, block_table, context_lens, max_context: int,
                    window: int, softmax_scale: float = 0.0, workspace=None, stream=None) -> None:
    """``q`` bf16 [B, Hq, D]; ``out`` fp32 [B, Hq, D]; ``block_table`` int32
    [B, max_pages]."""
    torch = _torch()
    b, hq, d = (int(x) for x in q.shape)
    if tuple(out.shape) != (b, hq, d):
        raise ValueError("out must have q's shape")
    ws_ptr = _dev_ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.mqa_gqa_decode_bf16(_dev_ptr(q, "q", torch.bfloat16),
                                   _dev_ptr(out, "out", torch.float32),
                                   _dev_ptr(pool, "pool", torch.uint8), int(pool.shape[0]),
                                   num_kv_heads, d, _dev_ptr(block_table, "block_table", torch.int32),
                                   int(block_table.shape[1]),
                                   _dev_ptr(context_lens, "context_lens", torch.int32),
                                   int(max_context), b, hq, int(window), float(softmax_scale),
                                   ws_ptr, ws_bytes, _stream_ptr(stream)))


_layout_cache = {}


def page_layout(head_dim: int):
    """Byte offsets inside a page record, from the library's own layout:
    ``(k_off [16, D], v_off [16, D], ks_off [16], vs_off [16])`` (int64)."""
    if head_dim in _layout_cache:
        return _layout_cache[head_dim]
    off = ctypes.c_int64()
    k = np.empty((PAGE_TOKENS, head_dim), np.int64)
    v = np.empty((PAGE_TOKENS, head_dim), np.int64)
    ks = np.empty(PAGE_TOKENS, np.int64)
    vs = np.empty(PAGE_TOKENS, np.int64)
    for j in range(PAGE_TOKENS):
        for c in range(head_dim):
            _check(lib.mqa_page_offset(head_dim, j, c, 0, ctypes.byref(off)))
            k[j, c] = off.value
            _check(lib.mqa_page_offset(head_dim, j, c, 1, ctypes.byref(off)))
            v[j, c] = off.value
        _check(lib.mqa_page_offset(head_dim, j, 0, 2, ctypes.byref(off)))
        ks[j] = off.value
        _check(lib.mqa_page_offset(head_dim, j, 0, 3, ctypes.byref(off)))
        vs[j] = off.value
    _layout_cache[head_dim] = (k, v, ks, vs)
    return _layout_cache[head_dim]


# --------------------------------------------------------------------------
# torch plumbing
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream_ptr(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev_ptr(t, name: str, dtype=None) -> int:
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _host_i32(x, n: int, name: str) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32).reshape(-1))
    if a.size != n:
        raise ValueError(f"{name} must have {n} entries")
    return a


class KVPool:
    """A paged int8 KV pool in device memory (a torch uint8 tensor).

    ``num_pages`` page records of ``page_bytes(head_dim)`` bytes.  Which
    slot/sequence/tokens a page holds is decided by the caller's block tables.
    """

    def __init__(self, num_pages: int, head_dim: int, device="cuda", fill: Optional[int] = 0):
        torch = _torch()
        self.head_dim = int(head_dim)
        self.num_pages = int(num_pages)
        self.page_bytes = page_bytes(head_dim)
        # torch's caching allocator returns 512-byte aligned blocks
        if fill is None:
            self.data = torch.empty((self.num_pages, self.page_bytes), dtype=torch.uint8,
                                    device=device)
        else:
            self.data = torch.full((self.num_pages, self.page_bytes), fill, dtype=torch.uint8,
                                   device=device)
        self._c = _Pool(self.data.data_ptr(), self.num_pages, self.head_dim, 0)

    @classmethod
    def wrap(cls, data, head_dim: int) -> "KVPool":
        """A pool over an existing uint8 tensor [num_pages, page_bytes]."""
        obj = cls.__new__(cls)
        obj.head_dim = int(head_dim)
        obj.page_bytes = page_bytes(head_dim)
        if data.dim() != 2 or data.shape[1] != obj.page_bytes:
            raise ValueError("pool tensor must be [num_pages, page_bytes]")
        obj.num_pages = int(data.shape[0])
        obj.data = data
        obj._c = _Pool(_dev_ptr(data, "pool"), obj.num_pages, obj.head_dim, 0)
        return obj

    @property
    def c(self) -> _Pool:
        return self._c


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return MQA_F32
    if t.dtype == torch.bfloat16:
        return MQA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


# --------------------------------------------------------------------------
# Entry points
# --------------------------------------------------------------------------
def kv_pack_int8(k, v, slot_mapping, pool: KVPool, stream=None) -> None:
    """Quantise K and V rows ``[T, head_dim]`` (fp32 or bf16, same dtype) and
    write them at ``slot_mapping`` (int64 [T], page*16 + offset; negative =
    skip)."""
    torch = _torch()
    if k.shape != v.shape or k.dtype != v.dtype:
        raise ValueError("k and v must have the same shape and dtype")
    if k.dim() != 2 or k.shape[1] != pool.head_dim:
        raise ValueError("k and v must be [T, head_dim]")
    t = int(k.shape[0])
    if slot_mapping.shape != (t,):
        raise ValueError("slot_mapping must be [T]")
    _check(lib.kv_pack_int8(_dev_ptr(k, "k"), _dev_ptr(v, "v"), _dtype_code(k), t,
                            pool.head_dim, _dev_ptr(slot_mapping, "slot_mapping", torch.int64),
                            ctypes.byref(pool.c), _stream_ptr(stream)))


def _q_dtype_code(q_dtype) -> int:
    """MQA_BF16 / MQA_F32 from "bf16" / "f32" (or "fp32") or a torch dtype."""
    t = _torch()
    if q_dtype in ("bf16", t.bfloat16):
        return MQA_BF16
    if q_dtype in ("f32", "fp32", t.float32):
        return MQA_F32
    raise ValueError(f"q dtype {q_dtype!r}: bf16 or f32")


def decode_workspace_bytes(batch: int, num_q_heads: int, layer_slot: Sequence[int],
                           layer_window: Sequence[int], max_context: int, head_dim: int,
                           q_dtype="bf16") -> int:
    """Workspace bytes (``mqa_decode_workspace_bytes``) of decode calls of these
    shapes with queries of ``q_dtype``."""
    n = len(layer_slot)
    ls = _host_i32(layer_slot, n, "layer_slot")
    lw = _host_i32(layer_window, n, "layer_window")
    return int(lib.mqa_decode_workspace_bytes(batch, num_q_heads, n, ls.ctypes.data,
                                              lw.ctypes.data, max_context, head_dim,
                                              _q_dtype_code(q_dtype)))


def decode_tuning(waves: int = 0, rows: int = 0, target_wgs: int = 0) -> None:
    """Process-wide decode tuning (``mqa_decode_tuning``); 0 = the planner
    decides.  Workspace sizes depend on it: query them after a change."""
    _check(lib.mqa_decode_tuning(int(waves), int(rows), int(target_wgs)))


def decode_workspace(batch: int, num_q_heads: int, layer_slot: Sequence[int],
                     layer_window: Sequence[int], max_context: int, head_dim: int,
                     device="cuda", q_dtype="bf16"):
    """A zero-filled workspace for these decode shapes (None when none is
    needed).  Zero-fill once; every call leaves it reusable."""
    n = decode_workspace_bytes(batch, num_q_heads, layer_slot, layer_window, max_context,
                               head_dim, q_dtype)
    return _torch().zeros(n, dtype=_torch().uint8, device=device) if n else None


def _decode_args(q, out, pool, block_table, context_lens, layer_slot, layer_window, workspace):
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [L, B, Hq, D]")
    n_layers, batch, hq, d = (int(x) for x in q.shape)
    if d != pool.head_dim:
        raise ValueError("q head_dim does not match the pool")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    if block_table.dim() != 3 or int(block_table.shape[1]) != batch:
        raise ValueError("block_table must be [num_slots, B, max_pages]")
    if tuple(context_lens.shape) != (batch,):
        raise ValueError("context_lens must be [B]")
    ls = _host_i32(layer_slot, n_layers, "layer_slot")
    lw = _host_i32(layer_window, n_layers, "layer_window")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size()
    return (n_layers, batch, hq, ls, lw, ws_ptr, ws_bytes,
            _dev_ptr(out, "out", torch.float32), _dev_ptr(block_table, "block_table", torch.int32),
            _dev_ptr(context_lens, "context_lens", torch.int32))


def mqa_decode_attn(q, out, pool: KVPool, block_table, context_lens, max_context: int,
                    layer_slot: Sequence[int], layer_window: Sequence[int],
                    softmax_scale: float = 0.0, workspace=None, stream=None) -> None:
    """One decode step.  ``q [L, B, Hq, D]`` (fp32/bf16), ``out`` fp32 of the
    same shape, ``block_table`` int32 [num_slots, B, max_pages],
    ``context_lens`` int32 [B] (device), ``layer_slot``/``layer_window`` host
    sequences of length L, ``workspace`` from :func:`decode_workspace`."""
    (n_layers, batch, hq, ls, lw, ws_ptr, ws_bytes, out_p, bt_p,
     cl_p) = _decode_args(q, out, pool, block_table, context_lens, layer_slot, layer_window,
                          workspace)
    _check(lib.mqa_decode_attn(
        _dev_ptr(q, "q"), _dtype_code(q), out_p, ctypes.byref(pool.c), bt_p,
        int(block_table.shape[2]), cl_p, int(max_context), batch, hq, n_layers,
        int(block_table.shape[0]), ls.ctypes.data, lw.ctypes.data, float(softmax_scale), ws_ptr,
        ws_bytes, _stream_ptr(stream)))


def mqa_decode_step(q, out, k_new, v_new, pool: KVPool, block_table, context_lens,
                    max_context: int, layer_slot: Sequence[int], layer_window: Sequence[int],
                    softmax_scale: float = 0.0, workspace=None, stream=None) -> None:
    """The current token's K/V (``k_new``, ``v_new`` [num_slots, B, D], fp32 or
    bf16) stored at position ``context_lens[b] - 1`` of each slot, fused with
    :func:`mqa_decode_attn` in one launch."""
    (n_layers, batch, hq, ls, lw, ws_ptr, ws_bytes, out_p, bt_p,
     cl_p) = _decode_args(q, out, pool, block_table, context_lens, layer_slot, layer_window,
                          workspace)
    num_slots = int(block_table.shape[0])
    want = (num_slots, batch, pool.head_dim)
    if tuple(k_new.shape) != want or tuple(v_new.shape) != want:
        raise ValueError(f"k_new and v_new must be {list(want)}")
    if k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must have the same dtype")
    _check(lib.mqa_decode_step(
        _dev_ptr(q, "q"), _dtype_code(q), out_p, _dev_ptr(k_new, "k_new"),
        _dev_ptr(v_new, "v_new"), _dtype_code(k_new), ctypes.byref(pool.c), bt_p,
        int(block_table.shape[2]), cl_p, int(max_context), batch, hq, n_layers, num_slots,
        ls.ctypes.data, lw.ctypes.data, float(softmax_scale), ws_ptr, ws_bytes,
        _stream_ptr(stream)))


DECODE_STATIC_SCRATCH_BYTES = 40 << 20


def mqa_decode_step_noalloc(q, out, k_new, v_new, pool: KVPool, block_table, context_lens,
                            max_context: int, layer_slot: Sequence[int],
                            layer_window: Sequence[int], softmax_scale: float = 0.0,
                            stream=None) -> None:
    """:func:`mqa_decode_step` with no workspace: its scratch is the library's
    static per-GPU array (calls that overlap on one GPU race)."""
    (n_layers, batch, hq, ls, lw, _, _, out_p, bt_p,
     cl_p) = _decode_args(q, out, pool, block_table, context_lens, layer_slot, layer_window, None)
    num_slots = int(block_table.shape[0])
    want = (num_slots, batch, pool.head_dim)
    if tuple(k_new.shape) != want or tuple(v_new.shape) != want:
        raise ValueError(f"k_new and v_new must be {list(want)}")
    if k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must have the same dtype")
    _check(lib.mqa_decode_step_noalloc(
        _dev_ptr(q, "q"), _dtype_code(q), out_p, _dev_ptr(k_new, "k_new"),
        _dev_ptr(v_new, "v_new"), _dtype_code(k_new), ctypes.byref(pool.c), bt_p,
        int(block_table.shape[2]), cl_p, int(max_context), batch, hq, n_layers, num_slots,
        ls.ctypes.data, lw.ctypes.data, float(softmax_scale), _stream_ptr(stream)))


def mqa_append_attn(q, out, pool: KVPool, block_table, context_lens, cu_q_lens, max_context: int,
                    max_q_len: int, layer_slot: Sequence[int], layer_window: Sequence[int],
                    softmax_scale: float = 0.0, stream=None) -> None:
    """Causal chunk attention.  ``q [L, total_q, Hq, D]``; ``cu_q_lens`` int32
    [B+1] (device); other arguments as for :func:`mqa_decode_attn`."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [L, total_q, Hq, D]")
    n_layers, total_q, hq, d = (int(x) for x in q.shape)
    if d != pool.head_dim:
        raise ValueError("q head_dim does not match the pool")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    batch = int(context_lens.shape[0])
    if block_table.dim() != 3 or int(block_table.shape[1]) != batch:
        raise ValueError("block_table must be [num_slots, B, max_pages]")
    if tuple(cu_q_lens.shape) != (batch + 1,):
        raise ValueError("cu_q_lens must be [B+1]")
    ls = _host_i32(layer_slot, n_layers, "layer_slot")
    lw = _host_i32(layer_window, n_layers, "layer_window")
    _check(lib.mqa_append_attn(
        _dev_ptr(q, "q"), _dtype_code(q), _dev_ptr(out, "out", torch.float32), ctypes.byref(pool.c),
        _dev_ptr(block_table, "block_table", torch.int32), int(block_table.shape[2]),
        _dev_ptr(context_lens, "context_lens", torch.int32),
        _dev_ptr(cu_q_lens, "cu_q_lens", torch.int32), int(max_context), int(max_q_len), total_q,
        batch, hq, n_layers, int(block_table.shape[0]), ls.ctypes.data, lw.ctypes.data,
        float(softmax_scale), _stream_ptr(stream)))


# --------------------------------------------------------------------------
# Host helpers (no device work)
# --------------------------------------------------------------------------
def slot_mapping_for(table_row: np.ndarray, start: int, stop: int) -> np.ndarray:
    """page*16 + offset of positions [start, stop) of one sequence, given its
    block-table row (logical page -> pool page)."""
    pos = np.arange(start, stop, dtype=np.int64)
    return np.asarray(table_row, dtype=np.int64)[pos // PAGE_TOKENS] * PAGE_TOKENS + pos % PAGE_TOKENS


def unpack_page_tokens(pool_bytes: np.ndarray, slots: np.ndarray, head_dim: int):
    """Read tokens back out of host copies of page records.

    ``pool_bytes`` uint8 [num_pages, page_bytes]; ``slots`` int64 [T]
    (page*16 + offset).  Returns ``(k_codes int8 [T, D], k_scales f32 [T],
    v_codes int8 [T, D], v_scales f32 [T])``.  A K or V code c is stored as
    the byte c + 128 (its sign bit flipped)."""
    k_off, v_off, ks_off, vs_off = page_layout(head_dim)
    slots = np.asarray(slots, dtype=np.int64)
    page, j = slots // PAGE_TOKENS, slots % PAGE_TOKENS
    rec = pool_bytes[page]                                   # [T, page_bytes]
    rows = np.arange(slots.size)[:, None]
    kc = (rec[rows, k_off[j]] ^ np.uint8(0x80)).view(np.int8)
    vc = (rec[rows, v_off[j]] ^ np.uint8(0x80)).view(np.int8)
    ks = np.stack([rec[np.arange(slots.size), ks_off[j] + b] for b in range(4)], 1).copy()
    vs = np.stack([rec[np.arange(slots.size), vs_off[j] + b] for b in range(4)], 1).copy()
    return kc, ks.view(np.float32).reshape(-1), vc, vs.view(np.float32).reshape(-1)
