"""The oracle: a plain CPU statement of the int8 MQA KV attention path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product library
(``int8_mqa_kv_amd``) never imports it, and this package imports nothing from
the product: the two share no code, header, table or constant.

What it computes (the pages, cited by title and section):

* "Como funciona a inferência de IA, explicando claramente", section
  "Por que o cache KV existe": each new token's query is compared with the key
  of every earlier token and the values are summed with those weights; keys and
  values are computed once per token and kept for every later step.
* "Character.AI: inference optimization", section 03, technique table:
  multi-query attention (one shared K/V head per layer), local layers with a
  horizon of 1024 interleaved with global ones, KV shared across layers;
  section 05: int8 on the attention KV cache.
* "Como funciona a inferência de IA", section "Qual é o tamanho real do cache
  KV?": bytes per token = 2 x layers x kv_heads x head_dim x dtype bytes.

Readings where the pages are silent: the
softmax scale is 1/sqrt(head_dim); the quantiser is symmetric per token with an
fp32 scale max|x|/127, codes rint(x/s) rounded half to even and clamped to
+-127; a window W covers the query's own position and the W-1 before it; the
context length counts the current token, whose K/V are already cached.

Arithmetic: attention in fp64 (C, ``oracle.c``); the quantiser in fp32 because
its output bits are part of the specification.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Callable, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.oracle_quantize_rows.argtypes = [i64, i32, p, p, p]
    lib.oracle_quantize_rows.restype = None
    lib.oracle_dequantize_rows.argtypes = [i64, i32, p, p, p]
    lib.oracle_dequantize_rows.restype = None
    lib.oracle_attend.argtypes = [i64, i32, p, p, p, i64, i64, p, p, p, p,
                                  ctypes.c_double, p]
    lib.oracle_attend.restype = i64
    lib.oracle_kv_bytes_per_token.argtypes = [i64, i64, i64, i64]
    lib.oracle_kv_bytes_per_token.restype = i64
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def num_threads() -> int:
    """OpenMP threads the oracle's attention uses (OMP_NUM_THREADS or all)."""
    return int(_load().oracle_num_threads())


# --------------------------------------------------------------------------
# Quantiser (fp32 specification) and dequantiser (exact fp64)
# --------------------------------------------------------------------------
def quantize(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric per-token int8 code of fp32 rows ``x[T, d]``.

    Returns ``codes int8 [T, d]`` and ``scales float32 [T]``, where
    ``scale = max|x| / 127`` and ``code = clamp(rint(x / scale), -127, 127)``
    (fp32 IEEE division, ties to even; an all-zero row gives scale 0 and
    zero codes).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("quantize expects [T, d]")
    t, d = x.shape
    codes = np.empty((t, d), dtype=np.int8)
    scales = np.empty((t,), dtype=np.float32)
    if t:
        _load().oracle_quantize_rows(t, d, _ptr(x), _ptr(codes), _ptr(scales))
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact fp64 ``scale * code`` for ``codes [T, d]`` and ``scales [T]``."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    t, d = codes.shape
    out = np.empty((t, d), dtype=np.float64)
    if t:
        _load().oracle_dequantize_rows(t, d, _ptr(codes), _ptr(scales), _ptr(out))
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 numbers given as their uint16 bit patterns."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int,
                       dtype_bytes: int) -> int:
    """Per-token KV bytes: 2 x layers x kv_heads x head_dim x dtype bytes."""
    return int(_load().oracle_kv_bytes_per_token(num_layers, num_kv_heads,
                                                 head_dim, dtype_bytes))


def default_scale(head_dim: int) -> float:
    """Softmax scale 1/sqrt(head_dim), in fp64."""
    return 1.0 / math.sqrt(head_dim)


# --------------------------------------------------------------------------
# Attention over one dequantised history
# --------------------------------------------------------------------------
def attend(q: np.ndarray, pos: np.ndarray, window: np.ndarray, key_start: int,
           k_codes: np.ndarray, k_scales: np.ndarray,
           v_codes: np.ndarray, v_scales: np.ndarray,
           softmax_scale: float) -> np.ndarray:
    """Attention of query rows over one single-head int8 KV history.

    ``q [R, d]`` (any float dtype, upcast exactly to fp64); ``pos [R]`` the
    absolute position of each query; ``window [R]`` (0 = global).  Keys and
    values are stored for absolute positions ``key_start ..
    key_start + n_keys - 1``.  Row r attends ``[max(0, pos-W+1), pos]``
    (``[0, pos]`` when W = 0).  Returns fp64 ``[R, d]``.
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    r, d = q.shape
    pos = np.ascontiguousarray(pos, dtype=np.int64).reshape(r)
    window = np.ascontiguousarray(window, dtype=np.int32).reshape(r)
    kc = np.ascontiguousarray(k_codes, dtype=np.int8)
    ks = np.ascontiguousarray(k_scales, dtype=np.float32)
    vc = np.ascontiguousarray(v_codes, dtype=np.int8)
    vs = np.ascontiguousarray(v_scales, dtype=np.float32)
    n_keys = kc.shape[0]
    if kc.shape != (n_keys, d) or vc.shape != (n_keys, d) or \
            ks.shape != (n_keys,) or vs.shape != (n_keys,):
        raise ValueError("KV history shapes do not match")
    out = np.empty((r, d), dtype=np.float64)
    if r == 0:
        return out
    bad = _load().oracle_attend(r, d, _ptr(q), _ptr(pos), _ptr(window),
                                int(key_start), n_keys, _ptr(kc), _ptr(ks),
                                _ptr(vc), _ptr(vs), float(softmax_scale),
                                _ptr(out))
    if bad:
        raise ValueError(f"{bad} query rows attend positions outside the "
                         "stored history")
    return out


# A KV source maps (slot, seq) to the logical history of that slot for that
# sequence: (key_start, k_codes [n, d], k_scales [n], v_codes [n, d],
# v_scales [n]).
KVSource = Callable[[int, int], Tuple[int, np.ndarray, np.ndarray,
                                      np.ndarray, np.ndarray]]


def decode(q: np.ndarray, context_lens: Sequence[int],
           layer_slot: Sequence[int], layer_window: Sequence[int],
           kv: KVSource, softmax_scale: Optional[float] = None,
           seqs: Optional[Sequence[int]] = None) -> np.ndarray:
    """One decode step: every layer, every sequence, every query head.

    ``q [L, B, Hq, d]`` (fp64-exact values).  Sequence b's query sits at
    position ``context_lens[b] - 1`` (its own K/V are already cached); layer
    l reads KV slot ``layer_slot[l]`` with window ``layer_window[l]``.
    Returns fp64 ``[L, B, Hq, d]`` (or ``[L, len(seqs), Hq, d]``).
    """
    q = np.asarray(q)
    n_layers, batch, hq, d = q.shape
    scale = default_scale(d) if softmax_scale is None else softmax_scale
    seqs = list(range(batch)) if seqs is None else list(seqs)
    out = np.empty((n_layers, len(seqs), hq, d), dtype=np.float64)
    for li in range(n_layers):
        for si, b in enumerate(seqs):
            ks_, kc, ksc, vc, vsc = kv(int(layer_slot[li]), b)
            p = int(context_lens[b]) - 1
            out[li, si] = attend(q[li, b], np.full(hq, p),
                                 np.full(hq, int(layer_window[li])), ks_,
                                 kc, ksc, vc, vsc, scale)
    return out


def append(q: np.ndarray, context_lens: Sequence[int],
           cu_q_lens: Sequence[int], layer_slot: Sequence[int],
           layer_window: Sequence[int], kv: KVSource,
           softmax_scale: Optional[float] = None,
           seqs: Optional[Sequence[int]] = None) -> np.ndarray:
    """A causal multi-token turn on top of a cached prefix.

    ``q [L, sum(q_len), Hq, d]``; sequence b owns query tokens
    ``cu_q_lens[b] .. cu_q_lens[b+1]-1`` and has ``context_lens[b]`` keys in
    the cache, the chunk included, so its token t sits at position
    ``context_lens[b] - q_len_b + t`` and attends every cached position up to
    and including its own (further limited by the layer's window).
    Returns fp64 of q's shape (rows of sequences not in ``seqs`` are NaN).
    """
    q = np.asarray(q)
    n_layers, total, hq, d = q.shape
    scale = default_scale(d) if softmax_scale is None else softmax_scale
    batch = len(context_lens)
    seqs = list(range(batch)) if seqs is None else list(seqs)
    out = np.full((n_layers, total, hq, d), np.nan, dtype=np.float64)
    for li in range(n_layers):
        for b in seqs:
            t0, t1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
            qlen = t1 - t0
            if qlen == 0:
                continue
            ks_, kc, ksc, vc, vsc = kv(int(layer_slot[li]), b)
            first = int(context_lens[b]) - qlen
            rows = q[li, t0:t1].reshape(qlen * hq, d)
            pos = np.repeat(np.arange(first, first + qlen), hq)
            win = np.full(qlen * hq, int(layer_window[li]))
            out[li, t0:t1] = attend(rows, pos, win, ks_, kc, ksc, vc, vsc,
                                    scale).reshape(qlen, hq, d)
    return out


# --------------------------------------------------------------------------
# Grouped-query attention over a float (bf16) history: the baseline that
# "Character.AI: inference optimization", section 03 (technique table),
# compares multi-query attention with.  Written out in fp64 numpy from the
# same definition as ``attend``: scores of the query against every key in its
# range, softmax, weighted sum of the values.
# --------------------------------------------------------------------------
def attend_float(q: np.ndarray, pos: np.ndarray, window: np.ndarray, key_start: int,
                 k: np.ndarray, v: np.ndarray, softmax_scale: float) -> np.ndarray:
    """Attention of query rows ``q [R, d]`` over one float history ``k, v
    [n, d]`` stored for positions ``key_start .. key_start + n - 1``; row r
    attends ``[max(0, pos-W+1), pos]`` (``[0, pos]`` when W = 0).  fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    r = q.shape[0]
    out = np.empty_like(q)
    for i in range(r):
        p, w = int(pos[i]), int(window[i])
        lo = max(0, p - w + 1) if w > 0 else 0
        if lo < key_start or p - key_start >= k.shape[0]:
            raise ValueError("query attends positions outside the stored history")
        ks = k[lo - key_start:p - key_start + 1]
        vs = v[lo - key_start:p - key_start + 1]
        s = (ks @ q[i]) * softmax_scale
        e = np.exp(s - s.max())
        out[i] = (e @ vs) / e.sum()
    return out


def decode_gqa(q: np.ndarray, context_lens: Sequence[int], window: int, num_kv_heads: int,
               kv: Callable[[int, int], Tuple[int, np.ndarray, np.ndarray]],
               softmax_scale: Optional[float] = None) -> np.ndarray:
    """One decode step of one grouped-query layer: ``q [B, Hq, d]``; query
    head j reads KV head j // (Hq / num_kv_heads); ``kv(seq, head)`` gives
    (key_start, k [n, d], v [n, d]).  Sequence b's query sits at position
    context_lens[b] - 1.  Returns fp64 ``[B, Hq, d]`` (zeros for an empty
    context)."""
    q = np.asarray(q)
    batch, hq, d = q.shape
    group = hq // num_kv_heads
    scale = default_scale(d) if softmax_scale is None else softmax_scale
    out = np.zeros((batch, hq, d), dtype=np.float64)
    for b in range(batch):
        p = int(context_lens[b]) - 1
        if p < 0:
            continue
        for h in range(num_kv_heads):
            ks_, k, v = kv(b, h)
            rows = q[b, h * group:(h + 1) * group]
            out[b, h * group:(h + 1) * group] = attend_float(
                rows, np.full(group, p), np.full(group, window), ks_, k, v, scale)
    return out
