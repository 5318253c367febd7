"""Helpers for the GPU parity tests: upload a synthetic workload through the
HIP path (kv_pack_int8 writes every page), build the oracle's logical view of
the same workload, and compare outputs.

Both sides start from the same seeded fp32 K/V rows and q values (``synth``);
the GPU quantises with its own kernel, the oracle with its own quantiser.
"""
import dataclasses
import math
import sys

import numpy as np
import torch

import int8_mqa_kv_amd as mk
import oracle
import synth

# Tolerances of the path (fp32 output vs the fp64 oracle)
MAX_ABS = 2e-3
REL_L2 = 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def q_tensor(w: synth.Workload, device="cuda"):
    """q on the GPU in the workload's dtype, and its exact fp64 values."""
    qf = w.q_f32()
    if w.q_dtype == "bf16":
        bits = synth.f32_to_bf16_bits(qf)
        t = torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
        return t, oracle.bf16_bits_to_f64(bits)
    return torch.from_numpy(qf).to(device), qf.astype(np.float64)


class GpuCase:
    """A workload resident on the GPU: pool, tables, lengths."""

    def __init__(self, w: synth.Workload, device="cuda", poison=True, chunk_tokens=1 << 20):
        self.w = w
        self.device = device
        self.pool = mk.KVPool(w.num_pages, w.head_dim, device=device)
        self.block_table = torch.from_numpy(np.ascontiguousarray(w.block_table)).to(device)
        self.context_lens = torch.from_numpy(w.context_lens.astype(np.int32)).to(device)
        self.cu_q_lens = torch.from_numpy(w.cu_q_lens.astype(np.int32)).to(device)
        self._pack_all(chunk_tokens)
        if poison:
            self.poison_page(w.poison_page)
        torch.cuda.synchronize()

    def _pack_all(self, chunk_tokens):
        w = self.w
        ks, vs, sm = [], [], []
        n = 0

        def flush():
            nonlocal ks, vs, sm, n
            if not ks:
                return
            k = torch.from_numpy(np.concatenate(ks)).to(self.device)
            v = torch.from_numpy(np.concatenate(vs)).to(self.device)
            s = torch.from_numpy(np.concatenate(sm)).to(self.device)
            mk.kv_pack_int8(k, v, s, self.pool)
            torch.cuda.synchronize()
            ks, vs, sm, n = [], [], [], 0

        for slot in range(w.num_slots):
            for b in range(w.batch):
                first, ctx = w.stored_range(slot, b)
                if ctx <= first:
                    continue
                k, v = w.kv_rows(slot, b, first, ctx)
                ks.append(k)
                vs.append(v)
                sm.append(mk.slot_mapping_for(w.block_table[slot, b], first, ctx))
                n += ctx - first
                if n >= chunk_tokens:
                    flush()
        flush()

    def poison_page(self, page):
        """Random codes and NaN scales: any read of this page that is not
        masked would turn the output into NaN."""
        w = self.w
        k, v = w.poison_kv()
        sm = torch.arange(page * 16, page * 16 + 16, dtype=torch.int64, device=self.device)
        mk.kv_pack_int8(torch.from_numpy(k).to(self.device), torch.from_numpy(v).to(self.device),
                        sm, self.pool)
        _, _, ks_off, vs_off = mk.page_layout(w.head_dim)
        nan = np.frombuffer(np.float32(np.nan).tobytes(), np.uint8)
        row = self.pool.data[page].cpu().numpy()
        for j in range(16):
            row[ks_off[j]:ks_off[j] + 4] = nan
            row[vs_off[j]:vs_off[j] + 4] = nan
        self.pool.data[page] = torch.from_numpy(row).to(self.device)

    # ------------------------------------------------------------------ runs
    def decode(self, q, layer_slot=None, layer_window=None, scale=0.0, out=None):
        w = self.w
        ls = w.layer_slot if layer_slot is None else layer_slot
        lw = w.layer_window if layer_window is None else layer_window
        if out is None:
            out = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=self.device)
        wsb = mk.decode_workspace_bytes(w.batch, w.num_q_heads, ls, lw, w.max_context, w.head_dim,
                                        w.q_dtype)
        # The workspace is zeroed once and reused by every later call of this
        # case (each call must leave its arrival counters at zero).
        ws = None
        if wsb:
            if not hasattr(self, "_ws") or self._ws.numel() < wsb:
                self._ws = torch.zeros(wsb, dtype=torch.uint8, device=self.device)
            ws = self._ws
        mk.mqa_decode_attn(q, out, self.pool, self.block_table, self.context_lens, w.max_context,
                           ls, lw, softmax_scale=scale, workspace=ws)
        torch.cuda.synchronize()
        return out

    def append(self, q, layer_slot=None, layer_window=None, scale=0.0):
        w = self.w
        ls = w.layer_slot if layer_slot is None else layer_slot
        lw = w.layer_window if layer_window is None else layer_window
        out = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=self.device)
        mk.mqa_append_attn(q, out, self.pool, self.block_table, self.context_lens, self.cu_q_lens,
                           w.max_context, w.max_q_len, ls, lw, softmax_scale=scale)
        torch.cuda.synchronize()
        return out


class OracleKV:
    """The oracle's logical view: per (slot, seq) int8 codes and scales of the
    stored positions, quantised by the oracle from the same fp32 rows."""

    def __init__(self, w: synth.Workload):
        self.w = w
        self.cache = {}

    def __call__(self, slot, seq):
        key = (slot, seq)
        if key not in self.cache:
            first, ctx = self.w.stored_range(slot, seq)
            k, v = self.w.kv_rows(slot, seq, first, ctx)
            kc, ksc = oracle.quantize(k)
            vc, vsc = oracle.quantize(v)
            self.cache[key] = (first, kc, ksc, vc, vsc)
        return self.cache[key]


def compare(got, want, what=""):
    """Max-abs and relative-L2 error of fp32 GPU output against fp64 oracle
    values (NaN entries of ``want`` are rows not checked)."""
    got = got.detach().cpu().numpy().astype(np.float64) if hasattr(got, "detach") else got
    mask = ~np.isnan(want)
    g, r = got[mask], want[mask]
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    diff = g - r
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(r), 1e-300)) if diff.size else 0.0
    return max_abs, rel


def assert_parity(got, want, what=""):
    max_abs, rel = compare(got, want, what)
    log(f"  parity {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= MAX_ABS, f"{what}: max abs error {max_abs:.3e} > {MAX_ABS}"
    assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e} > {REL_L2}"
    return max_abs, rel


def outlier_q(q, q64, gain, seed):
    """q with four seeded channels scaled by a power of two (exact in bf16),
    the same channels in every row, as activation outliers sit in fixed
    channels."""
    ch = np.sort(np.random.default_rng(seed).choice(q.shape[-1], 4, replace=False))
    q, q64 = q.clone(), q64.copy()
    q[..., torch.from_numpy(ch).to(q.device)] *= gain
    q64[..., ch] *= gain
    return q, q64


class _VGain(synth.Workload):
    """The workload with every V row multiplied by a power of two set by its
    position: zero rows for positions below 40, 2^-80 up to position 300, then
    2^-40 growing by one power of two every 128 positions up to 1.  A
    wavefront's largest V scale so far thus starts absent, then sits far below
    fp32's usual range, then grows again and again."""

    def kv_rows(self, slot, seq, start, stop):
        k, v = super().kv_rows(slot, seq, start, stop)
        pos = np.arange(start, stop, dtype=np.int64)
        e = np.where(pos < 300, -80, np.minimum(0, -40 + (pos - 300) // 128))
        g = np.ldexp(np.float32(1), e.astype(np.int32)).astype(np.float32)
        g[pos < 40] = 0
        return k, v * g[:, None]


def with_v_gain(w: synth.Workload) -> synth.Workload:
    return _VGain(**{f.name: getattr(w, f.name) for f in dataclasses.fields(w)})
