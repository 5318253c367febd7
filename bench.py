#!/usr/bin/env python3
"""Throughput of the int8 MQA KV attention path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--case 1|2|3|4] [--extra-cases 1,2,4] [--gpus 1]

One step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM:
  decode cases (1-3): mqa_decode_step -- the current token of every sequence
                      coded to int8 and stored, and decode attention over
                      every layer of the case, in one launch;
  append case (4):    kv_pack_int8 of the appended chunk into every slot, then
                      mqa_append_attn over all 12 layers.
The headline line is case 3 (three global layers reading one shared slot,
32 sequences at 16k context: the largest decode workload); the other cases
are timed in the same run and reported under "workloads", each with its own
roofline, counter traffic and CPU baseline.  Inputs are rotated over replicas
(pool, q, out, new rows) whose attended bytes together exceed 1 GB, so the
256 MB Infinity Cache and the L2s cannot serve a step from the previous one.
By default the steps are replayed from HIP graphs (one step per replica per
graph), as a serving loop replays its captured decode step; HIP events on
the replay stream time the region.  Before each timed region its graph is
replayed untimed for --settle-ms (default 300 ms): the GPU runs its first
fraction of a second of sustained load slower (case 3 measured 65 -> 58 ->
55 us per step over successive timed regions without it), and a serving
loop runs in the settled state.  The roofline's launch duration is that of
the dominant kernel: the decode step's single kernel (so the step time), or
for the append case the attention call timed alone from a graph of only
those calls.  --no-graph launches every call from the host instead (then the
host's launch rate, not the GPU, limits the small cases).

A streaming-read probe (mqa_hbm_read_probe) reports the HBM bandwidth a plain
read reaches on this GPU, beside the published 8 TB/s.

Prints one JSON line.  ``value`` is int8 KV GB/s of the whole step: the KV
bytes the step must stream (codes + fp32 scales of every attended key of every
slot, each once) divided by the step time.
"""
import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak, published
METRIC = "int8 KV GB/s (% of HBM peak) and decode tokens/s, MQA attention, 1 GPU"
KERNEL_SOURCES = ["int8_mqa_kv_amd/csrc/attn.hip", "int8_mqa_kv_amd/csrc/device.hpp",
                  "int8_mqa_kv_amd/csrc/pack.hip",
                  "int8_mqa_kv_amd/csrc/internal.hpp", "int8_mqa_kv_amd/csrc/layout.hpp",
                  "int8_mqa_kv_amd/csrc/api.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------
# Workload set-up on the GPU (all through the HIP path)
# --------------------------------------------------------------------------
class Replica:
    pass


def setup(w, replicas, torch, mk, synth):
    dev = "cuda"
    pool0 = mk.KVPool(w.num_pages, w.head_dim, device=dev)
    bt = torch.from_numpy(np.ascontiguousarray(w.block_table)).to(dev)
    ctx = torch.from_numpy(w.context_lens.astype(np.int32)).to(dev)
    cu = torch.from_numpy(w.cu_q_lens.astype(np.int32)).to(dev)
    # history of every slot, packed through kv_pack_int8
    ks, vs, sm, n = [], [], [], 0

    def flush():
        nonlocal ks, vs, sm, n
        if ks:
            mk.kv_pack_int8(torch.from_numpy(np.concatenate(ks)).to(dev),
                            torch.from_numpy(np.concatenate(vs)).to(dev),
                            torch.from_numpy(np.concatenate(sm)).to(dev), pool0)
            torch.cuda.synchronize()
        ks, vs, sm, n = [], [], [], 0

    for s in range(w.num_slots):
        for b in range(w.batch):
            first, c = w.stored_range(s, b)
            k, v = w.kv_rows(s, b, first, c)
            ks.append(k)
            vs.append(v)
            sm.append(mk.slot_mapping_for(w.block_table[s, b], first, c))
            n += c - first
            if n >= (1 << 20):
                flush()
    flush()
    # the rows the step stores: the current token of every (slot, sequence),
    # [num_slots, B, D] (decode), or the chunk, [tokens, D] + slot mapping (append)
    nk, nv, nsm = [], [], []
    for s in range(w.num_slots):
        for b in range(w.batch):
            c = int(w.context_lens[b])
            first = c - int(w.q_lens[b])
            k, v = w.kv_rows(s, b, first, c)
            nk.append(k)
            nv.append(v)
            nsm.append(mk.slot_mapping_for(w.block_table[s, b], first, c))
    new_k = torch.from_numpy(np.concatenate(nk)).to(dev)
    new_v = torch.from_numpy(np.concatenate(nv)).to(dev)
    new_sm = torch.from_numpy(np.concatenate(nsm)).to(dev)
    if w.kind == "decode":
        new_k = new_k.view(w.num_slots, w.batch, w.head_dim)
        new_v = new_v.view(w.num_slots, w.batch, w.head_dim)
    qf = w.q_f32()
    if w.q_dtype == "bf16":
        q0 = torch.from_numpy(synth.f32_to_bf16_bits(qf).view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        q0 = torch.from_numpy(qf).to(dev)
    reps = []
    for r in range(replicas):
        R = Replica()
        if r == 0:
            R.pool = pool0
        else:
            data = torch.empty_like(pool0.data)
            data.copy_(pool0.data)
            R.pool = mk.KVPool.wrap(data, w.head_dim)
        R.q = q0 if r == 0 else q0.clone()
        R.out = torch.empty(tuple(q0.shape), dtype=torch.float32, device=dev)
        R.k = new_k if r == 0 else new_k.clone()
        R.v = new_v if r == 0 else new_v.clone()
        reps.append(R)
    ws = None
    if w.kind == "decode":
        wsb = mk.decode_workspace_bytes(w.batch, w.num_q_heads, w.layer_slot, w.layer_window,
                                        w.max_context, w.head_dim, w.q_dtype)
        ws = torch.zeros(max(wsb, 256), dtype=torch.uint8, device=dev) if wsb else None
    torch.cuda.synchronize()
    return dict(bt=bt, ctx=ctx, cu=cu, sm=new_sm, reps=reps, ws=ws)


def attn_call(w, st, R, mk):
    if w.kind == "decode":
        mk.mqa_decode_attn(R.q, R.out, R.pool, st["bt"], st["ctx"], w.max_context, w.layer_slot,
                           w.layer_window, workspace=st["ws"])
    else:
        mk.mqa_append_attn(R.q, R.out, R.pool, st["bt"], st["ctx"], st["cu"], w.max_context,
                           w.max_q_len, w.layer_slot, w.layer_window)


def step(w, st, R, mk, ev=None):
    """One step; ``ev`` brackets the dominant kernel's launch."""
    if w.kind == "decode":
        if ev is not None:
            ev[0].record()
        mk.mqa_decode_step(R.q, R.out, R.k, R.v, R.pool, st["bt"], st["ctx"], w.max_context,
                           w.layer_slot, w.layer_window, workspace=st["ws"])
        if ev is not None:
            ev[1].record()
        return
    mk.kv_pack_int8(R.k, R.v, st["sm"], R.pool)
    if ev is not None:
        ev[0].record()
    attn_call(w, st, R, mk)
    if ev is not None:
        ev[1].record()


def attention_flops(w) -> float:
    """2*2*d flops per (query row, attended key): q.k and p*v."""
    total = 0.0
    for li in range(w.num_layers):
        win = int(w.layer_window[li])
        for b in range(w.batch):
            c = int(w.context_lens[b])
            ql = int(w.q_lens[b])
            for t in range(ql):
                p = c - ql + t
                lo = max(0, p - win + 1) if win > 0 else 0
                total += (p + 1 - lo)
    return total * w.num_q_heads * 4 * w.head_dim


# --------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same step
# --------------------------------------------------------------------------
def cpu_baseline(w, kv_bytes_step, budget_s):
    import oracle
    qf = w.q_f32().astype(np.float64)
    d = w.head_dim
    # logical histories the oracle reads (set-up, untimed)
    hist = {}
    for s in range(w.num_slots):
        for b in range(w.batch):
            first, c = w.stored_range(s, b)
            k, v = w.kv_rows(s, b, first, c)
            hist[(s, b)] = (first, *oracle.quantize(k), *oracle.quantize(v))
    new = [w.kv_rows(s, b, int(w.context_lens[b]) - int(w.q_lens[b]), int(w.context_lens[b]))
           for s in range(w.num_slots) for b in range(w.batch)]
    kv = lambda s, b: hist[(s, b)]
    # sample: whole steps for the decode cases; for the append case a few
    # sequences of one step (the unit is scaled by their share of the bytes)
    seqs = list(range(w.batch))
    frac = 1.0
    if w.kind == "append":
        seqs = list(range(0, w.batch, max(1, w.batch // 8)))[:8]
        per = [sum(int(w.context_lens[b]) for _ in range(w.num_layers)) for b in range(w.batch)]
        frac = sum(per[b] for b in seqs) / sum(per)
    n, t0 = 0, time.perf_counter()
    while True:
        for k, v in new:
            oracle.quantize(k)
            oracle.quantize(v)
        if w.kind == "decode":
            oracle.decode(qf, w.context_lens, w.layer_slot, w.layer_window, kv, seqs=seqs)
        else:
            oracle.append(qf, w.context_lens, w.cu_q_lens, w.layer_slot, w.layer_window, kv,
                          seqs=seqs)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or (n >= 1 and el * (n + 1) / n > 3 * budget_s):
            break
    per_step = el / n / frac
    sample = (f"{n} oracle step(s) of the same case" if w.kind == "decode" else
              f"{n} pass(es) over {len(seqs)} of {w.batch} sequences, scaled to the whole step")
    return {"value": kv_bytes_step / per_step / 1e9, "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle", "sample": sample,
            "seconds": round(el, 3), "s_per_step": per_step, "cpu": cpu_model()}


def cpu_model() -> str:
    """The host CPU's model name (as lscpu prints it), from /proc/cpuinfo."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def time_eager(w, st, R, reps, mk, torch, args):
    """Host-launched steps; events around every dominant kernel."""
    for i in range(args.warmup):
        step(w, st, R[i % reps], mk)
    torch.cuda.synchronize()
    E = torch.cuda.Event
    evs = [(E(enable_timing=True), E(enable_timing=True)) for _ in range(args.steps)]
    t0, t1 = E(enable_timing=True), E(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(w, st, R[i % reps], mk, evs[i])
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / args.steps, float(np.mean([a.elapsed_time(b) for a, b in evs]))


def time_graphs(w, st, R, reps, mk, torch, args):
    """Steps replayed from HIP graphs (one graph holds one step per replica),
    as a serving loop replays its captured decode step.  The timed region is
    exactly ``steps`` steps: full-graph replays plus one graph for the
    remainder.  The attention calls alone (mqa_decode_attn without the
    current token's store, or mqa_append_attn) are timed the same way from a
    graph holding only them."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # warm up (and plan) outside capture
        for i in range(max(args.warmup, 1)):
            step(w, st, R[i % reps], mk)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        return g

    full_n = min(reps, args.steps)
    g_full = capture(lambda i: step(w, st, R[i], mk), full_n)
    rem = args.steps % full_n
    g_rem = capture(lambda i: step(w, st, R[i], mk), rem) if rem else None
    a_full = capture(lambda i: attn_call(w, st, R[i], mk), full_n)
    a_rem = capture(lambda i: attn_call(w, st, R[i], mk), rem) if rem else None
    for g in (g_full, a_full):          # first replays are not timed
        g.replay()
    torch.cuda.synchronize()

    def settle(g):
        """Untimed replays for args.settle_ms of wall time (at least one),
        synchronising every few so the queue stays short."""
        end = time.perf_counter() + args.settle_ms * 1e-3
        n = 0
        while n == 0 or time.perf_counter() < end:
            g.replay()
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()

    def timed(gf, gr):
        E = torch.cuda.Event
        t0, t1 = E(enable_timing=True), E(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(args.steps // full_n):
            gf.replay()
        if gr is not None:
            gr.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps

    settle(g_full)
    t_step = timed(g_full, g_rem)
    settle(a_full)
    return t_step, timed(a_full, a_rem)


# --------------------------------------------------------------------------
def measure_case(case, args, torch, mk, synth, headline):
    """Set up, time and report one workload; frees its GPU memory after."""
    t_setup = time.perf_counter()
    w = synth.case(case)
    kv_bytes = w.attended_keys() * (2 * w.head_dim + 8)
    reps = args.replicas or max(1, math.ceil(1.0e9 / kv_bytes))
    if w.kind == "append":
        reps = args.replicas or 1   # footprint is several GB already
    log(f"case {w.case}: {w.name}; KV bytes/step {kv_bytes}; replicas {reps}")
    st = setup(w, reps, torch, mk, synth)
    R = st["reps"]
    log(f"  set-up {time.perf_counter() - t_setup:.1f} s")
    steps = args.steps if headline else args.extra_steps
    a = argparse.Namespace(**vars(args))
    a.steps = steps

    if args.no_graph:
        ms_step, attn_ms = time_eager(w, st, R, reps, mk, torch, a)
    else:
        ms_step, attn_ms = time_graphs(w, st, R, reps, mk, torch, a)
    log(f"  step {ms_step * 1e3:.2f} us, attention call {attn_ms * 1e3:.2f} us")
    # the dominant kernel: the decode step is one kernel, so its launch time
    # is the step time; for append it is the attention call
    # (host launches: the events around each step's kernel)
    dom_ms = ms_step if (w.kind == "decode" and not args.no_graph) else attn_ms

    tokens = int(w.q_lens.sum()) * w.num_layers
    value = kv_bytes / (ms_step * 1e-3) / 1e9
    res = {
        "steps": steps, "ms_per_step": round(ms_step, 6),
        "config": {"workload": f"case {w.case}: {w.name}", "batch": w.batch,
                   "num_q_heads": w.num_q_heads, "kv_heads": 1, "head_dim": w.head_dim,
                   "layers": w.num_layers, "layer_window": w.layer_window.tolist(),
                   "max_context": w.max_context, "q_dtype": w.q_dtype,
                   "parallelism": "none (1 GPU)", "replicas": reps},
        "value": round(value, 2), "unit": "GB/s",
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s" if w.kind == "decode" else "appended_tokens_per_s":
            round(tokens / (ms_step * 1e-3), 1),
        "kv_bytes_per_step": kv_bytes,
    }
    if w.kind == "decode":
        achieved = kv_bytes / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        fl = attention_flops(w)
        achieved = fl / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4)}
    roof["kernel"] = ("decode_kernel (mqa_decode_step: store + attention, one launch)"
                      if w.kind == "decode" else "append_kernel (mqa_append_attn)")
    roof["avg_launch_us"] = round(dom_ms * 1e3, 3)
    if w.kind == "decode" and not args.no_graph:
        roof["attention_only_us"] = round(attn_ms * 1e3, 3)
    roof["timing"] = ("host launches, events around each call" if args.no_graph else
                      f"HIP graph replay of back-to-back calls after {args.settle_ms:g} ms of untimed "
                      "replays, events on the replay stream around the timed replays")
    roof["traffic"] = traffic_from_profile(w.case, kv_bytes)
    res["roofline"] = roof
    res["memory"] = memory_report(w, mk)
    if w.kind == "decode" and not args.no_graph and w.num_layers == 1:
        log("  grouped-query bf16 baseline on the same step ...")
        res["gqa8_bf16_baseline"] = gqa_report(w, mk, torch, ms_step)
    if w.kind == "append":
        log("  prefix cache: offload and restore of the cached prefixes ...")
        res["memory"]["prefix_cache"] = prefix_restore_report(w, st, mk, torch)
    del st, R
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("  timing the oracle on the host cores ...")
        budget = args.cpu_seconds if headline else args.extra_cpu_seconds
        res["cpu_baseline"] = cpu_baseline(w, kv_bytes, budget)
    return res


def hbm_probe(torch, mk, sizes, total=2 << 30, launches=40):
    """mqa_hbm_read_probe over a 2 GiB buffer: each launch reads a fresh slice
    of ``size`` bytes (slices rotate through the buffer, so neither the L2s
    nor the 256 MB Infinity Cache hold a slice from an earlier launch);
    launches are replayed from a HIP graph and timed with events on the
    replay stream.  Returns GB/s per size."""
    buf = torch.empty(total, dtype=torch.uint8, device="cuda")
    buf.random_(0, 256)
    sink = torch.zeros(mk.PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    out = {}
    for size in sizes:
        size = min(int(size) // 4096 * 4096, total)
        n = max(1, total // size)
        views = [buf[i * size:(i + 1) * size] for i in range(n)]
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for v in views:
                mk.hbm_read_probe(v, sink)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        per = max(1, launches // n)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per):
                for v in views:
                    mk.hbm_read_probe(v, sink)
        g.replay()
        torch.cuda.synchronize()
        E = torch.cuda.Event
        e0, e1 = E(enable_timing=True), E(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3 / (per * n)
        out[str(size)] = {"bytes": size, "us_per_read": round(sec * 1e6, 3),
                          "gbs": round(size / sec / 1e9, 1),
                          "pct_of_8000": round(100 * size / sec / 1e9 / HBM_PEAK_GBS, 2)}
    # the probe's own check: the XOR of the sink words is that of the buffer
    mk.hbm_read_probe(buf[:1 << 20], sink)
    got = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))
    want = int(np.bitwise_xor.reduce(buf[:1 << 20].cpu().numpy().view(np.uint32)))
    del buf, sink
    torch.cuda.empty_cache()
    return {"kernel": "hbm_read_kernel (mqa_hbm_read_probe): 128-bit loads, 8 in flight per lane",
            "by_size": out, "xor_check": got == want}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--case", type=int, default=3, choices=[1, 2, 3, 4],
                    help="the headline workload (default 3, the largest decode case)")
    ap.add_argument("--extra-cases", default="1,2,4",
                    help="other cases timed in the same run ('' for none)")
    ap.add_argument("--extra-steps", type=int, default=100)
    ap.add_argument("--replicas", type=int, default=0, help="0: enough for >= 1 GB of KV")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--extra-cpu-seconds", type=float, default=4.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the HBM streaming-read probe")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB copy (counter calibration) and exit")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="turn rocprofv3 --pmc runs in DIR into profiles/attention_counters_caseN.json")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every step from the host instead of replaying HIP graphs")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed replays of each graph before its timed region (ms of wall time)")
    args = ap.parse_args()

    if args.copy_probe:
        copy_probe()
        return
    if args.summarize_counters:
        cmds = open(os.path.join(args.summarize_counters, "commands.txt")).read().splitlines()
        summarize_counters(args.case, args.summarize_counters, cmds)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); the library runs on one GPU per process, and no sharding across GPUs is built.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import int8_mqa_kv_amd as mk
    import synth

    extras = [int(c) for c in args.extra_cases.split(",") if c.strip()]
    extras = [c for c in extras if c != args.case]
    head = measure_case(args.case, args, torch, mk, synth, headline=True)
    res = {
        "metric": METRIC, "value": head.pop("value"), "unit": head.pop("unit"), "n_gpus": 1,
        "steps": head.pop("steps"), "warmup": args.warmup, "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8", "data": "synthetic (seeded)", "config": head.pop("config"),
    }
    res.update(head)
    if extras:
        res["workloads"] = {}
        for c in extras:
            res["workloads"][f"case {c}"] = measure_case(c, args, torch, mk, synth, headline=False)
    if not args.no_probe:
        log("HBM streaming-read probe ...")
        sizes = [2 << 30, res["kv_bytes_per_step"]] + [
            v["kv_bytes_per_step"] for v in res.get("workloads", {}).values()
            if v["config"]["layers"] == 1]
        res["hbm_read_probe"] = hbm_probe(torch, mk, sizes)
    print(json.dumps(res), flush=True)


def slot_windows(w):
    """Per KV slot: 0 if a global layer reads it, else its widest window."""
    out = []
    for s_ in range(w.num_slots):
        wins = [int(x) for x, l in zip(w.layer_window, w.layer_slot) if int(l) == s_]
        out.append(0 if (not wins or 0 in wins) else max(wins))
    return out


def memory_report(w, mk, steps=200):
    """KV bytes one sequence of the workload holds at its longest context:
    int8 pages with windowed slots recycled (mqa_kv_footprint_bytes), the same
    cache without recycling, and a bf16 grouped-query cache (8 KV heads) with
    every layer global and its own slot; plus the host time the page table
    (mqa_page_table_advance) takes for one decode step of the whole batch."""
    ls, lw = w.layer_slot.tolist(), w.layer_window.tolist()
    L, ctx = len(ls), int(w.max_context)
    held = mk.kv_footprint_bytes(ls, lw, 1, w.head_dim, 1, 4, ctx)
    no_recycle = mk.kv_footprint_bytes(ls, [0] * L, 1, w.head_dim, 1, 4, ctx)
    gqa = mk.kv_footprint_bytes(list(range(L)), [0] * L, 8, w.head_dim, 2, 0, ctx, 0)
    slot_window = slot_windows(w)
    max_pages = (ctx + steps + 15) // 16
    pages = w.batch * w.num_slots * max_pages
    pt = mk.PageTable(0, pages, slot_window, w.batch, max_pages)
    start = [int(c) for c in w.context_lens]
    for b, c in enumerate(start):
        pt.advance(b, c, c)
    ctx_now = np.array(start, np.int64)
    ones = np.ones(w.batch, np.int32)
    t0 = time.perf_counter()
    for _ in range(steps):
        ctx_now += 1
        pt.advance_all(ctx_now, ones)
    dt = (time.perf_counter() - t0) / steps
    pt.close()
    return {"context": ctx, "kv_bytes_held_per_seq": held,
            "without_recycling": no_recycle,
            "recycling_factor": round(no_recycle / held, 3),
            "vs_gqa8_bf16_every_layer_global": round(gqa / held, 2),
            "page_table_us_per_step": round(dt * 1e6, 1),
            "page_table_timing": f"one mqa_page_table_advance_all call (a decode step of the "
                                 f"{w.batch} sequences) from Python, mean of {steps} steps"}


def gqa_report(w, mk, torch, mqa_ms, steps=200, kv_heads=8):
    """The same decode step as grouped-query attention with 8 bf16 KV heads
    (mqa_gqa_decode_bf16; "Character.AI: inference optimization", section
    03: multi-query attention is 8X smaller than grouped-query attention).
    One layer, the workload's batch, contexts, window and query heads; K/V
    seeded N(0,1) in bf16, pages of the keys the step reads only, several
    replicas so that the stream comes from HBM; HIP graph replay timed with
    events, like the multi-query step."""
    if w.num_layers != 1:
        return None
    dev = "cuda"
    d, hq, b = w.head_dim, w.num_q_heads, w.batch
    ctx = [int(c) for c in w.context_lens]
    win = int(w.layer_window[0])
    firsts = [max(0, c - win) // 16 if win > 0 else 0 for c in ctx]
    pages = [(c - 1) // 16 + 1 - f for c, f in zip(ctx, firsts)]
    max_pages = max((c - 1) // 16 + 1 for c in ctx)
    num_pages = sum(pages)
    pb = mk.gqa_page_bytes(kv_heads, d)
    keys = sum(c - (max(0, c - win) if win > 0 else 0) for c in ctx)
    kv_bytes = keys * kv_heads * 4 * d
    reps = max(1, math.ceil(1.0e9 / (num_pages * pb)))
    bt = np.zeros((b, max_pages), np.int32)
    sm, at = [], 0
    for i, (c, f, n) in enumerate(zip(ctx, firsts, pages)):
        bt[i, f:f + n] = np.arange(at, at + n)
        pos = np.arange(f * 16, c)
        sm.append((bt[i, pos // 16].astype(np.int64) * 16 + pos % 16))
        at += n
    sm_t = torch.from_numpy(np.concatenate(sm)).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(5005)
    pools = []
    for r in range(reps):
        pool = torch.zeros((num_pages, pb), dtype=torch.uint8, device=dev)
        k = torch.randn((sm_t.numel(), kv_heads, d), generator=g, device=dev).to(torch.bfloat16)
        v = torch.randn((sm_t.numel(), kv_heads, d), generator=g, device=dev).to(torch.bfloat16)
        mk.gqa_pack_bf16(k, v, sm_t, pool, kv_heads)
        pools.append(pool)
    q = torch.randn((b, hq, d), generator=g, device=dev).to(torch.bfloat16)
    outs = [torch.empty((b, hq, d), dtype=torch.float32, device=dev) for _ in range(reps)]
    bt_t = torch.from_numpy(bt).to(dev)
    cl = torch.tensor(ctx, dtype=torch.int32, device=dev)
    ws = mk.gqa_decode_workspace(b, hq, kv_heads, w.max_context, win, d)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for r in range(reps):
            mk.gqa_decode_bf16(q, outs[r], pools[r], kv_heads, bt_t, cl, w.max_context, win,
                               workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for r in range(reps):
            mk.gqa_decode_bf16(q, outs[r], pools[r], kv_heads, bt_t, cl, w.max_context, win,
                               workspace=ws)
    gr.replay()
    torch.cuda.synchronize()
    n = max(1, steps // reps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        gr.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (n * reps)
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    mqa_bytes = w.attended_keys() * (2 * d + 8)
    return {"kv_heads": kv_heads, "dtype": "bf16", "kv_bytes_per_step": kv_bytes,
            "us_per_step": round(ms * 1e3, 3), "gbs": round(gbs, 1),
            "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "bytes_vs_mqa_int8": round(kv_bytes / mqa_bytes, 2),
            "time_vs_mqa_int8_step": round(ms / mqa_ms, 2), "replicas": reps}


def prefix_restore_report(w, st, mk, torch):
    """The hybrid turn starts from a cross-turn cache hit: every sequence's
    cached prefix (context - q_len tokens) is offloaded page by page from the
    pool into a pinned host arena (mqa_prefix_cache_insert, device -> host),
    looked up by its token ids, and restored into the pool pages the block
    table gives (mqa_prefix_cache_restore, host -> device).  One call per
    sequence, timed end to end with events; token ids are seeded synthetic."""
    R = st["reps"][0]
    bt = np.ascontiguousarray(w.block_table)
    slot_window = slot_windows(w)
    prefix = (w.context_lens - w.q_lens).astype(np.int64)
    rng = np.random.default_rng(4004)
    tokens = [rng.integers(0, 128000, int(c)).astype(np.int32) for c in w.context_lens]
    held = 0
    for b in range(w.batch):
        k = int(prefix[b]) // 16
        rows = bt[:, b, :k]
        held += int(np.count_nonzero((rows != w.poison_page) & (rows >= 0)))
    entry = -(-mk.page_bytes(w.head_dim) // 256) * 256
    pc = mk.PrefixCache(256 * 1024 + held * entry, slot_window, w.head_dim)
    E = torch.cuda.Event
    e0, e1, e2, e3 = (E(enable_timing=True) for _ in range(4))
    torch.cuda.synchronize()
    e0.record()
    for b in range(w.batch):
        pc.insert(tokens[b][:int(prefix[b])], R.pool, bt, b, invalid_page=w.poison_page)
    e1.record()
    torch.cuda.synchronize()
    matched = [pc.lookup(tokens[b]) for b in range(w.batch)]
    e2.record()
    for b in range(w.batch):
        pc.restore(tokens[b], matched[b], R.pool, bt, b, invalid_page=w.poison_page)
    e3.record()
    torch.cuda.synchronize()
    st_ = pc.stats()
    pb = mk.page_bytes(w.head_dim)
    off_b = st_["entries_inserted"] * pb
    res_b = st_["entries_restored"] * pb
    out = {"entries": pc.entries(), "arena_bytes": 256 * 1024 + held * entry,
           "offload_bytes": off_b,
           "offload_gbs": round(off_b / (e0.elapsed_time(e1) * 1e-3) / 1e9, 2),
           "restore_bytes": res_b,
           "restore_gbs": round(res_b / (e2.elapsed_time(e3) * 1e-3) / 1e9, 2),
           "matched_tokens_fraction": round(sum(matched) / float(prefix.sum()), 4),
           "timing": f"{w.batch} calls each way (one per sequence), events around the calls"}
    pc.close()
    return out


def counters_path(case):
    return os.path.join(ROOT, "profiles", f"attention_counters_case{case}.json")


def traffic_from_profile(case, kv_bytes):
    """HBM bytes per launch of the dominant kernel (reads + writes) from the
    committed counter summary, when it was taken on the current kernel
    sources (else null)."""
    p = counters_path(case)
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_call")


COPY_BYTES = 1 << 30


def copy_probe():
    """A plain copy of known size (1 GiB read + 1 GiB written), run under the
    same counters as the attention kernels to scale FETCH_SIZE / WRITE_SIZE
    into bytes."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copy probe done")


def _read_counters(d):
    """{kernel name: {counter: [values per dispatch]}} from a rocprofv3 csv dir."""
    import csv
    import glob
    out = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            out.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    return out


def summarize_counters(case, d, cmds):
    """Turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE, each for the
    copy probe and for the case) into HBM bytes per launch of the dominant
    kernel."""
    def per_dispatch(run, counter, pred):
        data = _read_counters(os.path.join(d, run))
        vals = [v for k, cs in data.items() if pred(k) for v in cs.get(counter, [])]
        return vals
    is_copy = lambda k: "copy" in k.lower() or "elementwise" in k.lower()
    fc = per_dispatch("fetch_copy", "FETCH_SIZE", is_copy)
    wc = per_dispatch("write_copy", "WRITE_SIZE", is_copy)
    fetch_scale = COPY_BYTES / max(fc)      # bytes per counter unit (largest = the 1 GiB copy)
    write_scale = COPY_BYTES / max(wc)
    out = {"case": case, "kernel_source_hash": kernel_source_hash(), "commands": cmds,
           "copy_fetch_units": max(fc), "copy_write_units": max(wc),
           "fetch_bytes_per_unit": fetch_scale, "write_bytes_per_unit": write_scale,
           "kernels": {}}
    total = 0.0
    for run, counter, scale in (("fetch_case", "FETCH_SIZE", fetch_scale),
                                ("write_case", "WRITE_SIZE", write_scale)):
        for k, cs in _read_counters(os.path.join(d, run)).items():
            if not any(t in k for t in ("decode_kernel", "append_kernel")):
                continue
            v = cs.get(counter, [])
            if not v:
                continue
            name = k.replace("void ", "").split(">(")[0] + ">"
            mean = float(np.mean(v))
            out["kernels"].setdefault(name, {})[counter] = {"mean_units": mean,
                                                             "bytes": mean * scale,
                                                             "dispatches": len(v)}
            total += mean * scale
    out["hbm_bytes_per_call"] = total
    os.makedirs(os.path.dirname(counters_path(case)), exist_ok=True)
    json.dump(out, open(counters_path(case), "w"), indent=1)
    log(f"wrote {counters_path(case)}: {total / 1e6:.2f} MB per call")


if __name__ == "__main__":
    main()
