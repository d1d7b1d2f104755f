#!/usr/bin/env python3
"""Benchmark of deferred-RoPE attention over a position-agnostic paged KV pool on one MI355X.

Headline (one step = the prefill of a 2048-token chunk for each of 4
requests): the Llama-3.1-70B single-layer attention shape in bf16 (64 query
heads, 8 KV heads, head_dim 128, RoPE theta 5e5, blocks of 16 tokens).  Each
request holds 64 distinct documents of 512 tokens drawn Zipf(1.0) from a pool
of 4096 and placed in random order (32768 context tokens); its 2048 new
tokens at positions 32768..34815 are prefilled causally over them.  The pool
holds content-only K/V; RoPE is applied inside the kernel.  Inputs are seeded
synthetic data already resident in HBM; the chunk's K/V are appended once
before timing.  Every timed step runs cold: a 1 GiB read evicts the 256 MiB
last-level cache before it, outside the step's own events (a read, so that no
dirty lines of the eviction are written back inside the timed span).

Also on the same line: the rotation-free control on the same inputs (the
deferred-RoPE overhead); the 128 decode steps that follow the chunk (split-K,
cold and warm, HBM roofline on unique bytes with the counter bytes beside
them); the Llama-3.1-8B prefill and decode shapes and the MQA stress mixed
step (32 prefills and 96 decodes on two streams) as extras; measured MFMA and
HBM peaks; block-pool hit ratios; and the fp64 CPU oracle timed on a stated
sample of the headline workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W]
  python bench.py --calibrate-copy           # a plain copy kernel, for counter scaling
  python bench.py --summarize-rocprof DIR    # print a rocprofv3 CSV directory as a summary
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill TFLOP/s + decode KV GB/s (% of MI355X peak), deferred-RoPE attention"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
FLUSH_BYTES = 1 << 30          # read before each cold step: four times the 256 MiB last-level (MALL) cache
KERNEL_SRC = os.path.join(ROOT, "position_agnostic_kv_pool_amd", "csrc", "lazyattn_kernels.hip")
PROBE_LIB = os.path.join(ROOT, "position_agnostic_kv_pool_amd", "liblazyattn_probe.so")
COUNTERS = {
    "prefill70b": os.path.join(ROOT, "profiles", "prefill_bf16_llama70b_counters.txt"),
    "decode70b": os.path.join(ROOT, "profiles", "decode_bf16_llama70b_counters.txt"),
    "prefill8b": os.path.join(ROOT, "profiles", "prefill_bf16_llama8b_counters.txt"),
    "decode8b": os.path.join(ROOT, "profiles", "decode_bf16_llama8b_counters.txt"),
    "mqa": os.path.join(ROOT, "profiles", "prefill_decode_mqa_counters_and_trace.txt"),
}
HEADLINE_WORKLOAD = ("prefill, Llama-3.1-70B attention layer (Hq 64, Hkv 8, d 128, RoPE theta 5e5, block 16): "
                     "2048-token causal chunk of each of 4 requests over 64 Zipf(1.0) documents x 512 tokens "
                     "(32k context); content-only pool, RoPE applied at attention time (each request's keys "
                     "turned once per call, queries in the attention kernel); cold (a 1 GiB read evicts the "
                     "last-level cache before each step)")


def kernel_code(text: str) -> str:
    """The kernel source without its comments and with runs of whitespace collapsed: what the
    compiler sees, so that a comment edit does not orphan counter summaries taken on the same code."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """sha256/16 of the kernel code (comments and layout stripped, see kernel_code)."""
    with open(KERNEL_SRC, encoding="utf-8") as f:
        return hashlib.sha256(kernel_code(f.read()).encode()).hexdigest()[:16]


def read_mqa_decode_counters(path: str):
    """{skew: fetch + write bytes per RoPE decode step} from the committed MQA summary, if it
    was taken on the current kernel code; else {}."""
    if not os.path.exists(path):
        return {}
    out, sha = {}, None
    with open(path) as f:
        for line in f:
            if line.startswith("kernel_code_sha256_16:"):
                sha = line.split(":", 1)[1].strip()
            elif line.startswith("decode RoPE"):
                parts = line.split()
                skew = parts[3].rstrip(":")
                fetch = float(parts[parts.index("fetch_GB") + 1])
                write = float(parts[parts.index("write_GB") + 1])
                out[skew] = (fetch + write) * 1e9
    return out if sha == kernel_source_hash() else {}


def read_counter_summary(path: str):
    """HBM bytes per dispatch (FETCH_SIZE + WRITE_SIZE, each scaled by the copy calibration)
    from a committed summary, if it was taken on the current kernel source; else None."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_code_sha256_16") != kernel_source_hash():
        return None
    try:
        fetch = float(kv["fetch_kib_per_dispatch"]) * float(kv["fetch_scale"])
        write = float(kv["write_kib_per_dispatch"]) * float(kv["write_scale"])
    except (KeyError, ValueError):
        return None
    return round((fetch + write) * 1024.0)


# ---------------------------------------------------------------------------
# rocprofv3 CSV summaries
# ---------------------------------------------------------------------------
def summarize_rocprof(d: str) -> None:
    import csv
    from collections import defaultdict
    for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        print(f"# kernel stats: {os.path.relpath(path, d)}")
        with open(path) as f:
            rows = list(csv.DictReader(f))
        for r in rows:
            name = r.get("Name", r.get("KernelName", "?"))
            print(f"{name[:90]:90s} calls {r.get('Calls')}  avg_ns {float(r.get('AverageNs', 0)):.0f}  "
                  f"min_ns {r.get('MinNs')}  max_ns {r.get('MaxNs')}  pct {float(r.get('Percentage', 0)):.2f}")
    for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
        # per-kernel median dispatch duration (the stats file gives only the mean)
        by = defaultdict(list)
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r.get("Kernel_Name", r.get("Kernel-Name", "?"))
                try:
                    by[name].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                except (KeyError, ValueError):
                    pass
        print(f"# kernel trace medians: {os.path.relpath(path, d)}")
        for name, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
            v = sorted(v)
            print(f"{name[:90]:90s} dispatches {len(v)}  median_ns {v[len(v) // 2]}  p10_ns {v[len(v) // 10]}  "
                  f"p90_ns {v[(9 * len(v)) // 10]}")
    for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        print(f"# counters: {os.path.relpath(path, d)}")
        acc = defaultdict(list)
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r.get("Kernel_Name", r.get("Kernel-Name", "?"))
                acc[(name, r.get("Counter_Name"))].append(float(r.get("Counter_Value", 0)))
        for (name, cn), vals in sorted(acc.items()):
            print(f"{name[:90]:90s} {cn:24s} dispatches {len(vals)}  mean_per_dispatch {sum(vals) / len(vals):.1f}")


# ---------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------
def prefill_flops(pb, head_dim: int, num_q_heads: int, token_subset=None) -> float:
    """4 * D * Hq * sum over queries of the keys each one sees (QK^T and PV, causal)."""
    tot = 0
    cu = pb["cu_q_lens"]
    for r, L in enumerate(pb["ctx_lens"]):
        m = int(cu[r + 1] - cu[r])
        p0 = int(L) - m
        if token_subset is None:
            tot += m * p0 + m * (m + 1) // 2        # sum_{j<m} (p0 + j + 1)
        elif r in token_subset:
            tot += sum(p0 + int(j) + 1 for j in token_subset[r])
    return 4.0 * head_dim * num_q_heads * tot


def decode_bytes(d, wl) -> dict:
    """Per-step bytes: logical (what a per-request paged kernel streams), unique (each
    (block, KV head) once: the HBM floor when shared blocks are read once), plus queries,
    outputs and table words."""
    s = wl.spec
    esz = 2 if s.dtype == "bf16" else 4
    R = len(d["ctx_lens"])
    kv_logical = sum(int(L) for L in d["ctx_lens"]) * s.num_kv_heads * s.head_dim * 2 * esz
    blocks = set()
    for i in range(R):
        n = int(d["num_entries"][i])
        blocks.update(int(b) for b in d["table_blocks"][i, :n])
    kv_unique = len(blocks) * s.num_kv_heads * s.block_size * s.head_dim * 2 * esz
    other = 2 * R * s.num_q_heads * s.head_dim * esz + int(sum(d["num_entries"])) * 8 + R * 8
    return {"logical": kv_logical + other, "unique": kv_unique + other, "kv_logical": kv_logical}


def med(v):
    v = sorted(v)
    return v[len(v) // 2]


def require_finite(torch, what, *outs):
    """Every timed call's output must be finite: NaN or inf there would mean the call
    read pool slots its setup never wrote, so it did not time the real workload."""
    for o in outs:
        if not bool(torch.isfinite(o.float()).all()):
            raise RuntimeError(f"{what}: non-finite output; the benchmark's inputs are not set up")


def pct(v):
    v = sorted(v)
    return [v[len(v) // 10], v[len(v) // 2], v[(9 * len(v)) // 10]]


def probe_lib():
    """liblazyattn_probe.so (peak probes: MFMA issue rate, streaming read, chunk gather)."""
    L = ctypes.CDLL(PROBE_LIB)
    L.lazyattn_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.lazyattn_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p]
    L.lazyattn_probe_gather_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_void_p, ctypes.c_void_p]
    return L


class Timer:
    """HIP events on the stream the kernels are launched on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.flush_buf = None
        self.probe = probe_lib()

    def busy(self):
        # keep the GPU busy while the host enqueues the timed launches, so host
        # launch latency never shows up between the events
        if hasattr(self.torch.cuda, "_sleep"):
            self.torch.cuda._sleep(2_000_000)

    def flush(self, rep=0):
        """Evict the last-level cache by reading FLUSH_BYTES of another buffer.  A write
        would leave that many dirty lines, whose write-back then lands inside the next timed
        span (measured: +58 us on one 70B decode step)."""
        t = self.torch
        if self.flush_buf is None:
            self.flush_buf = t.ones(FLUSH_BYTES, dtype=t.uint8, device="cuda")
            self.flush_sink = t.empty(8192 * 256, dtype=t.float32, device="cuda")
        st = t.cuda.current_stream().cuda_stream
        assert self.probe.lazyattn_probe_hbm_read(self.flush_buf.data_ptr(), FLUSH_BYTES // 16, 8192,
                                                  self.flush_sink.data_ptr(), st) == 0

    def release(self):
        self.flush_buf = None

    def span(self, fn, n):
        """ms per call of n back-to-back calls between two events."""
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        self.busy()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        t.cuda.synchronize()
        return a.elapsed_time(b) / n

    def steps(self, fns, n, cold=True, arg=False):
        """n steps; step i runs fns[0](i), fns[1](i), ... (or without the index), each
        between its own events; with ``cold`` the last-level cache is flushed before every
        step, outside its events.  Returns per-step lists of per-function ms."""
        t = self.torch
        ev = [[t.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(n)]
        t.cuda.synchronize()
        self.busy()
        for i in range(n):
            if cold:
                self.flush(i)
            ev[i][0].record()
            for j, fn in enumerate(fns):
                fn(i) if arg else fn()
                ev[i][j + 1].record()
        t.cuda.synchronize()
        return [[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(len(fns))] for i in range(n)]

    def rounds(self, variants, n, cold=True, arg=False):
        """n rounds; each times one step of every variant (a list of functions, as for
        steps()), in an order rotated by one place per round, each step cold as in steps().
        Variants compared this way see the same clocks and temperatures on average, so
        their ratios carry no drift over the run.  Returns, per variant, its per-step
        lists of per-function ms."""
        t = self.torch
        k = len(variants)
        ev = [[[t.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(n)]
              for fns in variants]
        t.cuda.synchronize()
        self.busy()
        for i in range(n):
            for j in range(k):
                v = (i + j) % k
                if cold:
                    self.flush(i)
                ev[v][i][0].record()
                for m, fn in enumerate(variants[v]):
                    fn(i) if arg else fn()
                    ev[v][i][m + 1].record()
        t.cuda.synchronize()
        return [[[e[i][m].elapsed_time(e[i][m + 1]) for m in range(len(fns))] for i in range(n)]
                for e, fns in zip(ev, variants)]

    def span_rounds(self, fns, n, reps=3):
        """Median ms per call of each function over reps rounds of back-to-back spans of n
        calls, the functions' order rotated by one place per round."""
        out = [[] for _ in fns]
        for r in range(reps):
            for j in range(len(fns)):
                v = (r + j) % len(fns)
                out[v].append(self.span(fns[v], n))
        return [med(x) for x in out]


# ---------------------------------------------------------------------------
# the headline: Llama-3.1-70B 32k chunk prefill, then its decode steps
# ---------------------------------------------------------------------------
def bench_headline(torch, args, W, staging, _abi):
    wl = W.build_workload(W.spec(4, n_decode=args.decode_steps))
    s = wl.spec
    pools = staging.DevicePools(wl, "cuda")
    pb = wl.prefill_batch()
    cfg = staging.config_for(s)
    cfg_none = staging.config_for(s, pe="none")
    staging.append_tokens(cfg, pools, pb, s.dtype, "cuda")
    call = staging.PrefillCall(cfg, s, pb, "cuda")
    call_none = staging.PrefillCall(cfg_none, s, pb, "cuda")
    # the same RoPE call with the keys turned inside the attention kernel (the library
    # turns them once first for this chunk of 64 query tiles per request and KV head)
    call_fused = staging.PrefillCall(staging.config_for(s, keys="fused"), s, pb, "cuda")
    keys_once = _abi.prefill_workspace_size(cfg, len(pb["ctx_lens"]), call.total_q, call.max_q_len,
                                            call.tables.batch.max_entries, call.num_splits) > \
        _abi.prefill_workspace_size(call_fused.cfg, len(pb["ctx_lens"]), call.total_q, call.max_q_len,
                                    call.tables.batch.max_entries, call.num_splits)
    torch.cuda.synchronize()
    timer = Timer(torch)
    fns = [lambda: call.attend(pools)] + ([call.merge] if call.splits > 1 else [])
    fns_none = [lambda: call_none.attend(pools)] + ([call_none.merge] if call_none.splits > 1 else [])
    fns_fused = [lambda: call_fused.attend(pools)] + ([call_fused.merge] if call_fused.splits > 1 else [])
    for _ in range(args.warmup):
        call.run(pools)
    torch.cuda.synchronize()
    # the timed steps: exactly args.steps cold steps
    st = timer.steps(fns, args.steps, cold=True)
    step_ms = [sum(x) for x in st]
    kern_ms = [x[0] for x in st]
    print(f"# headline prefill: {sum(step_ms) / len(step_ms) * 1e3:.1f} us/step (cold)", file=sys.stderr, flush=True)
    # RoPE against the rotation-free control (and the keys turned in the attention
    # kernel): alternating cold steps, then alternating warm spans
    st_rope, st_none, st_fused = timer.rounds([fns, fns_none, fns_fused], max(6, args.steps // 2), cold=True)
    warm, warm_none = timer.span_rounds([lambda: call.run(pools), lambda: call_none.run(pools)],
                                        max(3, args.steps // 4))
    require_finite(torch, "70B prefill", call.out, call_none.out, call_fused.out)
    flops = prefill_flops(pb, s.head_dim, s.num_q_heads)
    pre = dict(ms=sum(step_ms) / len(step_ms), step_ms=step_ms, kern_ms=kern_ms, flops=flops, splits=call.splits,
               rope_kern_ms=[x[0] for x in st_rope], none_kern_ms=[x[0] for x in st_none],
               fused_kern_ms=[x[0] for x in st_fused], keys_once=keys_once,
               warm_ms=warm, warm_none_ms=warm_none,
               seq_len=int(max(pb["ctx_lens"])), R=len(pb["ctx_lens"]))
    del call, call_none, call_fused

    # decode steps 0..n-1: every step's token is appended first (setup); a step's call
    # reads only its own context (ctx_lens, num_entries), so later tokens are invisible to it
    n = args.decode_steps
    allt = wl.tokens_before_step(n)
    staging.append_tokens(cfg, pools, allt, s.dtype, "cuda")
    steps = [wl.decode_step(i) for i in range(n)]
    calls = [staging.DecodeCall(cfg, s, d, "cuda") for d in steps]
    calls_none = [staging.DecodeCall(cfg_none, s, d, "cuda") for d in steps]
    by = [decode_bytes(d, wl) for d in steps]
    torch.cuda.synchronize()
    for c in calls[:3]:
        c.run(pools)
    # every step cold, the RoPE kernel and the rotation-free control in alternating order;
    # then warm (three back-to-back calls of the step), alternating the same way
    dec = {}
    variants = [[lambda i, cs=cs: cs[i].attend(pools), lambda i, cs=cs: cs[i].merge()] for cs in (calls, calls_none)]
    cold = timer.rounds(variants, n, cold=True, arg=True)
    warm = timer.rounds([[lambda i, cs=cs: (cs[i].run(pools), cs[i].run(pools), cs[i].run(pools))]
                         for cs in (calls, calls_none)], n, cold=False, arg=True)
    for v, (tag, cs) in enumerate((("rope", calls), ("none", calls_none))):
        require_finite(torch, f"70B decode ({tag})", *[c.out for c in cs])
        dec[tag] = dict(cold_att=[x[0] for x in cold[v]], cold_merge=[x[1] for x in cold[v]],
                        warm_step=[x[0] / 3.0 for x in warm[v]])
    print(f"# headline decode: {sum(dec['rope']['cold_att']) / n * 1e3:.1f} us attention per step (cold)",
          file=sys.stderr, flush=True)
    # decode step 0's own chunk list (each entry's K and V chunk of every KV head, in the
    # kernel's order) read by a plain gather kernel, cold: what this access pattern reaches
    # on this GPU, next to the decode kernel's time for the same step
    d0 = steps[0]
    chunk = s.block_size * s.head_dim * 2
    dv = pools.v.data_ptr() - pools.k.data_ptr()
    offs = []
    for r in range(len(d0["ctx_lens"])):
        blk = d0["table_blocks"][r, :int(d0["num_entries"][r])].astype("int64")
        for hh in range(s.num_kv_heads):
            for b in blk:
                o = (int(b) * s.num_kv_heads + hh) * chunk
                offs += [o, dv + o]
    ot = torch.tensor(offs, dtype=torch.int64, device="cuda")
    gsink = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream

    def gather():
        assert timer.probe.lazyattn_probe_gather_read(pools.k.data_ptr(), ot.data_ptr(), len(offs), chunk, 2048,
                                                      gsink.data_ptr(), st) == 0

    gather()
    g_ms = med([x[0] for x in timer.steps([gather], 7, cold=True)])
    d0_ms = med([x[0] for x in timer.steps([lambda: calls[0].attend(pools)], 7, cold=True)])
    gather_probe = dict(us_cold=round(g_ms * 1e3, 2), bytes=len(offs) * chunk,
                        GBps=round(len(offs) * chunk / (g_ms * 1e-3) / 1e9, 1),
                        decode_step0_attention_us_cold=round(d0_ms * 1e3, 2),
                        decode_vs_gather=round(g_ms / d0_ms, 4))
    del ot, gsink
    timer.release()
    out = dict(pre=pre, dec=dec, bytes=by, splits=calls[0].splits, n=n, wl=wl, pb=pb, steps=steps,
               gather_probe=gather_probe)
    del calls, calls_none, pools
    torch.cuda.empty_cache()
    return out


def headline_json(h, args):
    pre, dec, by, n = h["pre"], h["dec"], h["bytes"], h["n"]
    flops = pre["flops"]
    tflops = flops / (pre["ms"] * 1e-3) / 1e12
    k_med = med(pre["kern_ms"])
    kernel_tflops = flops / (k_med * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(kernel_tflops, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(kernel_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": read_counter_summary(COUNTERS["prefill70b"]),
                "kernel": ("turn_keys_kernel + prefill_bf16_kernel<KEYS_TURNED>" if pre["keys_once"]
                           else "prefill_bf16_kernel<ROPE>"),
                "flops_per_launch": flops,
                "launch_us_median_cold": round(k_med * 1e3, 2),
                "launch_us_p10_p50_p90_cold": [round(x * 1e3, 2) for x in pct(pre["kern_ms"])],
                "launch_us_warm_back_to_back": round(pre["warm_ms"] * 1e3, 2),
                "note": "achieved = algorithmic FLOPs / median cold launch (events around the call's kernels: "
                        "with the keys turned once, the key-turning kernel and the attention kernel together)"}
    none_med = med(pre["none_kern_ms"])
    rope_med = med(pre["rope_kern_ms"])
    fused_med = med(pre["fused_kern_ms"])
    rope_overhead = {"what": "RoPE kernel(s) against the rotation-free control on the same inputs, timed in "
                             "alternating order (medians); keys turned once first (the library's choice for "
                             "this chunk) and, beside it, turned inside the attention kernel",
                     "prefill_keys": "turned once" if pre["keys_once"] else "turned in the attention kernel",
                     "prefill_rope_us_cold": round(rope_med * 1e3, 2),
                     "prefill_norotation_us_cold": round(none_med * 1e3, 2),
                     "prefill_overhead_cold": round(rope_med / none_med - 1.0, 4),
                     "prefill_keys_in_kernel_us_cold": round(fused_med * 1e3, 2),
                     "prefill_keys_in_kernel_overhead_cold": round(fused_med / none_med - 1.0, 4),
                     "prefill_rope_us_warm": round(pre["warm_ms"] * 1e3, 2),
                     "prefill_norotation_us_warm": round(pre["warm_none_ms"] * 1e3, 2),
                     "prefill_overhead_warm": round(pre["warm_ms"] / pre["warm_none_ms"] - 1.0, 4),
                     # rotation work: 3 flops per rotated key element, each key tile rotated once per
                     # work-group of 256 query rows (the pages' 3/(4M) cost model with M = 256)
                     "prefill_rotation_flop_fraction": round(3.0 / (4.0 * 256), 5)}
    r, z = dec["rope"], dec["none"]
    att = sum(r["cold_att"]) / n
    mrg = sum(r["cold_merge"]) / n
    uniq = sum(b["unique"] for b in by) / n
    logical = sum(b["logical"] for b in by) / n
    traffic = read_counter_summary(COUNTERS["decode70b"])
    gbs_unique = uniq / (att * 1e-3) / 1e9
    decode = {
        "workload": f"decode steps 0..{n - 1} after the chunk: 4 requests x 34817..{34816 + n} tokens, split-K "
                    f"({h['splits']} splits) + merge; cold (a 1 GiB read evicts the cache before each step)",
        "us_per_step_cold": round((att + mrg) * 1e3, 2), "attention_kernel_us_cold": round(att * 1e3, 2),
        "merge_kernel_us_cold": round(mrg * 1e3, 2),
        "us_per_step_warm": round(sum(r["warm_step"]) / n * 1e3, 2),
        "tokens_per_s_cold": round(h["pre"]["R"] / ((att + mrg) * 1e-3), 1),
        "splits": h["splits"],
        "roofline": {"bound": "hbm", "achieved": round(gbs_unique, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs_unique / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": "decode_bf16_kernel<ROPE,1>",
                     "bytes_per_launch_unique": round(uniq),
                     "counter_GBps": round(traffic / (att * 1e-3) / 1e9, 1) if traffic else None,
                     "bytes_per_launch_logical": round(logical),
                     "logical_GBps_context": round(logical / (att * 1e-3) / 1e9, 1),
                     "note": "achieved = unique bytes (each block and KV head once, plus q, out, table words) / "
                             "mean cold attention-kernel time; logical bytes re-count shared blocks"},
        "gather_probe": dict(what="step 0's K and V chunks (4 KiB each, every entry and KV head, the kernel's "
                                  "order) read by a plain gather kernel, cold: the access pattern's practical "
                                  "roofline on this GPU", **h["gather_probe"]),
        "norotation_attention_us_cold": round(sum(z["cold_att"]) / n * 1e3, 2),
        "rope_overhead_cold": round(att / (sum(z["cold_att"]) / n) - 1.0, 4),
        "rope_overhead_warm": round(sum(r["warm_step"]) / sum(z["warm_step"]) - 1.0, 4),
    }
    out = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(pre["ms"], 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": HEADLINE_WORKLOAD, "global_batch": pre["R"], "seq_len": pre["seq_len"],
                   "parallelism": "single-gpu", "key_splits": pre["splits"],
                   "step": "one prefill call (key-turning kernel and attention kernel; the merge too when the key "
                           "range is split)"},
        "roofline": roofline,
        "rope_overhead": rope_overhead,
        "decode": decode,
    }
    return out


# ---------------------------------------------------------------------------
# extras: the Llama-3.1-8B prefill and decode shapes
# ---------------------------------------------------------------------------
def bench_llama8b_prefill(torch, args, W, staging, _abi):
    wl = W.build_workload(W.spec(2))
    s = wl.spec
    pools = staging.DevicePools(wl, "cuda")
    pb = wl.prefill_batch()
    cfg = staging.config_for(s)
    staging.append_tokens(cfg, pools, pb, s.dtype, "cuda")
    call = staging.PrefillCall(cfg, s, pb, "cuda")
    call_none = staging.PrefillCall(staging.config_for(s, pe="none"), s, pb, "cuda")
    fpools = staging.FramedPools(wl, cfg, "cuda")
    staging.append_tokens(cfg, fpools, pb, s.dtype, "cuda")
    call_framed = staging.PrefillCall(cfg, s, pb, "cuda", framed=True)
    cfg8 = staging.config_for(s, kv_format="fp8")
    pools8 = staging.WrittenPools(wl, cfg8, "cuda")
    staging.append_tokens(cfg8, pools8, pb, s.dtype, "cuda")
    call8 = staging.PrefillCall(cfg8, s, pb, "cuda")
    torch.cuda.synchronize()
    timer = Timer(torch)
    for _ in range(5):
        call.run(pools)
    timer.span(lambda: call.attend(pools), 200)        # clocks settle
    n = 20
    res = {}
    # the four variants in alternating order (cold steps, then warm spans)
    cases = (("rope", call, pools), ("none", call_none, pools), ("framed", call_framed, fpools), ("fp8", call8, pools8))
    cold = timer.rounds([[lambda c=c, p=p: c.attend(p)] + ([c.merge] if c.splits > 1 else []) for _, c, p in cases],
                        n, cold=True)
    warm_att = timer.span_rounds([lambda c=c, p=p: c.attend(p) for _, c, p in cases], n)
    warm_step = timer.span_rounds([lambda c=c, p=p: c.run(p) for _, c, p in cases], n)
    for v, (tag, c, p) in enumerate(cases):
        res[tag] = dict(cold_att=med([x[0] for x in cold[v]]), cold_step=med([sum(x) for x in cold[v]]),
                        warm_att=warm_att[v], warm_step=warm_step[v])
        require_finite(torch, f"8B prefill ({tag})", c.out)
    del fpools, pools8
    mat = staging.MaterializedPrefill(s, pb, "cuda")
    mat.run(pools)
    base = dict(materialize=timer.span(lambda: mat.materialize(pools), n),
                rotate_queries=timer.span(lambda: mat.rotate_queries(), n),
                attention=timer.span(lambda: mat.attend(), n),
                total=timer.span(lambda: mat.run(pools), n), copied_bytes=mat.bytes_copied)
    del mat
    timer.release()
    flops = prefill_flops(pb, s.head_dim, s.num_q_heads)
    r = res["rope"]
    traffic = read_counter_summary(COUNTERS["prefill8b"])
    out = {
        "workload": "prefill, Llama-3.1-8B attention layer (Hq 32, Hkv 8, d 128, RoPE theta 5e5, block 16): "
                    "16 requests x 8 Zipf(1.0) documents x 512 tokens + 64-token causal query",
        "key_splits": call.splits,
        "step_us_cold": round(r["cold_step"] * 1e3, 2), "attention_us_cold": round(r["cold_att"] * 1e3, 2),
        "step_us_warm": round(r["warm_step"] * 1e3, 2), "attention_us_warm": round(r["warm_att"] * 1e3, 2),
        "TFLOPs_step_cold": round(flops / (r["cold_step"] * 1e-3) / 1e12, 2),
        "roofline": {"bound": "mfma", "achieved": round(flops / (r["cold_att"] * 1e-3) / 1e12, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / (r["cold_att"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "flops_per_launch": flops},
        "rope_overhead_cold": round(r["cold_att"] / res["none"]["cold_att"] - 1.0, 4),
        "rope_overhead_warm": round(r["warm_att"] / res["none"]["warm_att"] - 1.0, 4),
        "norotation_attention_us_cold": round(res["none"]["cold_att"] * 1e3, 2),
        "document_frames": {"attention_us_cold": round(res["framed"]["cold_att"] * 1e3, 2),
                            "overhead_vs_norotation_cold": round(res["framed"]["cold_att"] /
                                                                 res["none"]["cold_att"] - 1.0, 4)},
        "fp8_pool": {"attention_us_cold": round(res["fp8"]["cold_att"] * 1e3, 2),
                     "vs_bf16_pool": round(r["cold_att"] / res["fp8"]["cold_att"], 3)},
        "materialize_baseline": {
            "what": "private copies of every request's blocks with K rotated at absolute positions, queries "
                    "rotated, then the rotation-free kernel over the copy (the approach deferred RoPE replaces); warm",
            "materialize_us": round(base["materialize"] * 1e3, 2),
            "rotate_queries_us": round(base["rotate_queries"] * 1e3, 2),
            "attention_us": round(base["attention"] * 1e3, 2), "total_us": round(base["total"] * 1e3, 2),
            "copied_bytes": int(base["copied_bytes"]),
            "deferred_step_us_warm": round(r["warm_step"] * 1e3, 2),
            "deferred_speedup": round(base["total"] / r["warm_step"], 3)},
    }
    del pools
    torch.cuda.empty_cache()
    return out


def bench_llama8b_decode(torch, args, W, staging, _abi, n_steps: int):
    """Decode steps 0..n_steps-1 of the 8B decode shape, cold and warm (3 back-to-back
    launches of the same step), with the rotation-free, framed and FP8 variants warm."""
    wl = W.build_workload(W.spec(3, n_decode=max(n_steps, 1)))
    s = wl.spec
    cfg = staging.config_for(s)
    cfg_none = staging.config_for(s, pe="none")
    cfg8 = staging.config_for(s, kv_format="fp8")
    allt = wl.tokens_before_step(n_steps)
    pools = staging.DevicePools(wl, "cuda")
    staging.append_tokens(cfg, pools, allt, s.dtype, "cuda")
    fpools = staging.FramedPools(wl, cfg, "cuda")
    staging.append_tokens(cfg, fpools, allt, s.dtype, "cuda")
    pools8 = staging.WrittenPools(wl, cfg8, "cuda")
    staging.append_tokens(cfg8, pools8, allt, s.dtype, "cuda")
    fpools8 = staging.FramedPools(wl, cfg8, "cuda")
    staging.append_tokens(cfg8, fpools8, allt, s.dtype, "cuda")
    torch.cuda.synchronize()
    timer = Timer(torch)
    acc = {k: 0.0 for k in ("cold", "cold_none", "cold_runs", "warm", "none", "runs", "framed", "fp8", "fp8f",
                            "plan_ms")}
    tot = {"logical": 0, "unique": 0, "kv_logical": 0}
    splits = 0
    for step in range(-2, n_steps):          # two untimed warm-up rounds on step 0's inputs
        d = wl.decode_step(max(step, 0))
        call = staging.DecodeCall(cfg, s, d, "cuda")
        cn = staging.DecodeCall(cfg_none, s, d, "cuda")
        cf = staging.DecodeCall(cfg, s, d, "cuda", framed=True)
        c8 = staging.DecodeCall(cfg8, s, d, "cuda")
        c8f = staging.DecodeCall(cfg8, s, d, "cuda", framed=True)
        t0 = time.perf_counter()
        cr = staging.RunDecodeCall(cfg, s, d, pools.num_blocks, "cuda")     # host plan + its upload
        plan_ms = (time.perf_counter() - t0) * 1e3
        splits = call.splits
        trio = timer.rounds([[lambda: call.run(pools)], [lambda: cn.run(pools)], [lambda: cr.run(pools)]], 2,
                            cold=True)
        cold, cold_none, cold_runs = (med([x[0] for x in v]) for v in trio)
        t = dict(cold=cold, cold_none=cold_none, cold_runs=cold_runs, warm=timer.span(lambda: call.run(pools), 3),
                 none=timer.span(lambda: cn.run(pools), 3), runs=timer.span(lambda: cr.run(pools), 3),
                 framed=timer.span(lambda: cf.run(fpools), 3),
                 fp8=timer.span(lambda: c8.run(pools8), 3), fp8f=timer.span(lambda: c8f.run(fpools8), 3),
                 plan_ms=plan_ms)
        if step < 0:
            continue
        if step in (0, n_steps - 1):
            require_finite(torch, f"8B decode step {step}", call.out, cn.out, cf.out, c8.out, c8f.out, cr.out)
        if step % 64 == 63:
            print(f"# 8B decode step {step + 1}/{n_steps}", file=sys.stderr, flush=True)
        for k in acc:
            acc[k] += t[k]
        b = decode_bytes(d, wl)
        for k in tot:
            tot[k] += b[k]
    timer.release()
    n = max(n_steps, 1)
    a = {k: v / n for k, v in acc.items()}
    b = {k: v / n for k, v in tot.items()}
    traffic = read_counter_summary(COUNTERS["decode8b"])
    kv_unique = b["unique"]
    out = {
        "workload": "decode, Llama-3.1-8B shape: 128 requests x 8 Zipf(1.2) documents x 512 tokens "
                    "+ 32-token suffix, steps 0..%d" % (n_steps - 1),
        "splits": splits,
        "us_per_step_cold": round(a["cold"] * 1e3, 2), "us_per_step_warm": round(a["warm"] * 1e3, 2),
        "tokens_per_s_cold": round(128 / (a["cold"] * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(kv_unique / (a["cold"] * 1e-3) / 1e9, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(kv_unique / (a["cold"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "counter_GBps": round(traffic / (a["cold"] * 1e-3) / 1e9, 1) if traffic else None,
                     "bytes_per_launch_unique": round(kv_unique),
                     "bytes_per_launch_logical": round(b["logical"]),
                     "logical_GBps_context": round(b["logical"] / (a["cold"] * 1e-3) / 1e9, 1),
                     "note": "achieved = unique bytes / cold step time"},
        "norotation_us_per_step_cold": round(a["cold_none"] * 1e3, 2),
        "rope_overhead_cold": round(a["cold"] / a["cold_none"] - 1.0, 4),
        "rope_overhead_warm": round(a["warm"] / a["none"] - 1.0, 4),
        "document_frames_us_warm": round(a["framed"] * 1e3, 2),
        "document_frames_overhead_warm": round(a["framed"] / a["none"] - 1.0, 4),
        "fp8_pool_us_warm": round(a["fp8"] * 1e3, 2),
        "fp8_framed_pool_us_warm": round(a["fp8f"] * 1e3, 2),
        "shared_run_decode": {
            "what": "lazyattn_decode_runs: the tables cut into runs shared by several requests, each run read "
                    "once per group of up to 4 requests (G = 4), partials merged per request; the plan is built "
                    "on the host for every step (plan_host_ms, outside the timed region)",
            "us_per_step_cold": round(a["cold_runs"] * 1e3, 2), "us_per_step_warm": round(a["runs"] * 1e3, 2),
            "speedup_vs_per_request_cold": round(a["cold"] / a["cold_runs"], 3),
            "unique_GBps": round(kv_unique / (a["cold_runs"] * 1e-3) / 1e9, 1),
            "frac_of_peak": round(kv_unique / (a["cold_runs"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "plan_host_ms_per_step": round(a["plan_ms"], 2)},
    }
    del pools, fpools, pools8, fpools8
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# extras: the MQA stress mixed step (32 prefills + 96 decodes on two streams)
# ---------------------------------------------------------------------------
def bench_mqa_mixed(torch, W, staging, _abi) -> dict:
    timer = Timer(torch)
    out = {"what": "MQA stress (Hq 32, Hkv 1): 32 prefill requests (128-token queries) and 96 decode requests, "
                   "4..32 lognormal documents each; one mixed step = the prefill call on one stream and the decode "
                   "call on another, started together; times are medians of 3 x 10 warm steps; skew 0.0 = uniform "
                   "access, the no-reuse control"}
    main = torch.cuda.current_stream()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()     # default priority

    def mixed(pc, dc, pools):
        start = torch.cuda.Event()
        start.record(main)
        sa.wait_event(start)
        sb.wait_event(start)
        pc.run(pools, stream=sa)
        dc.run(pools, stream=sb)
        ea, eb = torch.cuda.Event(), torch.cuda.Event()
        ea.record(sa)
        eb.record(sb)
        main.wait_event(ea)
        main.wait_event(eb)

    for skew in W.CFG5_SKEWS:
        wl = W.build_workload(W.spec(5, skew=skew))
        s = wl.spec
        pools = staging.DevicePools(wl, "cuda")
        pb = wl.prefill_batch()
        cfg = staging.config_for(s)
        staging.append_tokens(cfg, pools, pb, s.dtype, "cuda")
        staging.append_tokens(cfg, pools, wl.tokens_before_step(1), s.dtype, "cuda")
        d = wl.decode_step(0)
        flops = prefill_flops(pb, s.head_dim, s.num_q_heads)
        by = decode_bytes(d, wl)
        row = {}
        pes = ("rope", "alibi", "none")
        pcs, dcs = {}, {}
        for pe in pes:
            c = staging.config_for(s, pe=pe)
            pcs[pe] = staging.PrefillCall(c, s, pb, "cuda")
            dcs[pe] = staging.DecodeCall(c, s, d, "cuda")
            pcs[pe].run(pools)
            dcs[pe].run(pools)
            mixed(pcs[pe], dcs[pe], pools)
        # RoPE with the keys turned inside the attention kernel (the library turns them
        # once first for these 16 query tiles per request)
        pc_fused = staging.PrefillCall(staging.config_for(s, keys="fused"), s, pb, "cuda")
        pc_fused.run(pools)
        # the three encodings in alternating order: prefill, decode, mixed step
        tps = timer.span_rounds([lambda pc=pcs[pe]: pc.run(pools) for pe in pes] + [lambda: pc_fused.run(pools)], 10)
        tds = timer.span_rounds([lambda dc=dcs[pe]: dc.run(pools) for pe in pes], 10)
        tms = timer.span_rounds([lambda pe=pe: mixed(pcs[pe], dcs[pe], pools) for pe in pes], 10)
        for v, pe in enumerate(pes):
            tp, td, tm = tps[v], tds[v], tms[v]
            require_finite(torch, f"MQA stress skew {skew} ({pe})", pcs[pe].out, dcs[pe].out)
            row[pe] = {"prefill_us": round(tp * 1e3, 2), "prefill_TFLOPs": round(flops / (tp * 1e-3) / 1e12, 1),
                       "decode_us": round(td * 1e3, 2),
                       "decode_GBps_unique": round(by["unique"] / (td * 1e-3) / 1e9, 1),
                       "decode_GBps_logical": round(by["logical"] / (td * 1e-3) / 1e9, 1),
                       "mixed_step_us": round(tm * 1e3, 2),
                       "overlap_gain": round((tp + td) / tm, 3)}
        row["prefill_rope_overhead"] = round(row["rope"]["prefill_us"] / row["none"]["prefill_us"] - 1.0, 4)
        require_finite(torch, f"MQA stress skew {skew} (rope, keys in the kernel)", pc_fused.out)
        row["prefill_rope_keys_in_kernel_us"] = round(tps[len(pes)] * 1e3, 2)
        row["prefill_rope_keys_in_kernel_overhead"] = round(tps[len(pes)] / tps[pes.index("none")] - 1.0, 4)
        row["decode_rope_overhead"] = round(row["rope"]["decode_us"] / row["none"]["decode_us"] - 1.0, 4)
        row["mixed_rope_overhead"] = round(row["rope"]["mixed_step_us"] / row["none"]["mixed_step_us"] - 1.0, 4)
        row["decode_GB_unique"] = round(by["unique"] / 1e9, 4)
        row["decode_GB_logical"] = round(by["logical"] / 1e9, 4)
        cb = read_mqa_decode_counters(COUNTERS["mqa"]).get(f"{skew:.1f}")
        # FETCH + WRITE per step (the committed rocprofv3 summary) over this run's step time
        row["decode_counter_GB"] = round(cb / 1e9, 4) if cb else None
        row["decode_counter_GBps"] = round(cb / (row["rope"]["decode_us"] * 1e-6) / 1e9, 1) if cb else None
        row["prefill_GFLOP"] = round(flops / 1e9, 1)
        out[f"skew{skew}"] = row
        del pools, pc_fused
        torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# measured peaks, pool hit ratios, CPU baseline
# ---------------------------------------------------------------------------
def bench_tp8_share(torch, W, staging, _abi, n_decode: int = 8) -> dict:
    """One GPU's share of the Llama-3.1-70B layer under 8-way tensor parallelism over KV heads
    (Hq 8, Hkv 1, G 8) at the same 32k contexts: the 2048-token chunk and the first decode steps,
    every step cold.  No exchange is needed between the shares."""
    import dataclasses
    sp = dataclasses.replace(W.spec(4, n_decode=n_decode), num_q_heads=8, num_kv_heads=1,
                             name="llama70b-32k-tp8-share")
    wl = W.build_workload(sp)
    s = wl.spec
    pools = staging.DevicePools(wl, "cuda")
    pb = wl.prefill_batch()
    cfg = staging.config_for(s)
    staging.append_tokens(cfg, pools, pb, s.dtype, "cuda")
    call = staging.PrefillCall(cfg, s, pb, "cuda")
    timer = Timer(torch)
    for _ in range(2):
        call.run(pools)
    st = timer.steps([lambda: call.attend(pools)] + ([call.merge] if call.splits > 1 else []), 10, cold=True)
    require_finite(torch, "TP-8 share prefill", call.out)
    flops = prefill_flops(pb, s.head_dim, s.num_q_heads)
    att, step = med([x[0] for x in st]), med([sum(x) for x in st])
    allt = wl.tokens_before_step(n_decode)
    staging.append_tokens(cfg, pools, allt, s.dtype, "cuda")
    steps = [wl.decode_step(i) for i in range(n_decode)]
    calls = [staging.DecodeCall(cfg, s, d, "cuda") for d in steps]
    by = [decode_bytes(d, wl) for d in steps]
    for c in calls[:2]:
        c.run(pools)
    cold = timer.steps([lambda i: calls[i].attend(pools), lambda i: calls[i].merge()], n_decode, cold=True, arg=True)
    require_finite(torch, "TP-8 share decode", *[c.out for c in calls])
    d_att = sum(x[0] for x in cold) / n_decode
    d_mrg = sum(x[1] for x in cold) / n_decode
    uniq = sum(b["unique"] for b in by) / n_decode
    timer.release()
    out = {
        "workload": "one GPU's share of the Llama-3.1-70B layer under 8-way tensor parallelism over KV heads: "
                    "Hq 8, Hkv 1, the same 4 x 32k contexts, 2048-token chunk, then decode steps "
                    f"0..{n_decode - 1}; cold",
        "prefill": {"attention_us_cold": round(att * 1e3, 2), "step_us_cold": round(step * 1e3, 2),
                    "key_splits": call.splits, "TFLOPs_attention": round(flops / (att * 1e-3) / 1e12, 2),
                    "frac_of_peak": round(flops / (att * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "decode": {"us_per_step_cold": round((d_att + d_mrg) * 1e3, 2),
                   "attention_us_cold": round(d_att * 1e3, 2), "merge_us_cold": round(d_mrg * 1e3, 2),
                   "splits": calls[0].splits, "GBps_unique": round(uniq / (d_att * 1e-3) / 1e9, 1),
                   "frac_of_peak": round(uniq / (d_att * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
    }
    del calls, call, pools
    torch.cuda.empty_cache()
    return out


def measured_peaks(torch) -> dict:
    out = {}
    L = probe_lib()
    stream = torch.cuda.current_stream().cuda_stream
    timer = Timer(torch)
    nwg, iters = 4096, 2000
    sink = torch.empty(nwg * 256, dtype=torch.float32, device="cuda")

    def mfma():
        assert L.lazyattn_probe_mfma_bf16(nwg, iters, sink.data_ptr(), stream) == 0

    mfma()
    ms = med([timer.span(mfma, 3) for _ in range(3)])
    out["mfma_bf16_TFLOPs"] = round(nwg * 4 * iters * 8 * 32768 / (ms * 1e-3) / 1e12, 1)
    n16 = (4 << 30) // 16
    buf = torch.ones(n16 * 4, dtype=torch.int32, device="cuda")
    rwg = 256 * 32

    sink2 = torch.empty(rwg * 256, dtype=torch.float32, device="cuda")

    def rd():
        assert L.lazyattn_probe_hbm_read(buf.data_ptr(), n16, rwg, sink2.data_ptr(), stream) == 0

    rd()
    ms = med([timer.span(rd, 3) for _ in range(3)])
    out["hbm_read_GBps"] = round(n16 * 16 / (ms * 1e-3) / 1e9, 1)
    del buf, sink, sink2
    out["device_copy_GBps"] = round(copy_bandwidth(torch), 1)
    out["what"] = ("mfma: 4096 work-groups of 4 waves, 8 independent 32x32x16 bf16 MFMA chains each; hbm: "
                   "grid-stride read of 4 GiB; copy: torch 1 GiB device copy (read + write bytes)")
    torch.cuda.empty_cache()
    return out


def copy_bandwidth(torch) -> float:
    """GB/s of a plain 1 GiB device-to-device copy (2 GiB moved), median of 5."""
    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    ts = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del a, b
    return 2.0 * n / (sorted(ts)[2] * 1e-3) / 1e9


def hit_ratio_study(W, _abi) -> dict:
    """Document cache hit ratios of the native pool manager under three cache keys (host only).

    Trace: 4000 requests x 8 distinct documents of 512 tokens, Zipf over a pool of 2000 documents.
    Budgets are KV bytes of a whole Llama-3.1-8B model (32 layers x 8 KV heads x 128 x K,V x bf16
    = 128 KiB per token): 1 GiB (8192 tokens) and 8 GiB.
    """
    per_token = 32 * 8 * 128 * 2 * 2
    out = {"trace": "4000 requests x 8 Zipf documents x 512 tokens, pool of 2000 documents",
           "kv_bytes_per_token": per_token, "token_hit_ratio": {}}
    t_run, n_admits = 0.0, 0
    for skew in (0.8, 1.2):
        ids, lens, offs = W.cache_trace(2000, 4000, (8, 8), skew, seed=11)
        for gib in (1, 8):
            blocks = (gib << 30) // (per_token * 16)
            row = {}
            for pol in ("agnostic", "aware", "prefix"):
                pool = _abi.Pool(blocks, pol)
                t0 = time.perf_counter()
                pool.run_trace(ids, lens, offs)
                t_run += time.perf_counter() - t0
                n_admits += offs.size - 1
                st = pool.stats()
                row[pol] = round(st["token_hits"] / st["token_accesses"], 5)
                pool.close()
            row["agnostic_over_aware"] = round(row["agnostic"] / max(row["aware"], 1e-12), 2)
            row["agnostic_over_prefix"] = round(row["agnostic"] / max(row["prefix"], 1e-12), 2)
            out["token_hit_ratio"][f"zipf{skew}_{gib}GiB"] = row
    out["requests_per_s"] = round(n_admits / t_run, 1)
    return out


def cpu_baseline(h):
    """The fp64 oracle on a sample of the headline workload, on the host's BLAS threads:
    the first 256 chunk rows of requests 0, 1, ... (all 64 heads, each over its whole 32k
    context) until about 12 s have been spent, then whole decode steps (all 4 requests) until
    about 6 s more."""
    import numpy as np  # noqa: F401
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    wl, pb = h["wl"], h["pb"]
    s = wl.spec
    kp, vp = wl.pools()
    kp, vp = kp.copy(), vp.copy()
    O.append_kv(kp, vp, pb["k_new"], pb["v_new"], pb["slots"], s.block_size)
    words = O.pack_table(pb["table_blocks"], pb["table_starts"])
    t_pre, flops, done = 0.0, 0.0, []
    for r in range(len(pb["ctx_lens"])):
        rows = {r: list(range(256))}
        t0 = time.perf_counter()
        O.prefill(q=pb["q"], cu_q_lens=pb["cu_q_lens"], ctx_lens=pb["ctx_lens"], num_entries=pb["num_entries"],
                  table_words=words, k_pool=kp, v_pool=vp, num_kv_heads=s.num_kv_heads, block_size=s.block_size,
                  dtype=s.dtype, pe=s.pe, rope_theta=s.rope_theta, requests=[r], token_subset=rows)
        t_pre += time.perf_counter() - t0
        flops += prefill_flops(pb, s.head_dim, s.num_q_heads, token_subset=rows)
        done.append(r)
        if t_pre >= 12.0:
            break
    t_dec, n_dec, dec_bytes = 0.0, 0, 0
    for i, d in enumerate(h["steps"]):
        O.append_kv(kp, vp, d["k_new"], d["v_new"], d["slots"], s.block_size)
        t0 = time.perf_counter()
        O.decode(q=d["q"], ctx_lens=d["ctx_lens"], num_entries=d["num_entries"],
                 table_words=O.pack_table(d["table_blocks"], d["table_starts"]), k_pool=kp, v_pool=vp,
                 num_kv_heads=s.num_kv_heads, block_size=s.block_size, dtype=s.dtype, pe=s.pe,
                 rope_theta=s.rope_theta)
        t_dec += time.perf_counter() - t0
        n_dec += 1
        dec_bytes += h["bytes"][i]["unique"]
        if t_dec >= 6.0:
            break
    return {"value": round(flops / t_pre / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(t_pre, 3), "sample_flops": flops,
            "decode_step_s": round(t_dec / n_dec, 3), "decode_steps_timed": n_dec,
            "decode_GBps_unique": round(dec_bytes / t_dec / 1e9, 3),
            "sample": f"headline workload (Llama-3.1-70B 32k chunk): the first 256 chunk rows of requests {done}, "
                      "all 64 heads over each one's 32.8k-token context (the whole context gathered and rotated "
                      f"per call), then decode steps 0..{n_dec - 1} of all 4 requests; materialised-RoPE fp64 "
                      "numpy oracle, one call per request or step"}


def calibrate_copy(torch) -> None:
    """A plain device copy of 1 GiB (read 1 GiB, write 1 GiB) for counter scaling."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "dispatches": 3}), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=128, help="decode steps after the headline chunk")
    ap.add_argument("--decode8b-steps", type=int, default=256)
    ap.add_argument("--no-extras", action="store_true", help="headline only (8B and MQA extras, peaks skipped)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["llama8b", "mqa", "peaks", "tp8"], help="run one extra alone (profiling)")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--summarize-rocprof", metavar="DIR")
    args = ap.parse_args()

    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE {world}) is not supported: "
              "this path runs on a single MI355X and has no multi-GPU leg", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        calibrate_copy(torch)
        return 0

    import workloads as W
    from position_agnostic_kv_pool_amd import _abi, staging
    _abi.lib()

    if args.only:
        if args.only == "llama8b":
            res = {"llama8b_prefill": bench_llama8b_prefill(torch, args, W, staging, _abi),
                   "llama8b_decode": bench_llama8b_decode(torch, args, W, staging, _abi, args.decode8b_steps)}
        elif args.only == "mqa":
            res = {"mqa_mixed": bench_mqa_mixed(torch, W, staging, _abi)}
        elif args.only == "tp8":
            res = {"llama70b_tp8_share": bench_tp8_share(torch, W, staging, _abi)}
        else:
            res = {"measured_peaks": measured_peaks(torch)}
        print(json.dumps(res), flush=True)
        return 0

    h = bench_headline(torch, args, W, staging, _abi)
    out = headline_json(h, args)
    if not args.no_extras:
        pk = measured_peaks(torch)
        pk["prefill_frac_of_measured_mfma"] = round(out["roofline"]["achieved"] / pk["mfma_bf16_TFLOPs"], 4)
        pk["decode_frac_of_measured_hbm_read"] = round(out["decode"]["roofline"]["achieved"] / pk["hbm_read_GBps"], 4)
        out["measured_peaks"] = pk
        print("# peaks done", file=sys.stderr, flush=True)
        out["llama8b_prefill"] = bench_llama8b_prefill(torch, args, W, staging, _abi)
        print("# 8B prefill done", file=sys.stderr, flush=True)
        out["llama8b_decode"] = bench_llama8b_decode(torch, args, W, staging, _abi, args.decode8b_steps)
        print("# 8B decode done", file=sys.stderr, flush=True)
        out["mqa_mixed"] = bench_mqa_mixed(torch, W, staging, _abi)
        print("# MQA mixed done", file=sys.stderr, flush=True)
        out["llama70b_tp8_share"] = bench_tp8_share(torch, W, staging, _abi)
        print("# 70B TP-8 share done", file=sys.stderr, flush=True)
        out["pool_hit_ratio"] = hit_ratio_study(W, _abi)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(h)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
