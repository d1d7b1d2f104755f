#!/usr/bin/env python3
"""Benchmark of deferred-RoPE attention over a position-agnostic paged KV pool on one MI355X.

Workload (one step = one prefill launch over the whole batch): the
Llama-3.1-8B attention-layer shape in bf16 (32 query heads, 8 KV heads,
head_dim 128, RoPE theta 5e5, blocks of 16 tokens); 16 requests, each 8
distinct documents of 512 tokens drawn Zipf(1.0) from a pool of 256
documents and placed in random order (4096 context tokens), followed by a
64-token query prefilled causally.  Inputs are seeded synthetic data already
resident in HBM.  The new tokens' K/V are appended once before timing.

Also reported on the same line: the same launch with rotation disabled
(deferred-RoPE overhead), decode on the Llama-3.1-8B decode shape (128
requests x 8 Zipf(1.2) documents, per-step HBM bytes), and the fp64 CPU
oracle on the same prefill batch.

  python bench.py [--gpus 1] [--steps K] [--warmup W]
  python bench.py --calibrate-copy           # a plain copy kernel, for counter scaling
  python bench.py --summarize-rocprof DIR    # print a rocprofv3 CSV directory as a summary
"""
from __future__ import annotations

import argparse
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
KERNEL_SRC = os.path.join(ROOT, "position_agnostic_kv_pool_amd", "csrc", "lazyattn_kernels.hip")
PREFILL_COUNTERS = os.path.join(ROOT, "profiles", "prefill_bf16_llama8b_counters.txt")
DECODE_COUNTERS = os.path.join(ROOT, "profiles", "decode_bf16_llama8b_counters.txt")


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_counter_summary(path: str):
    """(bytes per dispatch from FETCH_SIZE + WRITE_SIZE scaled by the copy calibration) if the
    summary was taken on the current kernel source, else None."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
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
# workloads
# ---------------------------------------------------------------------------
def prefill_flops(pb, head_dim: int, num_q_heads: int) -> float:
    """4 * D * Hq * sum over queries of the keys each one sees (QK^T and PV, causal)."""
    tot = 0
    cu = pb["cu_q_lens"]
    for r, L in enumerate(pb["ctx_lens"]):
        m = int(cu[r + 1] - cu[r])
        p0 = int(L) - m
        tot += m * p0 + m * (m + 1) // 2        # sum_{j<m} (p0 + j + 1)
    return 4.0 * head_dim * num_q_heads * tot


def decode_bytes(d, wl) -> dict:
    """Per-step bytes: logical (what a per-request paged kernel streams), unique (each
    (block, KV head) once), plus queries, outputs and table words."""
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


class Timer:
    """HIP events on the stream the kernels are launched on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch

    def busy(self):
        # keep the GPU busy while the host enqueues the timed launches, so host
        # launch latency never shows up between the events
        if hasattr(self.torch.cuda, "_sleep"):
            self.torch.cuda._sleep(2_000_000)

    def span(self, fn, n):
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

    def launches(self, fn, n):
        """Per-launch times (ms) of n back-to-back launches, each bracketed by its own events."""
        t = self.torch
        ev = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)) for _ in range(n)]
        t.cuda.synchronize()
        self.busy()
        for a, b in ev:
            a.record()
            fn()
            b.record()
        t.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ev)

    def steps(self, attend, merge, n):
        """n steps of [attention kernel, merge kernel]: (ms per step, ms per attention launch)."""
        t = self.torch
        ev = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)) for _ in range(n)]
        end = t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        self.busy()
        for a, b in ev:
            a.record()
            attend()
            b.record()
            merge()
        end.record()
        t.cuda.synchronize()
        return ev[0][0].elapsed_time(end) / n, sum(a.elapsed_time(b) for a, b in ev) / n


def bench_prefill(torch, args, W, staging, _abi):
    wl = W.build_workload(W.spec(2))
    s = wl.spec
    pools = staging.DevicePools(wl, "cuda")
    pb = wl.prefill_batch()
    cfg = staging.config_for(s)
    staging.append_tokens(cfg, pools, pb, s.dtype, "cuda")
    call = staging.PrefillCall(cfg, s, pb, "cuda")
    cfg_none = staging.config_for(s, pe="none")
    call_none = staging.PrefillCall(cfg_none, s, pb, "cuda")
    # the same batch over a pool in document-local frames
    fpools = staging.FramedPools(wl, cfg, "cuda")
    staging.append_tokens(cfg, fpools, pb, s.dtype, "cuda")
    call_framed = staging.PrefillCall(cfg, s, pb, "cuda", framed=True)
    # and over an FP8 pool
    cfg8 = staging.config_for(s, kv_format="fp8")
    pools8 = staging.WrittenPools(wl, cfg8, "cuda")
    staging.append_tokens(cfg8, pools8, pb, s.dtype, "cuda")
    call8 = staging.PrefillCall(cfg8, s, pb, "cuda")
    torch.cuda.synchronize()
    timer = Timer(torch)
    for _ in range(args.warmup):
        call.run(pools)
    # clocks and caches settle over ~20 ms of untimed launches before anything is timed
    timer.span(lambda: call.attend(pools), 200)
    # the timed steps: exactly args.steps steps (attention kernel, then the split merge),
    # back-to-back between two events
    ms = timer.span(lambda: call.run(pools), args.steps)
    # the attention kernel alone and its rotation-free control, three interleaved rounds (medians)
    att, att_none, step_none, att_framed, att_fp8 = [], [], [], [], []
    call_framed.run(fpools)
    call8.run(pools8)
    for _ in range(3):
        att.append(timer.span(lambda: call.attend(pools), args.steps))
        att_none.append(timer.span(lambda: call_none.attend(pools), args.steps))
        step_none.append(timer.span(lambda: call_none.run(pools), args.steps))
        att_framed.append(timer.span(lambda: call_framed.attend(fpools), args.steps))
        att_fp8.append(timer.span(lambda: call8.attend(pools8), args.steps))
    del fpools, pools8
    # cold: the last-level cache flushed by a 512 MB write before each single launch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold, cold_none = [], []
    for rep in range(5):
        for fn, acc in ((call.attend, cold), (call_none.attend, cold_none)):
            flush.fill_(rep & 0xff)
            acc.append(timer.span(lambda: fn(pools), 1))
    del flush
    med = lambda v: sorted(v)[len(v) // 2]
    # distribution of single attention launches (50, each between its own events)
    per = timer.launches(lambda: call.attend(pools), 50)
    pct = {"p10": per[len(per) // 10], "p50": per[len(per) // 2], "p90": per[(9 * len(per)) // 10]}
    # materialise-then-attend baseline on the same batch: private rotated copies of every
    # request's blocks, rotated queries, then the rotation-free kernel over the copy
    mat = staging.MaterializedPrefill(s, pb, "cuda")
    mat.run(pools)
    base = dict(materialize=timer.span(lambda: mat.materialize(pools), args.steps),
                rotate_queries=timer.span(lambda: mat.rotate_queries(), args.steps),
                attention=timer.span(lambda: mat.attend(), args.steps),
                total=timer.span(lambda: mat.run(pools), args.steps), copied_bytes=mat.bytes_copied)
    del mat
    flops = prefill_flops(pb, s.head_dim, s.num_q_heads)
    return dict(wl=wl, pb=pb, ms=ms, ms_attend=med(att), ms_none=med(step_none), ms_none_attend=med(att_none),
                att=att, att_none=att_none, att_framed=att_framed, ms_framed_attend=med(att_framed),
                ms_fp8_attend=med(att_fp8), pct=pct, cold=med(cold), cold_none=med(cold_none), flops=flops, base=base,
                splits=call.splits, pools=pools)


def bench_decode(torch, args, W, staging, _abi, n_steps: int, framed: bool = True):
    """Decode steps 0..n_steps-1 of the 8B decode shape.  Each step's new token is appended
    untimed; then 3 back-to-back launches of its attention kernel are timed (they re-read the same
    step's pool, as the step itself would), with and without the merge, and rotation-free."""
    wl = W.build_workload(W.spec(3, n_decode=max(n_steps, 1)))
    s = wl.spec
    cfg = staging.config_for(s)
    cfg_none = staging.config_for(s, pe="none")
    pools = staging.DevicePools(wl, "cuda")
    staging.append_tokens(cfg, pools, wl.tokens_before_step(0), s.dtype, "cuda")
    fpools = staging.FramedPools(wl, cfg, "cuda") if framed else None
    if framed:
        staging.append_tokens(cfg, fpools, wl.tokens_before_step(0), s.dtype, "cuda")
    # the same steps over an FP8 pool (quantised by the library's append)
    cfg8 = staging.config_for(s, kv_format="fp8")
    pools8 = staging.WrittenPools(wl, cfg8, "cuda") if framed else None
    fpools8 = staging.FramedPools(wl, cfg8, "cuda") if framed else None
    if framed:
        staging.append_tokens(cfg8, pools8, wl.tokens_before_step(0), s.dtype, "cuda")
        staging.append_tokens(cfg8, fpools8, wl.tokens_before_step(0), s.dtype, "cuda")
    t = torch
    tot_ms, tot_merge_ms, tot_ms_none, tot_bytes, tot_unique, tokens = 0.0, 0.0, 0.0, 0, 0, 0
    tot_kv = 0
    tot_ms_framed, tot_ms_fp8, tot_ms_fp8f = 0.0, 0.0, 0.0
    for step in range(-2, n_steps):          # two untimed warm-up launches on step 0's inputs
        d = wl.decode_step(max(step, 0))
        if step >= 0:
            staging.append_tokens(cfg, pools, d, s.dtype, "cuda")
            if framed:
                staging.append_tokens(cfg, fpools, d, s.dtype, "cuda")
                staging.append_tokens(cfg8, pools8, d, s.dtype, "cuda")
                staging.append_tokens(cfg8, fpools8, d, s.dtype, "cuda")
        call = staging.DecodeCall(cfg, s, d, "cuda")
        call_none = staging.DecodeCall(cfg_none, s, d, "cuda")
        timer = Timer(t)
        ms_att = timer.span(lambda: call.attend(pools), 3)
        ms_step = timer.span(lambda: call.run(pools), 3)
        ms_none = timer.span(lambda: call_none.attend(pools), 3)
        ms_framed, ms_fp8, ms_fp8f = 0.0, 0.0, 0.0
        if framed:
            call_framed = staging.DecodeCall(cfg, s, d, "cuda", framed=True)
            ms_framed = timer.span(lambda: call_framed.attend(fpools), 3)
            call8 = staging.DecodeCall(cfg8, s, d, "cuda")
            ms_fp8 = timer.span(lambda: call8.attend(pools8), 3)
            call8f = staging.DecodeCall(cfg8, s, d, "cuda", framed=True)
            ms_fp8f = timer.span(lambda: call8f.attend(fpools8), 3)
        if step < 0:
            continue
        if step % 64 == 63:
            print(f"# decode step {step + 1}/{n_steps}", file=sys.stderr, flush=True)
        tot_ms += ms_att
        # with one split the step is the attention kernel alone (no merge is launched)
        if call.splits > 1:
            tot_merge_ms += max(ms_step - ms_att, 0.0)
        tot_ms_none += ms_none
        tot_ms_framed += ms_framed
        tot_ms_fp8 += ms_fp8
        tot_ms_fp8f += ms_fp8f
        by = decode_bytes(d, wl)
        tot_bytes += by["logical"]
        tot_kv += by["kv_logical"]
        tot_unique += by["unique"]
        tokens += len(d["ctx_lens"])
    n = max(n_steps, 1)
    return dict(ms=tot_ms / n, merge_ms=tot_merge_ms / n, ms_none=tot_ms_none / n, ms_framed=tot_ms_framed / n,
                ms_fp8=tot_ms_fp8 / n, ms_fp8f=tot_ms_fp8f / n, bytes=tot_bytes / n, kv_bytes=tot_kv / n,
                unique=tot_unique / n,
                tokens=tokens, splits=_abi.decode_splits(cfg, len(wl.requests), wl.table_arrays(wl.requests)[0].shape[1]))


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


def bench_configs(torch, W, staging, _abi) -> dict:
    """The other configurations, warm (medians of three 10-launch spans), each with its
    rotation-free control on the same inputs: the Llama-3.1-70B 32k shape (a 2048-token chunk of
    each of 4 requests, and a decode step with split-K) and the MQA stress sweep (four access skews,
    uniform = the no-reuse control, each under RoPE, ALiBi and no encoding)."""
    timer = Timer(torch)
    med = lambda v: sorted(v)[len(v) // 2]
    span = lambda fn: med([timer.span(fn, 10) for _ in range(3)])
    out = {}

    def one(wl, encodings):
        s = wl.spec
        pools = staging.DevicePools(wl, "cuda")
        pb = wl.prefill_batch()
        cfg = staging.config_for(s)
        res = {}
        if pb is not None:
            staging.append_tokens(cfg, pools, pb, s.dtype, "cuda")
            flops = prefill_flops(pb, s.head_dim, s.num_q_heads)
            for pe in encodings:
                c = staging.PrefillCall(staging.config_for(s, pe=pe), s, pb, "cuda")
                c.run(pools)
                ms = span(lambda: c.run(pools))
                res[f"prefill_{pe}_us"] = round(ms * 1e3, 2)
                res[f"prefill_{pe}_TFLOPs"] = round(flops / (ms * 1e-3) / 1e12, 2)
        staging.append_tokens(cfg, pools, wl.tokens_before_step(0), s.dtype, "cuda")
        d = wl.decode_step(0)
        if d is not None:
            staging.append_tokens(cfg, pools, d, s.dtype, "cuda")
            by = decode_bytes(d, wl)
            for pe in encodings:
                c = staging.DecodeCall(staging.config_for(s, pe=pe), s, d, "cuda")
                c.run(pools)
                ms = span(lambda: c.run(pools))
                res[f"decode_{pe}_us"] = round(ms * 1e3, 2)
                res[f"decode_{pe}_GBps_logical"] = round(by["logical"] / (ms * 1e-3) / 1e9, 1)
            res["decode_GB_logical"] = round(by["logical"] / 1e9, 4)
            res["decode_GB_unique"] = round(by["unique"] / 1e9, 4)
        for ph in ("prefill", "decode"):
            if f"{ph}_rope_us" in res and f"{ph}_none_us" in res:
                res[f"{ph}_rope_overhead"] = round(res[f"{ph}_rope_us"] / res[f"{ph}_none_us"] - 1.0, 4)
        del pools
        torch.cuda.empty_cache()
        return res

    wl = W.build_workload(W.spec(4, n_decode=1))
    out["llama70b_32k"] = dict(what="4 requests x 64 Zipf(1.0) documents x 512 tokens; 2048-token chunk; "
                                    "decode step 0 with the split-K heuristic", **one(wl, ("rope", "none")))
    print("# 70B config done", file=sys.stderr, flush=True)
    for skew in W.CFG5_SKEWS:
        wl = W.build_workload(W.spec(5, skew=skew))
        out[f"mqa_skew{skew}"] = one(wl, ("rope", "alibi", "none"))
    out["mqa_what"] = ("MQA stress: 32 prefill requests (128-token queries) + 96 decode requests, 4..32 lognormal "
                       "documents each; skew 0.0 = uniform access, the no-reuse control")
    return out


def cpu_baseline(pre, W):
    """The fp64 oracle on the same prefill batch (all 16 requests), host cores."""
    import numpy as np  # noqa: F401
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    wl, pb = pre["wl"], pre["pb"]
    s = wl.spec
    kp, vp = wl.pools()
    kp, vp = kp.copy(), vp.copy()
    O.append_kv(kp, vp, pb["k_new"], pb["v_new"], pb["slots"], s.block_size)
    words = O.pack_table(pb["table_blocks"], pb["table_starts"])
    # repeat whole calls until about 10 s of CPU work have been timed
    calls, t0 = 0, time.perf_counter()
    while True:
        O.prefill(q=pb["q"], cu_q_lens=pb["cu_q_lens"], ctx_lens=pb["ctx_lens"], num_entries=pb["num_entries"],
                  table_words=words, k_pool=kp, v_pool=vp, num_kv_heads=s.num_kv_heads, block_size=s.block_size,
                  dtype=s.dtype, pe=s.pe, rope_theta=s.rope_theta)
        calls += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or calls >= 30:
            break
    return {"value": round(calls * pre["flops"] / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(dt, 3), "calls": calls,
            "sample": "the whole timed prefill batch (16 requests x 64 queries over ~4.2k tokens), "
                      "materialised-RoPE fp64 numpy oracle, whole calls repeated for about 10 s"}


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


def copy_bandwidth(torch) -> float:
    """GB/s of a plain 1 GiB device-to-device copy (2 GiB moved), median of 5: the
    HBM bandwidth this GPU reaches with a library kernel, as context for the others."""
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
    torch.cuda.empty_cache()
    return 2.0 * n / (sorted(ts)[2] * 1e-3) / 1e9


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--no-configs", action="store_true", help="skip the 70B and MQA configuration timings")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true", help="time the prefill launches only")
    ap.add_argument("--decode-only", action="store_true", help="run decode launches only (for profiling)")
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

    if args.decode_only:
        dec = bench_decode(torch, args, W, staging, _abi, args.decode_steps, framed=False)
        print(json.dumps({"decode_ms_per_step": dec["ms"], "decode_GBps": dec["bytes"] / dec["ms"] / 1e6}),
              flush=True)
        return 0

    pre = bench_prefill(torch, args, W, staging, _abi)
    print(f"# prefill done: {pre['ms'] * 1e3:.1f} us/step, attention kernel {pre['ms_attend'] * 1e3:.1f} us",
          file=sys.stderr, flush=True)
    tflops = pre["flops"] / (pre["ms"] * 1e-3) / 1e12
    kernel_tflops = pre["flops"] / (pre["ms_attend"] * 1e-3) / 1e12
    traffic = read_counter_summary(PREFILL_COUNTERS)
    roofline = {"bound": "mfma", "achieved": round(kernel_tflops, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(kernel_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": "prefill_bf16_kernel<ROPE>", "flops_per_launch": pre["flops"],
                "avg_launch_us": round(pre["ms_attend"] * 1e3, 2),
                "launch_us_p10_p50_p90": [round(pre["pct"][k] * 1e3, 2) for k in ("p10", "p50", "p90")],
                "cold_launch_us": round(pre["cold"] * 1e3, 2),
                "merge_kernel_us": round((pre["ms"] - pre["ms_attend"]) * 1e3, 2)}
    rope_overhead = {"prefill_rope_us": round(pre["ms_attend"] * 1e3, 2),
                     "prefill_rope_rounds_us": [round(x * 1e3, 2) for x in pre["att"]],
                     "prefill_norotation_us": round(pre["ms_none_attend"] * 1e3, 2),
                     "prefill_norotation_rounds_us": [round(x * 1e3, 2) for x in pre["att_none"]],
                     "prefill_overhead": round(pre["ms_attend"] / pre["ms_none_attend"] - 1.0, 4),
                     # rotation work: 3 flops per rotated key element, each key tile rotated once per
                     # work-group of 256 query rows (the pages' 3/(4M) cost model with M = 256)
                     "prefill_rotation_flop_fraction": round(3.0 / (4.0 * 256), 5),
                     "prefill_cold_rope_us": round(pre["cold"] * 1e3, 2),
                     "prefill_cold_norotation_us": round(pre["cold_none"] * 1e3, 2)}
    out = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(pre["ms"], 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill, Llama-3.1-8B attention layer (Hq 32, Hkv 8, d 128, RoPE theta 5e5, "
                               "block 16): 16 requests x 8 Zipf(1.0) documents x 512 tokens + 64-token causal "
                               "query; content-only pool, RoPE applied in-kernel",
                   "global_batch": 16, "seq_len": int(max(pre["pb"]["ctx_lens"])), "parallelism": "single-gpu",
                   "key_splits": pre["splits"]},
        "roofline": roofline,
        "rope_overhead": rope_overhead,
        "materialize_baseline": {
            "what": "private copies of every request's blocks with K rotated at absolute positions, queries "
                    "rotated, then the rotation-free kernel over the copy (the approach deferred RoPE replaces)",
            "materialize_us": round(pre["base"]["materialize"] * 1e3, 2),
            "rotate_queries_us": round(pre["base"]["rotate_queries"] * 1e3, 2),
            "attention_us": round(pre["base"]["attention"] * 1e3, 2),
            "total_us": round(pre["base"]["total"] * 1e3, 2),
            "copied_bytes": int(pre["base"]["copied_bytes"]),
            "deferred_step_us": round(pre["ms"] * 1e3, 2),
            "deferred_speedup": round(pre["base"]["total"] / pre["ms"], 3)},
        "fp8_pool_prefill": {
            "what": "the prefill over an e4m3 pool with per-row power-of-two scales, converted to bf16 in staging",
            "attention_us": round(pre["ms_fp8_attend"] * 1e3, 2),
            "vs_bf16_pool": round(pre["ms_attend"] / pre["ms_fp8_attend"], 3)},
        "document_frames": {
            "what": "the same attention over a pool whose keys carry their index inside their document "
                    "(stored R(j) k): prefill turns each key entry once by R(F - p0), decode turns the query "
                    "once per document",
            "prefill_attention_us": round(pre["ms_framed_attend"] * 1e3, 2),
            "prefill_rounds_us": [round(x * 1e3, 2) for x in pre["att_framed"]],
            "prefill_overhead_vs_norotation": round(pre["ms_framed_attend"] / pre["ms_none_attend"] - 1.0, 4)},
    }
    if not args.prefill_only:
        del pre["pools"]
        torch.cuda.empty_cache()
        dec = bench_decode(torch, args, W, staging, _abi, args.decode_steps)
        gbs = dec["bytes"] / (dec["ms"] * 1e-3) / 1e9
        dtraffic = read_counter_summary(DECODE_COUNTERS)
        out["decode"] = {
            "workload": "decode, Llama-3.1-8B shape: 128 requests x 8 Zipf(1.2) documents x 512 tokens "
                        "+ 32-token suffix, steps 0..%d" % (args.decode_steps - 1),
            "value": round(gbs, 1), "unit": "GB/s", "us_per_step": round((dec["ms"] + dec["merge_ms"]) * 1e3, 2),
            "attention_kernel_us": round(dec["ms"] * 1e3, 2), "merge_kernel_us": round(dec["merge_ms"] * 1e3, 2),
            "tokens_per_s": round(128 / ((dec["ms"] + dec["merge_ms"]) * 1e-3), 1), "splits": dec["splits"],
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": dtraffic,
                         "kernel": "decode_bf16_kernel<ROPE,1>", "bytes_per_launch_logical": round(dec["bytes"]),
                         "bytes_per_launch_unique": round(dec["unique"])},
            "norotation_us_per_step": round(dec["ms_none"] * 1e3, 2),
            "rope_overhead": round(dec["ms"] / dec["ms_none"] - 1.0, 4),
        }
        fp8_bytes = dec["bytes"] - dec["kv_bytes"] + dec["kv_bytes"] * 2064 / 4096
        out["decode"]["fp8_pool"] = {
            "what": "the same decode steps over an e4m3 pool with per-row power-of-two scales "
                    "(2064-byte chunks per block and KV head instead of 4096)",
            "attention_kernel_us": round(dec["ms_fp8"] * 1e3, 2),
            "bytes_per_launch_logical": round(fp8_bytes),
            "GBps": round(fp8_bytes / (dec["ms_fp8"] * 1e-3) / 1e9, 1),
            "speedup_vs_bf16_pool": round(dec["ms"] / dec["ms_fp8"], 3),
            "framed_attention_kernel_us": round(dec["ms_fp8f"] * 1e3, 2)}
        out["document_frames"]["decode_attention_us"] = round(dec["ms_framed"] * 1e3, 2)
        out["document_frames"]["decode_overhead_vs_norotation"] = round(dec["ms_framed"] / dec["ms_none"] - 1.0, 4)
        print(f"# decode done: {dec['ms'] * 1e3:.1f} us/step", file=sys.stderr, flush=True)
    if not args.prefill_only and not args.no_configs:
        out["configs"] = bench_configs(torch, W, staging, _abi)
        print("# configs done", file=sys.stderr, flush=True)
    out["device_copy_GBps"] = round(copy_bandwidth(torch), 1)
    out["pool_hit_ratio"] = hit_ratio_study(W, _abi)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(pre, W)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
