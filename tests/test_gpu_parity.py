"""Parity of the HIP path (through the C interface) with the fp64 oracle, on an MI355X.

Every case prints its name before touching the GPU so that a failure is
attributable.  Sizes: the tiny fp32 case in full; the Llama-3.1-8B prefill
case in full; the other cases at their real shapes with requests or query
tokens sampled where the oracle would take minutes.
"""
import dataclasses
import sys
import types

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
import workloads as W  # noqa: E402
from position_agnostic_kv_pool_amd import _abi, staging  # noqa: E402
from _helpers import OracleFp8State, OracleState, assert_parity, diff_stats, gpu_f64, half_ulp, within  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    _abi.lib()  # raises if the library was not built


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def sync():
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# helpers running one phase on both sides
# ---------------------------------------------------------------------------
def run_prefill(wl, num_splits=0, pe=None, block_permutation=None, pools=None, exact_max=False, pb=None, keys=None):
    s = wl.spec
    cfg = staging.config_for(s, pe=pe, exact_max=exact_max, keys=keys)
    if pb is None:
        pb = wl.prefill_batch()
    if pools is None:
        pools = staging.DevicePools(wl, DEV, block_permutation)
    staging.append_tokens(cfg, pools, pb, s.dtype, DEV, block_permutation)
    call = staging.PrefillCall(cfg, s, pb, DEV, num_splits, block_permutation)
    out = call.run(pools)
    sync()
    return pb, gpu_f64(out), pools


def sample_tokens(q_len, k, rng):
    if q_len <= k:
        return np.arange(q_len)
    pick = set([0, q_len - 1]) | set(rng.choice(q_len, k - 2, replace=False).tolist())
    return np.array(sorted(pick))


def compare_prefill(wl, pb, got, orc, requests=None, token_subset=None, pe=None, label="", ref=None):
    """ref: the oracle's rows from an earlier call with the same arguments (else computed here)."""
    if ref is None:
        ref = orc.prefill(pb, token_subset=token_subset, requests=requests, pe=pe)
    cu = pb["cu_q_lens"]
    gs, rs = [], []
    for r, o in ref.items():
        local = np.arange(cu[r + 1] - cu[r]) if token_subset is None else np.asarray(token_subset[r])
        gs.append(got[cu[r] + local])
        rs.append(o)
    g, rr = np.concatenate(gs), np.concatenate(rs)
    mx, mn = assert_parity(g, rr, wl.spec.dtype, label)
    say(f"{label}: max {mx:.2e} mean {mn:.2e} over {g.shape[0]} tokens")
    return g, ref


# ---------------------------------------------------------------------------
# metadata and append: bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg_id,kw", [(1, {}), (2, {}), (4, {"requests": [2]}), (5, {"skew": 1.2})])
def test_debug_decode_tables_bit_exact(cfg_id, kw):
    say("debug-decode", cfg_id, kw)
    wl = W.build_workload(W.spec(cfg_id, **kw))
    inputs = wl.prefill_batch() or wl.decode_step(0)
    dt = staging.DeviceTables.from_inputs(inputs, DEV)
    E = dt.batch.max_entries
    out = torch.empty((len(inputs["ctx_lens"]), E, 3), dtype=torch.int32, device=DEV)
    _abi.debug_decode_tables(dt.batch, out)
    sync()
    got = out.cpu().numpy()
    words = O.pack_table(inputs["table_blocks"], inputs["table_starts"])
    for r in range(len(inputs["ctx_lens"])):
        n = int(inputs["num_entries"][r])
        b, s, l = O.decode_table(words[r], n, int(inputs["ctx_lens"][r]), 16, wl.num_blocks)
        assert np.array_equal(got[r, :n, 0], b)
        assert np.array_equal(got[r, :n, 1], s)
        assert np.array_equal(got[r, :n, 2], l)
        assert np.array_equal(got[r, :n, 0], inputs["table_blocks"][r, :n].astype(np.int64))
        assert np.all(got[r, n:] == -1)


@pytest.mark.parametrize("cfg_id", [1, 5])
def test_append_kv_bit_exact(cfg_id):
    say("append", cfg_id)
    wl = W.build_workload(W.spec(cfg_id, requests=[4, 4]) if cfg_id == 5 else W.spec(cfg_id))
    s = wl.spec
    cfg = staging.config_for(s)
    pools = staging.DevicePools(wl, DEV)
    k_before = pools.k.clone()
    pb = wl.prefill_batch()
    staging.append_tokens(cfg, pools, pb, s.dtype, DEV)
    sync()
    orc = OracleState(wl)
    orc.append(pb)
    blocks = np.unique(pb["slots"] // 16)
    view = np.int16 if s.dtype == "bf16" else np.float32
    gk = pools.k[torch.from_numpy(blocks).to(DEV)].cpu().view(torch.int16 if s.dtype == "bf16" else torch.float32).numpy()
    gv = pools.v[torch.from_numpy(blocks).to(DEV)].cpu().view(torch.int16 if s.dtype == "bf16" else torch.float32).numpy()
    ok_k = orc.k[blocks].view(view)
    ok_v = orc.v[blocks].view(view)
    # compare bit patterns (NaN padding included)
    assert np.array_equal(gk.view(np.uint8), np.ascontiguousarray(ok_k).view(np.uint8))
    assert np.array_equal(gv.view(np.uint8), np.ascontiguousarray(ok_v).view(np.uint8))
    # nothing else in the pool moved
    mask = torch.ones(wl.num_blocks, dtype=torch.bool, device=DEV)
    mask[torch.from_numpy(blocks).to(DEV)] = False
    a = pools.k[mask].view(torch.int16 if s.dtype == "bf16" else torch.int32)
    b = k_before[mask].view(torch.int16 if s.dtype == "bf16" else torch.int32)
    assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# parity on the five configurations
# ---------------------------------------------------------------------------
def test_parity_tiny_f32_prefill_and_decode():
    say("tiny fp32: prefill + 8 decode steps")
    wl = W.build_workload(W.spec(1))
    s = wl.spec
    cfg = staging.config_for(s)
    pb, got, pools = run_prefill(wl)
    orc = OracleState(wl)
    orc.append(pb)
    compare_prefill(wl, pb, got, orc, label="tiny prefill")
    for step in range(8):
        d = wl.decode_step(step)
        staging.append_tokens(cfg, pools, d, s.dtype, DEV)
        orc.append(d)
        out = gpu_f64(staging.DecodeCall(cfg, s, d, DEV).run(pools))
        ref = orc.decode(d)
        mx, mn = assert_parity(out, np.stack([ref[r] for r in range(len(ref))]), "f32", f"tiny decode {step}")
    say(f"tiny decode last step: max {mx:.2e}")


@pytest.mark.parametrize("num_splits", [0, 1])
def test_parity_llama8b_prefill_full(num_splits):
    say("8B prefill full, splits", num_splits)
    wl = W.build_workload(W.spec(2))
    pb, got, _ = run_prefill(wl, num_splits=num_splits)
    orc = OracleState(wl)
    orc.append(pb)
    compare_prefill(wl, pb, got, orc, label=f"8B prefill splits={num_splits}")


def test_parity_llama8b_decode():
    say("8B decode: 16 requests, suffix prefill then steps 0, 1, 15, 16, 40")
    wl = W.build_workload(W.spec(3, requests=[16], n_decode=41))
    s = wl.spec
    cfg = staging.config_for(s)
    pb, got, pools = run_prefill(wl)
    orc = OracleState(wl)
    orc.append(pb)
    compare_prefill(wl, pb, got, orc, label="8B suffix prefill")
    for step in range(41):
        d = wl.decode_step(step)
        staging.append_tokens(cfg, pools, d, s.dtype, DEV)
        orc.append(d)
        if step in (0, 1, 15, 16, 40):
            out = gpu_f64(staging.DecodeCall(cfg, s, d, DEV).run(pools))
            ref = orc.decode(d)
            mx, mn = assert_parity(out, np.stack([ref[r] for r in range(len(ref))]), "bf16", f"8B decode {step}")
            say(f"8B decode step {step}: max {mx:.2e} mean {mn:.2e}")


@pytest.mark.timeout(300)
def test_parity_llama8b_decode_full_batch_as_benched():
    # the decode launch the benchmark times: all 128 requests, the heuristic split
    # count (one split: the attention kernel writes bf16 outputs directly, no merge);
    # the oracle checks every 8th request at the first two steps and the last one
    say("8B decode, full batch of 128 requests, heuristic splits, steps 0, 1, 255 (every 8th request)")
    wl = W.build_workload(W.spec(3, n_decode=256))
    s = wl.spec
    cfg = staging.config_for(s)
    pools = staging.DevicePools(wl, DEV)
    orc = OracleState(wl)
    reqs = list(range(0, 128, 8))
    before = wl.tokens_before_step(0)
    staging.append_tokens(cfg, pools, before, s.dtype, DEV)
    orc.append(before)
    for step in (0, 1, 255):
        if step == 255:
            # every token of steps 2..254, then step 255's own
            rest = wl.tokens_before_step(255)
            prev = wl.tokens_before_step(2)
            keep = ~np.isin(rest["slots"], prev["slots"])
            rest = {k: v[keep] for k, v in rest.items()}
            staging.append_tokens(cfg, pools, rest, s.dtype, DEV)
            orc.append(rest)
        d = wl.decode_step(step)
        staging.append_tokens(cfg, pools, d, s.dtype, DEV)
        orc.append(d)
        call = staging.DecodeCall(cfg, s, d, DEV)
        assert len(d["ctx_lens"]) == 128 and call.splits == 1 and call.workspace is None
        out = gpu_f64(call.run(pools))
        ref = orc.decode(d, requests=reqs)
        mx, mn = assert_parity(out[reqs], np.stack([ref[r] for r in reqs]), "bf16",
                               f"8B decode 128 req splits=1 step {step}")
        say(f"8B decode full batch step {step}: max {mx:.2e} mean {mn:.2e}")


@pytest.mark.timeout(400)
def test_parity_llama70b_all_requests_as_benched():
    # the 70B launches the benchmark times: the 2048-token chunk of all 4 requests
    # (sampled rows of each), then decode of all 4 requests at the heuristic split
    # count, steps 0 and 127
    say("70B 32k: 4 requests, chunk prefill (sampled rows of each), decode steps 0 and 127 at heuristic splits")
    wl = W.build_workload(W.spec(4, n_decode=128))
    s = wl.spec
    cfg = staging.config_for(s)
    pb, got, pools = run_prefill(wl)
    orc = OracleState(wl)
    orc.append(pb)
    rng = np.random.default_rng(7)
    # request 0: rows at and around the 32-position tile boundaries; the others sampled
    subset = {0: np.array(sorted(set([0, 1, 31, 32, 33, 1023, 1024, 2046, 2047]) |
                                 set(rng.choice(2048, 6, replace=False).tolist())))}
    subset.update({r: sample_tokens(2048, 6, rng) for r in range(1, 4)})
    assert _abi.prefill_workspace_size(cfg, 4, int(pb["total_q"]), int(pb["max_q_len"]), 1, 1) > 0   # keys turned once
    _, ref = compare_prefill(wl, pb, got, orc, token_subset=subset, label="70B chunk prefill, 4 requests")
    fused = run_prefill(wl, pools=pools, pb=pb, keys="fused")[1]
    compare_prefill(wl, pb, fused, orc, token_subset=subset, ref=ref,
                    label="70B chunk prefill, 4 requests, keys turned in the attention kernel")
    mx, mn = diff_stats(got, fused)
    say(f"70B chunk: keys turned once vs in the kernel, every row: max {mx:.2e} mean {mn:.2e}")
    assert mx <= 2e-2 and mn <= 1e-3
    d0 = wl.decode_step(0)
    staging.append_tokens(cfg, pools, d0, s.dtype, DEV)
    orc.append(d0)
    ref0 = orc.decode(d0)
    for splits in (1, 7, 64):
        out = gpu_f64(staging.DecodeCall(cfg, s, d0, DEV, num_splits=splits).run(pools))
        mx, mn = assert_parity(out, np.stack([ref0[r] for r in range(4)]), "bf16",
                               f"70B decode 4 req splits={splits} step 0")
        say(f"70B decode step 0 splits={splits}: max {mx:.2e} mean {mn:.2e}")
    for step, d in ((0, d0), (127, None)):
        if d is None:
            rest = wl.tokens_before_step(127)
            keep = ~np.isin(rest["slots"], wl.tokens_before_step(1)["slots"])
            rest = {k: v[keep] for k, v in rest.items()}
            staging.append_tokens(cfg, pools, rest, s.dtype, DEV)
            orc.append(rest)
            d = wl.decode_step(127)
            staging.append_tokens(cfg, pools, d, s.dtype, DEV)
            orc.append(d)
        call = staging.DecodeCall(cfg, s, d, DEV)
        assert call.splits == _abi.decode_splits(cfg, 4, call.tables.batch.max_entries) and call.splits > 1
        out = gpu_f64(call.run(pools))
        ref = ref0 if step == 0 else orc.decode(d)
        mx, mn = assert_parity(out, np.stack([ref[r] for r in range(4)]), "bf16",
                               f"70B decode 4 req splits={call.splits} step {step}")
        say(f"70B decode 4 requests step {step} splits {call.splits}: max {mx:.2e} mean {mn:.2e}")


# ---------------------------------------------------------------------------
# shared-run decode (one read of a shared block serves every request holding it)
# ---------------------------------------------------------------------------
@pytest.mark.timeout(300)
def test_decode_runs_llama8b_full_batch():
    say("shared-run decode: 8B, all 128 requests, steps 0 and 1 (oracle on every 8th request), "
        "against the per-request decode on all")
    wl = W.build_workload(W.spec(3, n_decode=2))
    s = wl.spec
    cfg = staging.config_for(s)
    pools = staging.DevicePools(wl, DEV)
    orc = OracleState(wl)
    reqs = list(range(0, 128, 8))
    before = wl.tokens_before_step(0)
    staging.append_tokens(cfg, pools, before, s.dtype, DEV)
    orc.append(before)
    for step in (0, 1):
        d = wl.decode_step(step)
        staging.append_tokens(cfg, pools, d, s.dtype, DEV)
        orc.append(d)
        call = staging.RunDecodeCall(cfg, s, d, pools.num_blocks, DEV)
        # the shared documents are read far fewer times than the tables name them
        assert len(call.plan_host["words"]) < 0.5 * int(np.sum(d["num_entries"]))
        out = gpu_f64(call.run(pools))
        ref = orc.decode(d, requests=reqs)
        mx, mn = assert_parity(out[reqs], np.stack([ref[r] for r in reqs]), "bf16",
                               f"8B shared-run decode step {step}")
        say(f"8B shared-run decode step {step}: max {mx:.2e} mean {mn:.2e}")
        per_req = gpu_f64(staging.DecodeCall(cfg, s, d, DEV).run(pools))
        dmx, dmn = diff_stats(out, per_req)
        say(f"  vs per-request decode, all 128: max {dmx:.2e} mean {dmn:.2e}")
        assert dmx <= 2e-2 and dmn <= 1e-3


@pytest.mark.timeout(300)
def test_decode_runs_encodings_repeats_and_long_context():
    say("shared-run decode: rotation-free and ALiBi (8B, 16 requests), a request holding another's "
        "whole table, FP8 pool, and the 70B 32k step 0 (G = 8)")
    wl = W.build_workload(W.spec(3, requests=[16], n_decode=1))
    s = wl.spec
    pools = staging.DevicePools(wl, DEV)
    orc = OracleState(wl)
    cfg = staging.config_for(s)
    before = wl.tokens_before_step(0)
    staging.append_tokens(cfg, pools, before, s.dtype, DEV)
    orc.append(before)
    d = wl.decode_step(0)
    staging.append_tokens(cfg, pools, d, s.dtype, DEV)
    orc.append(d)
    for pe in ("rope", "none", "alibi"):
        c = staging.config_for(s, pe=pe)
        out = gpu_f64(staging.RunDecodeCall(c, s, d, pools.num_blocks, DEV).run(pools))
        ref = orc.decode(d, pe=pe)
        mx, mn = assert_parity(out, np.stack([ref[r] for r in range(16)]), "bf16", f"8B shared-run decode {pe}")
        say(f"8B shared-run decode {pe}: max {mx:.2e} mean {mn:.2e}")
    # request 1 holds request 0's table (the same blocks at the same positions), with its own query
    d2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in d.items()}
    for key in ("table_blocks", "table_starts"):
        d2[key][1] = d2[key][0]
    for key in ("num_entries", "ctx_lens"):
        d2[key][1] = d2[key][0]
    call = staging.RunDecodeCall(cfg, s, d2, pools.num_blocks, DEV)
    out = gpu_f64(call.run(pools))
    ref = orc.decode(d2, requests=[0, 1, 2])
    mx, mn = assert_parity(out[:3], np.stack([ref[r] for r in range(3)]), "bf16", "shared-run decode, shared table")
    say(f"shared-run decode, request 1 = request 0's table: max {mx:.2e} mean {mn:.2e}")
    # FP8 pool
    cfg8 = staging.config_for(s, kv_format="fp8")
    pools8 = staging.WrittenPools(wl, cfg8, DEV)
    orc8 = OracleFp8State(wl)
    for inp in (before, d):
        staging.append_tokens(cfg8, pools8, inp, s.dtype, DEV)
        orc8.append(inp)
    out = gpu_f64(staging.RunDecodeCall(cfg8, s, d, pools8.num_blocks, DEV).run(pools8))
    ref = orc8.decode(d)
    mx, mn = assert_parity(out, np.stack([ref[r] for r in range(16)]), "bf16", "FP8 shared-run decode")
    say(f"FP8 8B shared-run decode: max {mx:.2e} mean {mn:.2e}")
    del pools, pools8
    # 70B, 4 requests over 32k contexts: long runs cut into pieces of 64 entries
    wl = W.build_workload(W.spec(4, n_decode=1))
    s = wl.spec
    cfg = staging.config_for(s)
    pools = staging.DevicePools(wl, DEV)
    orc = OracleState(wl)
    for inp in (wl.prefill_batch(), wl.decode_step(0)):
        staging.append_tokens(cfg, pools, inp, s.dtype, DEV)
        orc.append(inp)
    d = wl.decode_step(0)
    out = gpu_f64(staging.RunDecodeCall(cfg, s, d, pools.num_blocks, DEV).run(pools))
    ref = orc.decode(d)
    mx, mn = assert_parity(out, np.stack([ref[r] for r in range(4)]), "bf16", "70B shared-run decode")
    say(f"70B shared-run decode step 0: max {mx:.2e} mean {mn:.2e}")


@pytest.mark.parametrize("skew", W.CFG5_SKEWS)
@pytest.mark.parametrize("pe", W.CFG5_PES)
def test_parity_mqa_stress(skew, pe):
    say(f"MQA stress skew={skew} pe={pe}: 32 prefill requests (sampled rows), 96 decode requests steps 0..7")
    wl = W.build_workload(W.spec(5, skew=skew, pe=pe))
    s = wl.spec
    cfg = staging.config_for(s)
    pb, got, pools = run_prefill(wl)
    orc = OracleState(wl)
    orc.append(pb)
    rng = np.random.default_rng(1)
    subset = {r: sample_tokens(128, 10, rng) for r in range(len(pb["ctx_lens"]))}
    _, ref = compare_prefill(wl, pb, got, orc, token_subset=subset, label=f"MQA prefill {skew}/{pe}")
    if pe == "rope":   # 16 query tiles per request: the keys were turned once; the fused route too
        fused = run_prefill(wl, pools=pools, pb=pb, keys="fused")[1]
        compare_prefill(wl, pb, fused, orc, token_subset=subset, ref=ref,
                        label=f"MQA prefill {skew}/{pe}, keys turned in the attention kernel")
    for step in range(8):
        d = wl.decode_step(step)
        staging.append_tokens(cfg, pools, d, s.dtype, DEV)
        orc.append(d)
        if step in (0, 7):
            out = gpu_f64(staging.DecodeCall(cfg, s, d, DEV).run(pools))
            reqs = list(range(0, len(d["ctx_lens"]), 4))      # every 4th of the 96 for the oracle
            ref = orc.decode(d, requests=reqs)
            mx, mn = assert_parity(out[reqs], np.stack([ref[r] for r in reqs]), "bf16",
                                   f"MQA decode {skew}/{pe} step {step}")
            say(f"MQA decode step {step}: max {mx:.2e} mean {mn:.2e}")


# ---------------------------------------------------------------------------
# invariances the method relies on
# ---------------------------------------------------------------------------
def test_physical_relocation_is_bit_identical():
    say("relocation: same logical inputs, permuted physical blocks")
    wl = W.build_workload(W.spec(2, requests=[4]))
    perm = np.random.default_rng(5).permutation(wl.num_blocks).astype(np.int64)
    _, a, _ = run_prefill(wl)
    _, b, _ = run_prefill(wl, block_permutation=perm)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("keys", [None, "fused"])
def test_pool_is_read_only_and_padding_poison_stays_out(keys):
    say(f"pools unchanged by prefill (keys {keys or 'turned once: the default here'}) and decode; "
        "outputs finite despite NaN padding")
    wl = W.build_workload(W.spec(5, requests=[6, 6], skew=1.6))
    s = wl.spec
    cfg = staging.config_for(s, keys=keys)
    pools = staging.DevicePools(wl, DEV)
    pb = wl.prefill_batch()
    staging.append_tokens(cfg, pools, pb, s.dtype, DEV)
    d = wl.decode_step(0)
    staging.append_tokens(cfg, pools, d, s.dtype, DEV)
    k0, v0 = pools.k.view(torch.int16).clone(), pools.v.view(torch.int16).clone()
    o1 = staging.PrefillCall(cfg, s, pb, DEV).run(pools)
    o2 = staging.DecodeCall(cfg, s, d, DEV).run(pools)
    sync()
    assert torch.equal(pools.k.view(torch.int16), k0) and torch.equal(pools.v.view(torch.int16), v0)
    assert torch.isfinite(o1.float()).all() and torch.isfinite(o2.float()).all()


def test_decode_split_count_invariance():
    say("decode split counts 1..37 agree")
    wl = W.build_workload(W.spec(4, requests=[2], n_decode=1))
    s = wl.spec
    cfg = staging.config_for(s)
    pools = staging.DevicePools(wl, DEV)
    staging.append_tokens(cfg, pools, wl.tokens_before_step(0), s.dtype, DEV)
    d = wl.decode_step(0)
    staging.append_tokens(cfg, pools, d, s.dtype, DEV)
    outs = [gpu_f64(staging.DecodeCall(cfg, s, d, DEV, num_splits=k).run(pools)) for k in (1, 2, 5, 37, 256)]
    for o in outs[1:]:
        mx, mn = diff_stats(o, outs[0])
        assert mx <= 4e-3 and mn <= 2e-4


def test_decode_matches_last_prefill_row():
    say("decode == last row of prefill over the same context")
    wl = W.build_workload(W.spec(3, requests=[8], n_decode=0, q_len=17))
    s = wl.spec
    cfg = staging.config_for(s)
    pb, got, pools = run_prefill(wl)
    # decode inputs built from the prefill batch: the last query row of each request
    cu = pb["cu_q_lens"]
    d = dict(pb)
    d["q"] = pb["q"][cu[1:] - 1]
    out = gpu_f64(staging.DecodeCall(cfg, s, d, DEV).run(pools))
    mx, mn = diff_stats(out, got[cu[1:] - 1])
    assert mx <= 1e-2 and mn <= 1e-3


def test_prefill_split_count_invariance_and_empty_splits():
    say("prefill split counts 1..64 (many splits are empty) agree")
    wl = W.build_workload(W.spec(2, requests=[2], docs=(1, 1)))
    outs = [run_prefill(wl, num_splits=k)[1] for k in (1, 3, 64)]
    for o in outs[1:]:
        mx, mn = diff_stats(o, outs[0])
        assert mx <= 4e-3 and mn <= 2e-4


@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_prefill_keys_once_llama8b_full(num_splits):
    say("8B prefill full, keys turned once first (forced), splits", num_splits)
    wl = W.build_workload(W.spec(2))
    pb, got, pools = run_prefill(wl, num_splits=num_splits, keys="once")
    orc = OracleState(wl)
    orc.append(pb)
    compare_prefill(wl, pb, got, orc, label=f"8B prefill, keys once, splits={num_splits}")
    fused = run_prefill(wl, num_splits=num_splits, pools=pools, pb=pb, keys="fused")[1]
    mx, mn = diff_stats(got, fused)
    say(f"keys once vs fused: max {mx:.2e} mean {mn:.2e}")
    assert mx <= 2e-2 and mn <= 1e-3


def test_prefill_keys_once_exact_maximum_route():
    say("8B prefill, keys turned once (forced) on the two-pass exact-maximum route")
    wl = W.build_workload(W.spec(2, requests=[6]))
    pb, got, _ = run_prefill(wl, num_splits=2, keys="once", exact_max=True)
    orc = OracleState(wl)
    orc.append(pb)
    compare_prefill(wl, pb, got, orc, label="8B prefill, keys once, exact route")


def test_prefill_keys_once_ragged_edges_and_workspace_reuse():
    say("keys turned once: ragged query tiles, long chunk over few documents, requests without documents, "
        "a zero-length request, one workspace reused by a smaller call")
    # 300 positions x 4 heads = 4.7 query tiles; 3 splits over 1..3 documents
    wl = W.build_workload(W.spec(2, requests=[5], q_len=300, docs=(1, 3)))
    pb, got, pools = run_prefill(wl, num_splits=3, keys="once")
    orc = OracleState(wl)
    orc.append(pb)
    compare_prefill(wl, pb, got, orc, label="ragged 300-token chunks, keys once, 3 splits")
    # no documents: each context is the chunk itself; chunks of 1 and 40 tokens
    for q_len in (1, 40):
        wl1 = W.build_workload(W.spec(2, requests=[3], docs=(0, 0), q_len=q_len))
        pb1, got1, _ = run_prefill(wl1, keys="once")
        orc1 = OracleState(wl1)
        orc1.append(pb1)
        compare_prefill(wl1, pb1, got1, orc1, label=f"{q_len}-token contexts without documents, keys once")
    # a request with no new tokens in the middle of the batch
    s = wl.spec
    cfg = staging.config_for(s, keys="once")
    ins = dict(pb)
    cu = pb["cu_q_lens"]
    ins["cu_q_lens"] = np.array([0, 300, 300, 600, 900, 1200], dtype=np.int32)
    keep = np.r_[cu[0]:cu[1], cu[2]:cu[5]]
    ins["q"] = pb["q"][keep]
    ins["total_q"] = 1200
    ctx = pb["ctx_lens"].copy()
    ctx[1] -= 300
    ins["ctx_lens"] = ctx
    ne = pb["num_entries"].copy()
    ne[1] = wl.requests[1].n_doc_entries
    ins["num_entries"] = ne
    call = staging.PrefillCall(cfg, s, ins, DEV, 2)
    out = gpu_f64(call.run(pools))
    ref = orc.prefill(pb)
    for r, rows in ((0, slice(0, 300)), (2, slice(300, 600)), (4, slice(900, 1200))):
        assert_parity(out[rows], ref[r], "bf16", f"zero-length request: request {r}")
    # the same workspace, dirty from the call above, serves a smaller batch
    small = W.build_workload(W.spec(2, requests=[2], q_len=70, docs=(1, 1)))
    spb = small.prefill_batch()
    spools = staging.DevicePools(small, DEV)
    staging.append_tokens(cfg, spools, spb, s.dtype, DEV)
    scall = staging.PrefillCall(cfg, s, spb, DEV, 2)
    need = scall.workspace.numel()
    assert need <= call.workspace.numel()
    scall.workspace = call.workspace
    sout = gpu_f64(scall.run(spools))
    sorc = OracleState(small)
    sorc.append(spb)
    compare_prefill(small, spb, sout, sorc, label="smaller call in a reused workspace, keys once")


@pytest.mark.parametrize("num_splits,heads", [(1, (32, 8)), (3, (32, 8)), (1, (8, 1))])
def test_prefill_long_chunk_tiles_grouped_per_xcd(num_splits, heads):
    # 8B shape: a 2048-token chunk spans 32 query tiles per (request, KV head) and the
    # (split, request, KV head) units are a multiple of 8, so every unit's tiles run on one
    # XCD.  Hq 8, Hkv 1 (one GPU's share under 8-way tensor parallelism): 1024 tokens make
    # 32 tiles and the 2 requests 2 units, each spread over 4 XCDs
    hq, hkv = heads
    say(f"Hq {hq} Hkv {hkv}, long chunks over one document, {num_splits} splits: tiles grouped per XCD, "
        "keys turned once / in the kernel / rotation-free")
    spec = W.spec(2, requests=[2], q_len=2048 if hkv == 8 else 1024, docs=(1, 1))
    wl = W.build_workload(dataclasses.replace(spec, num_q_heads=hq, num_kv_heads=hkv))
    pb = wl.prefill_batch()
    orc = OracleState(wl)
    orc.append(pb)
    rng = np.random.default_rng(11)
    subset = {r: sample_tokens(int(pb["max_q_len"]), 12, rng) for r in range(2)}
    pools = None
    for pe, keys in (("rope", None), ("rope", "fused"), ("none", None)):
        _, got, pools = run_prefill(wl, num_splits=num_splits, pe=pe, keys=keys, pools=pools, pb=pb)
        compare_prefill(wl, pb, got, orc, token_subset=subset, pe=pe,
                        label=f"{int(pb['max_q_len'])}-token chunks, Hq={hq}, splits={num_splits}, pe={pe}, "
                              f"keys={keys or 'auto'}")


def test_decode_request_order_is_bit_identical():
    say("decode (MQA: 32-column waves; 8B: 16-column waves): requests longest first, reversed, in batch order, "
        "or through an out-of-range entry agree bit for bit")
    for cid, kw in ((5, dict(skew=1.2, requests=[0, 24])), (3, dict(requests=[16], n_decode=1))):
        wl = W.build_workload(W.spec(cid, **kw))
        s = wl.spec
        cfg = staging.config_for(s)
        pools = staging.DevicePools(wl, DEV)
        staging.append_tokens(cfg, pools, wl.tokens_before_step(1), s.dtype, DEV)
        d = wl.decode_step(0)
        staging.append_tokens(cfg, pools, d, s.dtype, DEV)
        R = len(d["ctx_lens"])
        odd = np.arange(R, dtype=np.int32)
        odd[1] = -3                                     # stands for its own index, 1
        orders = [None, "longest_first", np.arange(R, dtype=np.int32)[::-1].copy(), odd]
        for splits in (1, 5):
            outs = [staging.DecodeCall(cfg, s, d, DEV, splits, req_order=o).run(pools).clone() for o in orders]
            sync()
            for o in outs[1:]:
                assert torch.equal(o, outs[0])


def test_prefill_request_order_is_bit_identical():
    say("prefill: requests taken longest first, reversed, in batch order, or through an out-of-range entry agree bit for bit")
    wl = W.build_workload(W.spec(5, skew=0.0, requests=[12, 1]))
    s = wl.spec
    cfg = staging.config_for(s)
    pb = wl.prefill_batch()
    R = len(pb["ctx_lens"])
    pools = staging.DevicePools(wl, DEV)
    staging.append_tokens(cfg, pools, pb, s.dtype, DEV)
    lf = staging.longest_first(pb["num_entries"])
    assert sorted(lf.tolist()) == list(range(R)) and np.all(np.diff(pb["num_entries"][lf]) <= 0)
    odd = np.arange(R, dtype=np.int32)
    odd[1] = R + 5                                    # stands for its own index, 1
    orders = [None, "longest_first", np.arange(R, dtype=np.int32)[::-1].copy(), odd]
    for splits in (1, 3):
        outs = []
        for order in orders:
            call = staging.PrefillCall(cfg, s, pb, DEV, splits, req_order=order)
            outs.append(call.run(pools).clone())
        sync()
        for o in outs[1:]:
            assert torch.equal(o, outs[0])
    mx, _ = diff_stats(gpu_f64(outs[0]), run_prefill(wl, num_splits=3, pools=pools, pb=pb)[1])
    assert mx == 0.0


# ---------------------------------------------------------------------------
# rotation-free and ALiBi instantiations on the same inputs
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("pe", ["none", "alibi"])
def test_other_encodings_llama8b_prefill(pe):
    say("8B prefill with pe", pe)
    wl = W.build_workload(W.spec(2, requests=[4]))
    pb, got, _ = run_prefill(wl, pe=pe)
    orc = OracleState(wl)
    orc.append(pb)
    compare_prefill(wl, pb, got, orc, pe=pe, label=f"8B prefill pe={pe}")


@pytest.mark.parametrize("num_splits", [1, 5])
def test_alibi_prefill_running_reference(num_splits):
    """ALiBi's softmax reference follows the running row maximum.  One split puts a
    whole 4k-token context in one work-group (the reference moves tile after tile);
    five splits start some work-groups far from the query.  Both against the oracle
    and against the exact-maximum route on the same inputs."""
    say(f"8B ALiBi prefill, running reference, splits={num_splits}")
    wl = W.build_workload(W.spec(2, requests=[4]))
    pb, got, pools = run_prefill(wl, pe="alibi", num_splits=num_splits)
    orc = OracleState(wl)
    orc.append(pb)
    compare_prefill(wl, pb, got, orc, pe="alibi", label=f"8B ALiBi prefill splits={num_splits}")
    _, exact, _ = run_prefill(wl, pe="alibi", exact_max=True, num_splits=num_splits, pools=pools, pb=pb)
    compare_prefill(wl, pb, exact, orc, pe="alibi", label=f"8B ALiBi prefill, exact route, splits={num_splits}")
    # steep heads weigh a few keys, so outputs reach |o| ~ 4 and each route carries
    # the bf16 weights' rounding (~1e-2 there): two results each within the bf16 bar
    # of the exact value (half a step + 1e-2) are within one step + 2e-2 of each other
    d = np.abs(got - exact)
    excess = d - 2.0 * half_ulp(np.maximum(np.abs(got), np.abs(exact)), "bf16")
    say(f"running vs exact reference: max {d.max():.2e} (beyond one bf16 step {excess.max():.2e}) "
        f"mean {d.mean():.2e}")
    assert excess.max() <= 2e-2 and d.mean() <= 5e-4


# ---------------------------------------------------------------------------
# softmax reference: the exact two-pass route, forced and triggered
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("pe", ["rope", "none"])
def test_prefill_exact_maximum_route(pe):
    say("8B prefill, exact-maximum route forced, pe", pe)
    wl = W.build_workload(W.spec(2, requests=[4]))
    pb, got, _ = run_prefill(wl, pe=pe, exact_max=True)
    orc = OracleState(wl)
    orc.append(pb)
    compare_prefill(wl, pb, got, orc, pe=pe, label=f"8B prefill exact route pe={pe}")
    _, fast, _ = run_prefill(wl, pe=pe)
    mx, mn = diff_stats(fast, got)
    say(f"fast vs exact route: max {mx:.2e} mean {mn:.2e}")
    assert mx <= 4e-3 and mn <= 2e-4


def test_prefill_redo_when_scores_outgrow_the_first_tile():
    # queries scaled by 64 (exact in bf16) spread each row's scores over
    # hundreds of base-2 units, so later key tiles exceed the first tile's
    # maximum by far more than 2^64 and the work-groups must redo their rows
    # with the exact maximum: the result is then the exact route's, bit for
    # bit (without the redo it would overflow)
    say("8B prefill with queries scaled by 64 (redo route)")
    wl = W.build_workload(W.spec(2, requests=[2]))
    pb = dict(wl.prefill_batch())
    pb["q"] = W.f32_to_bf16_bits(W.bf16_bits_to_f32(pb["q"]) * np.float32(64.0))
    for splits in (1, 2):
        _, fast, _ = run_prefill(wl, pb=pb, num_splits=splits)
        _, exact, _ = run_prefill(wl, pb=pb, num_splits=splits, exact_max=True)
        assert np.all(np.isfinite(fast))
        assert np.array_equal(fast, exact)
    # the peaked softmax still follows the oracle (scores carry bf16 rounding
    # of a few tenths of a base-2 unit at this scale, hence the loose bound)
    orc = OracleState(wl)
    orc.append(pb)
    ref = orc.prefill(pb)
    cu = pb["cu_q_lens"]
    g = np.concatenate([exact[cu[r]:cu[r + 1]] for r in ref])
    rr = np.concatenate([ref[r] for r in ref])
    mx, mn = diff_stats(g, rr)
    say(f"scaled queries vs oracle: max {mx:.2e} mean {mn:.2e}")
    assert mn <= 5e-2


def test_alibi_prefill_far_keys_with_huge_scores():
    # ALiBi walks each work-group's key tiles nearest-first and takes the softmax
    # reference from the nearest tile.  Request 0's first document with keys
    # scaled by 64 (exact in bf16) scores ~200 base-2 units above the rest.  On
    # heads 0..11 (slope >= 1/8) its bias over > 3.5k positions exceeds 600 units:
    # it weighs nothing, and the outputs follow the oracle at the usual bar.  On
    # heads 20..31 it dominates and the row sums pass 2^64, so those work-groups
    # redo their rows with the exact maximum: bit for bit the exact route's.
    say("8B ALiBi prefill, first document's keys scaled by 64")
    wl = W.build_workload(W.spec(2, requests=[2]))
    pb = wl.prefill_batch()
    blocks = wl.doc_blocks(int(pb["requests"][0].doc_ids[0]))
    pools = staging.DevicePools(wl, DEV)
    bi = torch.from_numpy(np.asarray(blocks, dtype=np.int64)).to(DEV)
    pools.k[bi] = pools.k[bi] * 64
    orc = OracleState(wl)
    orc.k[blocks] = W.f32_to_bf16_bits(W.bf16_bits_to_f32(orc.k[blocks]) * np.float32(64.0))
    orc.append(pb)
    _, fast, _ = run_prefill(wl, pe="alibi", num_splits=1, pools=pools, pb=pb)
    _, exact, _ = run_prefill(wl, pe="alibi", num_splits=1, pools=pools, pb=pb, exact_max=True)
    assert np.all(np.isfinite(fast))
    a, b = int(pb["cu_q_lens"][0]), int(pb["cu_q_lens"][1])
    assert np.array_equal(fast[a:b, 20:], exact[a:b, 20:])
    steep = list(range(12))
    ref = orc.prefill(pb, pe="alibi", requests=[0], heads=steep)[0]
    mx, mn = assert_parity(fast[a:b, steep], ref, "bf16", "ALiBi, far keys with huge scores")
    say(f"ALiBi far huge keys, heads 0..11 of request 0: max {mx:.2e} mean {mn:.2e}")


def test_alibi_prefill_redo_when_every_weight_underflows():
    # A 496-token document (31 entries) then a 64-token chunk: one split holds
    # 35 entries, so the nearest tile is entries 32..34 (positions 512..559) and
    # the chunk's first 16 rows (positions 496..511) see none of its keys; they
    # keep reference 0.  Every key equal to (1, ..., 1) and every query to
    # -12.25 (..., 1) put every score at -200 base-2 units: those rows' weights
    # all underflow, and the work-groups must redo them with the exact maximum
    # (bit for bit the exact route's; without the redo they would divide 0 by 0).
    say("8B ALiBi prefill, constant scores of -200 (underflow redo route)")
    wl = W.build_workload(W.spec(2, requests=[1], docs=(1, 1), doc_len=496))
    s = wl.spec
    pb = dict(wl.prefill_batch())
    assert int(pb["num_entries"][0]) == 35 and int(pb["table_starts"][0][31]) == 496
    one = W.f32_to_bf16_bits(np.float32(1.0))
    pb["k_new"] = np.full_like(pb["k_new"], one)
    pb["q"] = np.full_like(pb["q"], W.f32_to_bf16_bits(np.float32(-12.25)))
    blocks = wl.doc_blocks(int(pb["requests"][0].doc_ids[0]))
    pools = staging.DevicePools(wl, DEV)
    bi = torch.from_numpy(np.asarray(blocks, dtype=np.int64)).to(DEV)
    pools.k[bi] = 1.0
    orc = OracleState(wl)
    orc.k[blocks] = np.full_like(orc.k[blocks], one)
    orc.append(pb)
    _, fast, _ = run_prefill(wl, pe="alibi", num_splits=1, pools=pools, pb=pb)
    _, exact, _ = run_prefill(wl, pe="alibi", num_splits=1, pools=pools, pb=pb, exact_max=True)
    assert np.all(np.isfinite(fast))
    assert np.array_equal(fast, exact)
    ref = orc.prefill(pb, pe="alibi")[0]
    mx, mn = assert_parity(fast, ref, s.dtype, "ALiBi underflow redo")
    say(f"ALiBi underflow redo: max {mx:.2e} mean {mn:.2e}")


# ---------------------------------------------------------------------------
# the materialise-then-attend baseline computes the same attention
# ---------------------------------------------------------------------------
def test_materialized_baseline_matches_oracle_and_leaves_the_pool():
    say("8B prefill through the materialise-then-attend baseline")
    wl = W.build_workload(W.spec(2, requests=[3]))
    s = wl.spec
    cfg = staging.config_for(s)
    pb = wl.prefill_batch()
    pools = staging.DevicePools(wl, DEV)
    staging.append_tokens(cfg, pools, pb, s.dtype, DEV)
    k_before = pools.k.clone()
    mat = staging.MaterializedPrefill(s, pb, DEV)
    got = gpu_f64(mat.run(pools))
    sync()
    assert torch.equal(pools.k.view(torch.int16), k_before.view(torch.int16))
    orc = OracleState(wl)
    orc.append(pb)
    compare_prefill(wl, pb, got, orc, label="materialised baseline")
    _, lazy, _ = run_prefill(wl, pools=pools, pb=pb)
    mx, mn = diff_stats(lazy, got)
    say(f"deferred vs materialised: max {mx:.2e} mean {mn:.2e}")
    assert mx <= 1e-2 and mn <= 1e-3


# ---------------------------------------------------------------------------
# document-local frames: keys stored as R(j) k, j the index inside their
# document; the results must be those of the content-only definition
# ---------------------------------------------------------------------------
def test_append_kv_framed_rounds_the_exact_rotation():
    say("framed append: 8B documents written as R(j) k")
    wl = W.build_workload(W.spec(2, requests=[2]))
    s = wl.spec
    cfg = staging.config_for(s)
    pools = staging.FramedPools(wl, cfg, DEV)
    sync()
    inv = O.rope_inv_freq(s.head_dim, s.rope_theta)
    agree, total = 0, 0
    for d in wl.referenced_docs[:4]:
        k, v = wl.doc_kv(int(d))
        slots, j = wl.doc_frame_tokens(int(d))
        exact = O.rotate_into_frames(O.bf16_to_f64(k), j, inv)             # [L][Hkv][D]
        bi = torch.from_numpy(slots // 16).to(DEV)
        ri = torch.from_numpy(slots % 16).to(DEV)
        got = gpu_f64(pools.k[bi, :, ri])                                    # [L][Hkv][D]
        # within half a bf16 ulp of the exact value, plus the float32 rotation
        # error, which scales with the magnitude of the channel pair
        kf = O.bf16_to_f64(k)
        pair = np.sqrt(kf[..., 0::2] ** 2 + kf[..., 1::2] ** 2).repeat(2, axis=-1)
        excess = np.abs(got - exact) - half_ulp(exact, "bf16") - 1e-6 * pair
        say(f"framed append doc {int(d)}: worst excess over the bar {excess.max():.3e}")
        assert excess.max() <= 0
        rounded = O.bf16_to_f64(W.f32_to_bf16_bits(exact.astype(np.float32)))
        agree += int(np.sum(got == rounded))
        total += got.size
        # values are stored unchanged, bit for bit
        gv = pools.v[bi, :, :, ri].cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(gv, v)
        # the rows past the document's end stay poisoned
        L = k.shape[0]
        if L % 16:
            tail = pools.k[int(slots[-1] // 16), :, L % 16:]
            assert torch.isnan(tail.float()).all()
    say(f"framed append: {agree}/{total} values equal the rounded exact rotation")
    assert agree >= 0.999 * total


def _framed_prefill(wl, num_splits=0, exact_max=False):
    s = wl.spec
    cfg = staging.config_for(s, exact_max=exact_max)
    pools = staging.FramedPools(wl, cfg, DEV)
    pb = wl.prefill_batch()
    staging.append_tokens(cfg, pools, pb, s.dtype, DEV)
    out = staging.PrefillCall(cfg, s, pb, DEV, num_splits, framed=True).run(pools)
    sync()
    return pb, gpu_f64(out), pools


@pytest.mark.parametrize("num_splits", [0, 1])
def test_framed_prefill_llama8b_full(num_splits):
    say("framed 8B prefill full, splits", num_splits)
    wl = W.build_workload(W.spec(2))
    pb, got, _ = _framed_prefill(wl, num_splits)
    orc = OracleState(wl)
    orc.append(pb)
    rng = np.random.default_rng(3)
    subset = None if num_splits == 0 else \
        {r: sample_tokens(int(pb["cu_q_lens"][r + 1] - pb["cu_q_lens"][r]), 24, rng) for r in range(len(pb["ctx_lens"]))}
    compare_prefill(wl, pb, got, orc, token_subset=subset, label=f"framed 8B prefill splits={num_splits}")
    _, content, _ = run_prefill(wl, num_splits=num_splits, pb=pb)
    mx, mn = diff_stats(got, content)
    say(f"framed vs content-only kernel: max {mx:.2e} mean {mn:.2e}")


def test_framed_prefill_long_chunks_ignore_the_key_turning_route():
    # MQA stress shape (16 query tiles per request): the content-only pool would take the
    # keys-turned-once route; a framed batch keeps its own kernel, even with KEYS_ONCE set
    say("framed MQA prefill (16 query tiles per request), library choice and KEYS_ONCE forced: framed kernel")
    wl = W.build_workload(W.spec(5, skew=1.2, requests=[6, 0]))
    s = wl.spec
    orc = OracleState(wl)
    rng = np.random.default_rng(9)
    ref = None
    for keys in (None, "once"):
        cfg = staging.config_for(s, keys=keys)
        pools = staging.FramedPools(wl, cfg, DEV)
        pb = wl.prefill_batch()
        staging.append_tokens(cfg, pools, pb, s.dtype, DEV)
        if ref is None:
            orc.append(pb)
            subset = {r: sample_tokens(128, 16, rng) for r in range(len(pb["ctx_lens"]))}
        out = gpu_f64(staging.PrefillCall(cfg, s, pb, DEV, framed=True).run(pools))
        _, ref = compare_prefill(wl, pb, out, orc, token_subset=subset, ref=ref,
                                 label=f"framed MQA prefill, keys={keys or 'auto'}")


def test_framed_prefill_exact_maximum_route():
    say("framed 8B prefill, exact-maximum route")
    wl = W.build_workload(W.spec(2, requests=[3]))
    pb, got, _ = _framed_prefill(wl, exact_max=True)
    orc = OracleState(wl)
    orc.append(pb)
    compare_prefill(wl, pb, got, orc, label="framed 8B prefill exact max")


def test_framed_decode_llama8b():
    say("framed 8B decode: 16 requests, suffix prefill then steps 0, 1, 15, 16, 40")
    wl = W.build_workload(W.spec(3, requests=[16], n_decode=41))
    s = wl.spec
    cfg = staging.config_for(s)
    pb, got, pools = _framed_prefill(wl)
    orc = OracleState(wl)
    orc.append(pb)
    compare_prefill(wl, pb, got, orc, label="framed 8B suffix prefill")
    for step in range(41):
        d = wl.decode_step(step)
        staging.append_tokens(cfg, pools, d, s.dtype, DEV)
        orc.append(d)
        if step in (0, 1, 15, 16, 40):
            out = gpu_f64(staging.DecodeCall(cfg, s, d, DEV, framed=True).run(pools))
            ref = orc.decode(d)
            mx, mn = assert_parity(out, np.stack([ref[r] for r in range(len(ref))]), "bf16",
                                   f"framed 8B decode {step}")
            say(f"framed 8B decode step {step}: max {mx:.2e} mean {mn:.2e}")


def test_framed_decode_long_context_splits_and_mqa():
    say("framed decode: 70B 32k step 0 at splits 0, 1, 7, 64; MQA (G = 32) step 0")
    wl = W.build_workload(W.spec(4, requests=[1], n_decode=1))
    s = wl.spec
    cfg = staging.config_for(s)
    pools = staging.FramedPools(wl, cfg, DEV)
    pb = wl.prefill_batch()
    staging.append_tokens(cfg, pools, pb, s.dtype, DEV)
    d = wl.decode_step(0)
    staging.append_tokens(cfg, pools, d, s.dtype, DEV)
    orc = OracleState(wl)
    orc.append(pb)
    orc.append(d)
    ref = orc.decode(d)
    for splits in (0, 1, 7, 64):
        out = gpu_f64(staging.DecodeCall(cfg, s, d, DEV, num_splits=splits, framed=True).run(pools))
        mx, mn = assert_parity(out, ref[0][None], "bf16", f"framed 70B decode splits={splits}")
        say(f"framed 70B decode splits={splits}: max {mx:.2e} mean {mn:.2e}")
    wl = W.build_workload(W.spec(5, requests=[2, 24], skew=1.2))
    s = wl.spec
    cfg = staging.config_for(s)
    pools = staging.FramedPools(wl, cfg, DEV)
    staging.append_tokens(cfg, pools, wl.tokens_before_step(0), s.dtype, DEV)
    d = wl.decode_step(0)
    staging.append_tokens(cfg, pools, d, s.dtype, DEV)
    orc = OracleState(wl)
    orc.append(wl.tokens_before_step(0))
    orc.append(d)
    out = gpu_f64(staging.DecodeCall(cfg, s, d, DEV, framed=True).run(pools))
    reqs = list(range(0, len(d["ctx_lens"]), 3))
    ref = orc.decode(d, requests=reqs)
    mx, mn = assert_parity(out[reqs], np.stack([ref[r] for r in reqs]), "bf16", "framed MQA decode")
    say(f"framed MQA decode: max {mx:.2e} mean {mn:.2e}")


# ---------------------------------------------------------------------------
# the pool manager places documents; the kernels read its tables
# ---------------------------------------------------------------------------
def test_pool_manager_tables_feed_the_prefill():
    say("pool manager: 8B prefill, 6 requests, documents placed by lazyattn_pool_admit")
    wl = W.build_workload(W.spec(2, requests=[6]))
    s = wl.spec
    cfg = staging.config_for(s)
    pb = wl.prefill_batch()
    reqs = pb["requests"]
    budget = int(sum(wl.doc_nblk[d] for d in wl.referenced_docs))        # room for every document
    n_priv = sum(len(q.private_blocks) for q in reqs)
    nb = budget + n_priv
    dt = staging.torch_dtype(s.dtype)
    kp = torch.full((nb, s.num_kv_heads, 16, s.head_dim), float("nan"), dtype=dt, device=DEV)
    vp = torch.full((nb, s.num_kv_heads, s.head_dim, 16), float("nan"), dtype=dt, device=DEV)
    pool = _abi.Pool(budget, "agnostic")
    E = max(q.entry_blocks.size for q in reqs)
    tb = np.zeros((len(reqs), E), np.uint32)
    ts = np.full((len(reqs), E), 0x7FFFFFFF, np.uint32)
    ne = np.zeros(len(reqs), np.int32)
    priv_map, writes, hits, nxt = {}, 0, 0, budget
    for r, q in enumerate(reqs):
        st, bl, sta, _ = pool.admit(q.doc_ids, q.doc_lens)
        assert np.all(st != _abi.DOC_BYPASS)
        col = 0
        for k, d in enumerate(q.doc_ids):
            nblk = int(wl.doc_nblk[d])
            if st[k] == _abi.DOC_MISS:          # the caller writes a missed document once
                kk, vv = wl.doc_kv(int(d))
                L = kk.shape[0]
                j = np.arange(L)
                slots = bl[col + j // 16].astype(np.int64) * 16 + j % 16
                _abi.append_kv(cfg, kp, vp, nb, staging.to_device(kk, s.dtype, DEV), staging.to_device(vv, s.dtype, DEV),
                               torch.from_numpy(slots).to(DEV))
                writes += 1
            else:
                hits += 1
            col += nblk
        tb[r, :col], ts[r, :col] = bl, sta
        for j, b in enumerate(q.private_blocks):
            priv_map[int(b)] = nxt
            tb[r, col + j] = nxt
            ts[r, col + j] = q.ctx_docs + 16 * j
            nxt += 1
        ne[r] = q.num_entries_after(q.q_len)
    assert writes == len(set(int(d) for q in reqs for d in q.doc_ids)) and hits > 0
    remap = np.array([priv_map[int(b)] for b in pb["slots"] // 16], dtype=np.int64) * 16 + pb["slots"] % 16
    _abi.append_kv(cfg, kp, vp, nb, staging.to_device(pb["k_new"], s.dtype, DEV),
                   staging.to_device(pb["v_new"], s.dtype, DEV), torch.from_numpy(remap).to(DEV))
    inp = dict(pb, table_blocks=tb, table_starts=ts, num_entries=ne)
    placed = types.SimpleNamespace(k=kp, v=vp, num_blocks=nb)
    got = gpu_f64(staging.PrefillCall(cfg, s, inp, DEV).run(placed))
    sync()
    orc = OracleState(wl)
    orc.append(pb)
    compare_prefill(wl, pb, got, orc, label="prefill over pool-manager tables")
    say(f"pool manager: {writes} documents written, {hits} document hits served from shared blocks")


# ---------------------------------------------------------------------------
# RoPE variants: a caller-supplied frequency table (Llama 3.1 rescaling,
# partial rotary), content-only and framed pools
# ---------------------------------------------------------------------------
_VARIANTS = {
    "llama31": lambda s: O.rope_inv_freq_llama31(s.head_dim, s.rope_theta, 8.0, 1.0, 4.0, 8192),
    "partial64": lambda s: O.rope_inv_freq_partial(s.head_dim, 64, s.rope_theta),
}


@pytest.mark.parametrize("variant", sorted(_VARIANTS))
def test_rope_variants_prefill_and_decode(variant):
    say(f"RoPE variant {variant}: 8B prefill (3 requests), decode steps 0 and 5 (8 requests), framed decode")
    wl = W.build_workload(W.spec(2, requests=[3]))
    s = wl.spec
    table = _VARIANTS[variant](s)
    # the library's own table generator gives the same frequencies
    lib_table = _abi.rope_inv_freq_llama31(s.head_dim, s.rope_theta, 8.0, 1.0, 4.0, 8192) \
        if variant == "llama31" else _abi.rope_inv_freq(s.head_dim, 64, s.rope_theta)
    np.testing.assert_allclose(lib_table, table, rtol=1e-14)
    cfg = staging.config_for(s, inv_freq=lib_table)
    pb = wl.prefill_batch()
    pools = staging.DevicePools(wl, DEV)
    staging.append_tokens(cfg, pools, pb, s.dtype, DEV)
    got = gpu_f64(staging.PrefillCall(cfg, s, pb, DEV).run(pools))
    orc = OracleState(wl)
    orc.append(pb)
    ref = orc.prefill(pb, inv_freq=table)
    cu = pb["cu_q_lens"]
    mx, mn = assert_parity(np.concatenate([got[cu[r]:cu[r + 1]] for r in ref]),
                           np.concatenate([ref[r] for r in ref]), "bf16", f"{variant} prefill")
    say(f"{variant} prefill: max {mx:.2e} mean {mn:.2e}")
    # the variant matters: plain RoPE is far from it
    plain = orc.prefill(pb, requests=[0])[0]
    assert np.max(np.abs(plain - ref[0])) > 5e-2

    wl = W.build_workload(W.spec(3, requests=[8], n_decode=6))
    s = wl.spec
    pools = staging.DevicePools(wl, DEV)
    fpools = staging.FramedPools(wl, cfg, DEV)
    orc = OracleState(wl)
    for inp in (wl.tokens_before_step(0),):
        staging.append_tokens(cfg, pools, inp, s.dtype, DEV)
        staging.append_tokens(cfg, fpools, inp, s.dtype, DEV)
        orc.append(inp)
    for step in range(6):
        d = wl.decode_step(step)
        staging.append_tokens(cfg, pools, d, s.dtype, DEV)
        staging.append_tokens(cfg, fpools, d, s.dtype, DEV)
        orc.append(d)
        if step in (0, 5):
            ref = orc.decode(d, inv_freq=table)
            ref = np.stack([ref[r] for r in range(len(ref))])
            out = gpu_f64(staging.DecodeCall(cfg, s, d, DEV).run(pools))
            mx, mn = assert_parity(out, ref, "bf16", f"{variant} decode {step}")
            fout = gpu_f64(staging.DecodeCall(cfg, s, d, DEV, framed=True).run(fpools))
            fmx, fmn = assert_parity(fout, ref, "bf16", f"{variant} framed decode {step}")
            say(f"{variant} decode step {step}: max {mx:.2e} mean {mn:.2e}; framed max {fmx:.2e} mean {fmn:.2e}")


# ---------------------------------------------------------------------------
# FP8 (e4m3) pools: bytes bit-exact with the oracle's quantiser, attention
# against the oracle over the dequantised values
# ---------------------------------------------------------------------------
def test_fp8_append_bit_exact():
    say("FP8 append: 8B documents and query tokens quantised by lazyattn_append_kv")
    wl = W.build_workload(W.spec(2, requests=[2]))
    s = wl.spec
    cfg = staging.config_for(s, kv_format="fp8")
    pools = staging.WrittenPools(wl, cfg, DEV)
    pb = wl.prefill_batch()
    staging.append_tokens(cfg, pools, pb, s.dtype, DEV)
    sync()
    orc = OracleFp8State(wl)
    orc.append(pb)
    blocks = np.unique(np.concatenate([wl.doc_blocks(int(d)) for d in wl.referenced_docs] + [pb["slots"] // 16]))
    bi = torch.from_numpy(blocks).to(DEV)
    gk, gv = pools.k[bi].cpu().numpy(), pools.v[bi].cpu().numpy()
    assert np.array_equal(gk, orc.kc[blocks]), f"K chunks differ in {int(np.sum(gk != orc.kc[blocks]))} bytes"
    assert np.array_equal(gv, orc.vc[blocks]), f"V chunks differ in {int(np.sum(gv != orc.vc[blocks]))} bytes"
    say(f"FP8 append: {blocks.size} blocks x {s.num_kv_heads} heads bit-exact")


@pytest.mark.parametrize("pe,num_splits,exact", [("rope", 0, False), ("rope", 1, False), ("rope", 0, True),
                                                  ("none", 0, False), ("alibi", 0, False)])
def test_fp8_prefill_llama8b(pe, num_splits, exact):
    say(f"FP8 prefill: 8B, 4 requests, pe={pe} splits={num_splits} exact_max={exact}")
    wl = W.build_workload(W.spec(2, requests=[4]))
    s = wl.spec
    cfg = staging.config_for(s, pe=pe, exact_max=exact, kv_format="fp8")
    pools = staging.WrittenPools(wl, cfg, DEV)
    pb = wl.prefill_batch()
    staging.append_tokens(cfg, pools, pb, s.dtype, DEV)
    got = gpu_f64(staging.PrefillCall(cfg, s, pb, DEV, num_splits).run(pools))
    orc = OracleFp8State(wl)
    orc.append(pb)
    ref = orc.prefill(pb, pe=pe)
    cu = pb["cu_q_lens"]
    mx, mn = assert_parity(np.concatenate([got[cu[r]:cu[r + 1]] for r in ref]), np.concatenate([ref[r] for r in ref]),
                           "bf16", f"FP8 8B prefill {pe}")
    say(f"FP8 8B prefill {pe} splits={num_splits} exact={exact}: max {mx:.2e} mean {mn:.2e}")


def test_fp8_prefill_mqa_sampled():
    say("FP8 prefill: MQA (G = 32), 8 requests, sampled rows")
    wl = W.build_workload(W.spec(5, requests=[8, 0], skew=0.8))
    s = wl.spec
    cfg = staging.config_for(s, kv_format="fp8")
    pools = staging.WrittenPools(wl, cfg, DEV)
    pb = wl.prefill_batch()
    staging.append_tokens(cfg, pools, pb, s.dtype, DEV)
    got = gpu_f64(staging.PrefillCall(cfg, s, pb, DEV).run(pools))
    orc = OracleFp8State(wl)
    orc.append(pb)
    rng = np.random.default_rng(4)
    subset = {r: sample_tokens(128, 12, rng) for r in range(len(pb["ctx_lens"]))}
    ref = orc.prefill(pb, token_subset=subset)
    cu = pb["cu_q_lens"]
    g = np.concatenate([got[cu[r] + subset[r]] for r in ref])
    mx, mn = assert_parity(g, np.concatenate([ref[r] for r in ref]), "bf16", "FP8 MQA prefill")
    say(f"FP8 MQA prefill: max {mx:.2e} mean {mn:.2e}")


def test_fp8_edge_single_token_contexts_and_zero_rows():
    say("FP8 edge: requests without documents (one-token contexts), then all-zero K/V rows")
    wl = W.build_workload(W.spec(2, requests=[3], docs=(0, 0), q_len=1, n_decode=2))
    s = wl.spec
    cfg = staging.config_for(s, kv_format="fp8")
    pools = staging.WrittenPools(wl, cfg, DEV)
    orc = OracleFp8State(wl)
    pb = wl.prefill_batch()
    # token 1 of the batch: K and V rows all zero (exponent 0, every code +0)
    pb = dict(pb, k_new=pb["k_new"].copy(), v_new=pb["v_new"].copy())
    pb["k_new"][1] = 0
    pb["v_new"][1] = 0
    staging.append_tokens(cfg, pools, pb, s.dtype, DEV)
    orc.append(pb)
    got = gpu_f64(staging.PrefillCall(cfg, s, pb, DEV).run(pools))
    ref = orc.prefill(pb)
    cu = pb["cu_q_lens"]
    assert_parity(np.concatenate([got[cu[r]:cu[r + 1]] for r in ref]), np.concatenate([ref[r] for r in ref]),
                  "bf16", "FP8 one-token contexts")
    np.testing.assert_array_equal(got[1], 0.0)      # the zero token attends only to itself
    for step in range(2):
        d = wl.decode_step(step)
        staging.append_tokens(cfg, pools, d, s.dtype, DEV)
        orc.append(d)
    out = gpu_f64(staging.DecodeCall(cfg, s, d, DEV).run(pools))
    ref = orc.decode(d)
    mx, mn = assert_parity(out, np.stack([ref[r] for r in range(len(ref))]), "bf16", "FP8 decode after zero rows")
    say(f"FP8 edge decode: max {mx:.2e} mean {mn:.2e}")


def test_fp8_framed_pool_append_prefill_and_decode():
    say("FP8 pool in document-local frames: append (vs exact rotation), 8B prefill and decode")
    wl = W.build_workload(W.spec(3, requests=[6], n_decode=3))
    s = wl.spec
    cfg = staging.config_for(s, kv_format="fp8")
    pools = staging.FramedPools(wl, cfg, DEV)
    sync()
    # appended chunks: every value within half a code step (or half a subnormal step) of the
    # exact R(j) k, and almost every code equal to the oracle's (float rounding of the rotation
    # may move a value across a rounding boundary)
    orc = OracleFp8State(wl, framed=True)
    d0 = int(wl.referenced_docs[0])
    k, _ = wl.doc_kv(d0)
    slots, j = wl.doc_frame_tokens(d0)
    exact = O.rotate_into_frames(O.bf16_to_f64(k), j, O.rope_inv_freq(s.head_dim, s.rope_theta))
    blocks = np.unique(slots // 16)
    got = O.Fp8PoolView(pools.k[torch.from_numpy(blocks).to(DEV)].cpu().numpy(), "k")[np.arange(blocks.size)]
    pos = {int(b): i for i, b in enumerate(blocks)}
    g = np.stack([got[pos[int(sl // 16)], :, int(sl % 16), :] for sl in slots])
    _, exps = O.quantize_fp8_rows(exact.astype(np.float32))
    bound = np.maximum(2.0 ** -4 * np.abs(exact), np.ldexp(1.0, exps.astype(np.int32) - 10)[..., None]) * (1 + 1e-5)
    assert np.all(np.abs(g - exact) <= bound + 1e-30)
    gb = pools.k[torch.from_numpy(blocks).to(DEV)].cpu().numpy()
    same = float(np.mean(gb == orc.kc[blocks]))
    say(f"framed FP8 append: {same:.5f} of the K chunk bytes equal the oracle's")
    assert same >= 0.99
    # prefill and decode against the oracle over its own framed FP8 pool
    pb = wl.prefill_batch()
    staging.append_tokens(cfg, pools, pb, s.dtype, DEV)
    orc.append(pb)
    got = gpu_f64(staging.PrefillCall(cfg, s, pb, DEV, framed=True).run(pools))
    ref = orc.prefill(pb)
    cu = pb["cu_q_lens"]
    mx, mn = assert_parity(np.concatenate([got[cu[r]:cu[r + 1]] for r in ref]), np.concatenate([ref[r] for r in ref]),
                           "bf16", "framed FP8 prefill")
    say(f"framed FP8 prefill: max {mx:.2e} mean {mn:.2e}")
    for step in range(3):
        d = wl.decode_step(step)
        staging.append_tokens(cfg, pools, d, s.dtype, DEV)
        orc.append(d)
    out = gpu_f64(staging.DecodeCall(cfg, s, d, DEV, framed=True).run(pools))
    ref = orc.decode(d)
    mx, mn = assert_parity(out, np.stack([ref[r] for r in range(len(ref))]), "bf16", "framed FP8 decode")
    say(f"framed FP8 decode step 2: max {mx:.2e} mean {mn:.2e}")


@pytest.mark.parametrize("hq,fmt,framed,pe", [(24, "plain", False, "rope"), (17, "plain", False, "rope"),
                                              (31, "plain", False, "alibi"), (32, "plain", False, "none"),
                                              (24, "fp8", False, "rope"), (32, "plain", True, "rope"),
                                              (24, "fp8", True, "rope")])
def test_decode_group_halves(hq, fmt, framed, pe):
    # Groups of 17..32 query heads: over a plain content-only pool one wave holds
    # them all as two 16-column tiles (17 heads: the second tile holds 1); over FP8
    # pools and framed batches they decode as two work-groups of 16 heads each over
    # the same entries (24 heads: the second holds 8).  MQA shape, 8 decode
    # requests, step 1, with the heuristic's splits and forced 1 and 5.
    say(f"decode of a group of more than 16 heads: Hq={hq}, Hkv=1, pool {fmt}, framed={framed}, pe={pe}")
    spec = dataclasses.replace(W.spec(5, requests=[0, 8], n_decode=2, skew=1.2), num_q_heads=hq)
    wl = W.build_workload(spec)
    s = wl.spec
    cfg = staging.config_for(s, kv_format=fmt, pe=pe)
    pools = (staging.FramedPools if framed else staging.WrittenPools)(wl, cfg, DEV)
    orc = OracleFp8State(wl, framed=framed) if fmt == "fp8" else OracleState(wl)
    hist = wl.tokens_before_step(0)
    staging.append_tokens(cfg, pools, hist, s.dtype, DEV)
    orc.append(hist)
    for step in range(2):
        d = wl.decode_step(step)
        staging.append_tokens(cfg, pools, d, s.dtype, DEV)
        orc.append(d)
    ref = orc.decode(d) if fmt == "fp8" else orc.decode(d, pe=pe)
    ref = np.stack([ref[r] for r in range(len(ref))])
    for splits in (0, 1, 5):
        call = staging.DecodeCall(cfg, s, d, DEV, num_splits=splits, framed=framed)
        out = gpu_f64(call.run(pools))
        mx, mn = assert_parity(out, ref, "bf16", f"halves Hq={hq} {fmt} framed={framed} pe={pe} splits={splits}")
        say(f"halves Hq={hq} {fmt} framed={framed} pe={pe} splits={call.splits}: max {mx:.2e} mean {mn:.2e}")


def test_fp8_decode_llama8b():
    say("FP8 decode: 8B, 16 requests, steps 0 and 16 (RoPE), step 16 rotation-free and ALiBi")
    wl = W.build_workload(W.spec(3, requests=[16], n_decode=17))
    s = wl.spec
    cfg = staging.config_for(s, kv_format="fp8")
    pools = staging.WrittenPools(wl, cfg, DEV)
    orc = OracleFp8State(wl)
    hist = wl.tokens_before_step(0)
    staging.append_tokens(cfg, pools, hist, s.dtype, DEV)
    orc.append(hist)
    for step in range(17):
        d = wl.decode_step(step)
        staging.append_tokens(cfg, pools, d, s.dtype, DEV)
        orc.append(d)
        if step in (0, 16):
            pes = ("rope",) if step == 0 else ("rope", "none", "alibi")
            for pe in pes:
                c = staging.config_for(s, pe=pe, kv_format="fp8")
                out = gpu_f64(staging.DecodeCall(c, s, d, DEV).run(pools))
                ref = orc.decode(d, pe=pe)
                mx, mn = assert_parity(out, np.stack([ref[r] for r in range(len(ref))]), "bf16",
                                       f"FP8 8B decode {pe} step {step}")
                say(f"FP8 8B decode {pe} step {step}: max {mx:.2e} mean {mn:.2e}")


def test_fp8_decode_long_context_and_mqa():
    say("FP8 decode: 70B 32k step 0 at splits 0 and 7; MQA (G = 32) step 0")
    wl = W.build_workload(W.spec(4, requests=[1], n_decode=1))
    s = wl.spec
    cfg = staging.config_for(s, kv_format="fp8")
    pools = staging.WrittenPools(wl, cfg, DEV)
    orc = OracleFp8State(wl)
    for inp in (wl.prefill_batch(), wl.decode_step(0)):
        staging.append_tokens(cfg, pools, inp, s.dtype, DEV)
        orc.append(inp)
    d = wl.decode_step(0)
    ref = orc.decode(d)
    for splits in (0, 7):
        out = gpu_f64(staging.DecodeCall(cfg, s, d, DEV, num_splits=splits).run(pools))
        mx, mn = assert_parity(out, ref[0][None], "bf16", f"FP8 70B decode splits={splits}")
        say(f"FP8 70B decode splits={splits}: max {mx:.2e} mean {mn:.2e}")
    wl = W.build_workload(W.spec(5, requests=[2, 24], skew=1.2))
    s = wl.spec
    cfg = staging.config_for(s, kv_format="fp8")
    pools = staging.WrittenPools(wl, cfg, DEV)
    orc = OracleFp8State(wl)
    for inp in (wl.tokens_before_step(0), wl.decode_step(0)):
        staging.append_tokens(cfg, pools, inp, s.dtype, DEV)
        orc.append(inp)
    d = wl.decode_step(0)
    out = gpu_f64(staging.DecodeCall(cfg, s, d, DEV).run(pools))
    reqs = list(range(0, len(d["ctx_lens"]), 3))
    ref = orc.decode(d, requests=reqs)
    mx, mn = assert_parity(out[reqs], np.stack([ref[r] for r in reqs]), "bf16", "FP8 MQA decode")
    say(f"FP8 MQA decode: max {mx:.2e} mean {mn:.2e}")


# ---------------------------------------------------------------------------
# negative controls: planted mistakes in the oracle must fail the bar
# ---------------------------------------------------------------------------
def test_negative_controls_fail_the_tolerance():
    say("negative controls (oracle with planted mistakes vs the GPU output)")
    wl = W.build_workload(W.spec(2, requests=[2]))
    pb, got, _ = run_prefill(wl)
    orc = OracleState(wl)
    orc.append(pb)
    cu = pb["cu_q_lens"]
    good = orc.prefill(pb)
    g = np.concatenate([got[cu[r]:cu[r + 1]] for r in good])
    assert within(g, np.concatenate(list(good.values())), "bf16")
    D = wl.spec.head_dim
    half = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])
    for name, bad in (("off by one", orc.prefill(pb, q_shift=1)),
                      ("rotation off", orc.prefill(pb, pe="none")),
                      ("half-split pairs", orc.prefill(pb, pair_perm=half))):
        b = np.concatenate(list(bad.values()))
        mx, mn = diff_stats(g, b)
        say(f"control {name}: max {mx:.2e} mean {mn:.2e}")
        assert not within(g, b, "bf16"), name


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
def test_edge_single_token_contexts_and_zero_length_queries():
    say("edge: requests without documents (context = the query itself) and zero-length query rows")
    wl = W.build_workload(W.spec(2, requests=[3], docs=(0, 0), q_len=1))
    pb, got, _ = run_prefill(wl)
    orc = OracleState(wl)
    orc.append(pb)
    compare_prefill(wl, pb, got, orc, label="single-token contexts")
    # add a request with no new tokens in the middle of the batch
    wl2 = W.build_workload(W.spec(2, requests=[3], q_len=5))
    s = wl2.spec
    cfg = staging.config_for(s)
    pb2 = wl2.prefill_batch()
    pools = staging.DevicePools(wl2, DEV)
    staging.append_tokens(cfg, pools, pb2, s.dtype, DEV)
    orc2 = OracleState(wl2)
    orc2.append(pb2)
    ref = orc2.prefill(pb2)
    ins = dict(pb2)
    # request 1 contributes nothing this call: its context ends before its new tokens
    ins["cu_q_lens"] = np.array([0, 5, 5, 10], dtype=np.int32)
    ins["q"] = np.concatenate([pb2["q"][0:5], pb2["q"][10:15]])
    ins["total_q"] = 10
    ctx = pb2["ctx_lens"].copy()
    ctx[1] -= 5
    ins["ctx_lens"] = ctx
    ne = pb2["num_entries"].copy()
    ne[1] = wl2.requests[1].n_doc_entries
    ins["num_entries"] = ne
    out = gpu_f64(staging.PrefillCall(cfg, s, ins, DEV).run(pools))
    assert_parity(out[0:5], ref[0], "bf16", "zero-length row: request 0")
    assert_parity(out[5:10], ref[2], "bf16", "zero-length row: request 2")


def test_split_workspace_reuse_across_calls_of_different_sizes():
    say("one workspace reused by split prefill and decode calls of different sizes")
    wl = W.build_workload(W.spec(4, requests=[2], n_decode=1, q_len=100))
    s = wl.spec
    cfg = staging.config_for(s)
    pools = staging.DevicePools(wl, DEV)
    pb = wl.prefill_batch()
    staging.append_tokens(cfg, pools, pb, s.dtype, DEV)
    d = wl.decode_step(0)
    staging.append_tokens(cfg, pools, d, s.dtype, DEV)
    orc = OracleState(wl)
    orc.append(pb)
    ref_p = orc.prefill(pb, token_subset={0: [0, 99], 1: [0, 50, 99]})
    orc.append(d)
    ref_d = orc.decode(d)
    big = max([_abi.prefill_workspace_size(cfg, 2, pb["total_q"], pb["max_q_len"], pb["table_blocks"].shape[1], k)
               for k in (9, 3, 17)] + [_abi.decode_workspace_size(cfg, 2, d["table_blocks"].shape[1], k)
                                       for k in (50, 4)])
    ws = torch.zeros(big, dtype=torch.uint8, device=DEV)
    pc = staging.PrefillCall(cfg, s, pb, DEV)
    dc = staging.DecodeCall(cfg, s, d, DEV)
    for rep in range(2):
        for k in (9, 3, 17):
            _abi.prefill(cfg, pc.q, pc.cu_q, pc.total_q, pc.max_q_len, pools.k, pools.v, pools.num_blocks,
                         pc.tables.batch, pc.out, ws, k)
            got = gpu_f64(pc.out)
            for r, toks in ((0, [0, 99]), (1, [0, 50, 99])):
                assert_parity(got[pb["cu_q_lens"][r] + np.array(toks)], ref_p[r], "bf16", f"prefill splits {k}")
            for kd in (50, 4):
                _abi.decode(cfg, dc.q, pools.k, pools.v, pools.num_blocks, dc.tables.batch, dc.out, ws, kd)
                out = gpu_f64(dc.out)
                assert_parity(out, np.stack([ref_d[0], ref_d[1]]), "bf16", f"decode splits {kd}")
    sync()


def test_attend_then_merge_equals_single_call():
    say("attend + merge as two calls == one prefill call; decode likewise")
    wl = W.build_workload(W.spec(2, requests=[3]))
    s = wl.spec
    cfg = staging.config_for(s)
    pools = staging.DevicePools(wl, DEV)
    pb = wl.prefill_batch()
    staging.append_tokens(cfg, pools, pb, s.dtype, DEV)
    for k in (1, 3):
        one = staging.PrefillCall(cfg, s, pb, DEV, num_splits=k)
        two = staging.PrefillCall(cfg, s, pb, DEV, num_splits=k)
        a = gpu_f64(one.run(pools))
        two.attend(pools)
        two.merge()
        assert np.array_equal(a, gpu_f64(two.out))
    wl2 = W.build_workload(W.spec(4, requests=[1], n_decode=1))
    pools2 = staging.DevicePools(wl2, DEV)
    staging.append_tokens(cfg, pools2, wl2.tokens_before_step(0), s.dtype, DEV)
    d = wl2.decode_step(0)
    staging.append_tokens(cfg, pools2, d, s.dtype, DEV)
    cfg4 = staging.config_for(wl2.spec)
    one = staging.DecodeCall(cfg4, wl2.spec, d, DEV, num_splits=9)
    two = staging.DecodeCall(cfg4, wl2.spec, d, DEV, num_splits=9)
    a = gpu_f64(one.run(pools2))
    two.attend(pools2)
    two.merge()
    assert np.array_equal(a, gpu_f64(two.out))


def test_split_partials_hold_large_values_within_half_range():
    # split partials are stored as IEEE half: values up to |v| <= 65504 must come
    # through a split call intact.  V scaled by 2^13 (exact in bf16; |v| up to ~4e4):
    # the output scales by exactly 2^13, so it is checked against the unscaled oracle
    say("large |V| (x 2^13) through split prefill and decode: splits 1 vs several vs the oracle")
    wl = W.build_workload(W.spec(2, requests=[2], n_decode=1))
    s = wl.spec
    cfg = staging.config_for(s)
    pools = staging.DevicePools(wl, DEV)
    pb = wl.prefill_batch()
    staging.append_tokens(cfg, pools, pb, s.dtype, DEV)
    orc = OracleState(wl)
    orc.append(pb)
    ref = orc.prefill(pb)
    pools.v.mul_(8192.0)
    vmax = float(torch.nan_to_num(pools.v.float(), nan=0.0).abs().max())
    assert 8192.0 < vmax <= 65504.0
    outs = {}
    for k in (1, 5):
        outs[k] = gpu_f64(staging.PrefillCall(cfg, s, pb, DEV, num_splits=k).run(pools)) / 8192.0
        cu = pb["cu_q_lens"]
        assert_parity(outs[k], np.concatenate([ref[r] for r in range(2)]), "bf16", f"large-V prefill splits={k}")
    mx, mn = diff_stats(outs[5], outs[1])
    assert mx <= 4e-3 and mn <= 2e-4
    d = wl.decode_step(0)
    dk = {key: d[key] for key in ("k_new", "v_new", "slots")}
    orc.append(dk)
    ref_d = orc.decode(d)
    staging.append_tokens(cfg, pools, {"k_new": d["k_new"], "v_new": d["v_new"], "slots": d["slots"]}, s.dtype, DEV)
    # the new token's value row is appended unscaled; scale that slot too
    slots = torch.from_numpy(d["slots"]).to(DEV)
    pools.v[slots // 16, :, :, slots % 16] *= 8192.0
    for k in (1, 7):
        out = gpu_f64(staging.DecodeCall(cfg, s, d, DEV, num_splits=k).run(pools)) / 8192.0
        assert_parity(out, np.stack([ref_d[r] for r in range(2)]), "bf16", f"large-V decode splits={k}")
