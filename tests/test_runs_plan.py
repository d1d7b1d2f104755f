"""The shared-run decode plan (lazyattn_decode_runs_plan), host only.

The plan must cover every entry of every request exactly once, with the
positions the kernel will give its keys; these tests rebuild each request's
table from the plan and compare it with the input, and check the bounds the
kernel relies on (occurrences per item, entries per item, a multiple of 32
items) and the per-request occurrence lists the merge reads.
"""
import numpy as np
import pytest

import workloads as W
from position_agnostic_kv_pool_amd import _abi


def _cfg(hq=32, hkv=8, dtype="bf16"):
    return _abi.make_config(hq, hkv, 128, dtype=dtype, pe="rope", rope_theta=5e5)


def _tables(blocks_per_req, lens_per_req):
    """Host tables from per-request block lists and valid lengths (starts are the prefix sums)."""
    R = len(blocks_per_req)
    E = max(1, max(len(b) for b in blocks_per_req))
    tb = np.zeros((R, E), dtype=np.uint32)
    ts = np.zeros((R, E), dtype=np.uint32)
    ne = np.zeros(R, dtype=np.int32)
    ctx = np.zeros(R, dtype=np.int32)
    for r, (bl, ln) in enumerate(zip(blocks_per_req, lens_per_req)):
        pos = 0
        for e, (b, l) in enumerate(zip(bl, ln)):
            tb[r, e] = b
            ts[r, e] = pos
            pos += l
        ne[r] = len(bl)
        ctx[r] = pos
    return _abi.pack_entries(tb, ts), ne, ctx


def _entries(words, ne, ctx):
    """Per request: sorted (start, block, length) of its table."""
    out = []
    for r in range(len(ne)):
        row = []
        for e in range(int(ne[r])):
            w = int(words[r, e])
            s, b = w >> 32, w & 0xffffffff
            end = (int(words[r, e + 1]) >> 32) if e + 1 < ne[r] else int(ctx[r])
            row.append((s, b, end - s))
        out.append(sorted(row))
    return out


def _check_plan(cfg, words, ne, ctx, num_blocks):
    plan = _abi.decode_runs_plan(cfg, words, ne, ctx, num_blocks)
    items, wds, refs = plan["items"], plan["words"], plan["refs"]
    begin, rrefs = plan["req_ref_begin"], plan["req_refs"]
    G = cfg.num_q_heads // cfg.num_kv_heads
    R = len(ne)
    assert items.shape[0] % 32 == 0
    got = [[] for _ in range(R)]
    seen_refs = set()
    for it in items:
        w0, n, ref0, nref = (int(x) for x in it)
        if n == 0:
            assert nref == 0
            continue
        # shared pieces: at most 64 entries and 16 / G occurrences; a request's own: 128 and one
        assert 1 <= nref <= max(1, 16 // G) and 1 <= n <= (64 if nref > 1 else 128)
        ent = [(int(w) & 0xffffffff, (int(w) >> 32) & 0x7ffffff, int(w) >> 59) for w in wds[w0:w0 + n]]
        assert all(1 <= l <= 16 for _, _, l in ent)
        for j in range(ref0, ref0 + nref):
            assert j not in seen_refs
            seen_refs.add(j)
            rq, turn = int(refs[j, 0]), int(refs[j, 1])
            s = int(ctx[rq]) - 1 - turn                     # the item's key base in request rq
            for b, o, l in ent:
                got[rq].append((s + o, b, l))
    assert seen_refs == set(range(refs.shape[0]))
    assert [sorted(g) for g in got] == _entries(words, ne, ctx)
    # the merge's lists: request r's occurrences, each once, in ascending order
    assert begin[0] == 0 and begin[-1] == refs.shape[0] and np.all(np.diff(begin) >= 0)
    for r in range(R):
        mine = rrefs[begin[r]:begin[r + 1]]
        assert list(mine) == sorted(np.nonzero(refs[:, 0] == r)[0].tolist())
    return plan


def test_plan_covers_the_decode_batches_once():
    for cid in (3, 4):
        wl = W.build_workload(W.spec(cid, n_decode=1) if cid == 3 else W.spec(4, n_decode=1))
        d = wl.decode_step(0)
        words = _abi.pack_entries(d["table_blocks"], d["table_starts"])
        s = wl.spec
        plan = _check_plan(_cfg(s.num_q_heads, s.num_kv_heads), words, d["num_entries"], d["ctx_lens"],
                           wl.num_blocks)
        # every distinct (block, length) is read by one run piece: the words are exactly those
        keys = {(int(w) & 0xffffffff, l) for row in _entries(words, d["num_entries"], d["ctx_lens"])
                for (_, b, l) in row for w in [b]}
        assert len(plan["words"]) == len(keys)
        if cid == 3:   # shared documents: far fewer block reads than table entries
            assert len(plan["words"]) < 0.5 * int(np.sum(d["num_entries"]))


def test_plan_edge_cases():
    cfg = _cfg()
    # a document twice in one request, a shared partial block with two lengths,
    # a one-entry request, an empty request, a block both whole and partial
    reqs = [
        ([1, 2, 3, 1, 2, 3, 9], [16, 16, 5, 16, 16, 5, 3]),
        ([1, 2, 3, 7], [16, 16, 5, 1]),
        ([1, 2, 3], [16, 16, 11]),
        ([4], [7]),
        ([], []),
        ([4, 5], [16, 2]),
    ]
    words, ne, ctx = _tables([b for b, _ in reqs], [l for _, l in reqs])
    plan = _check_plan(cfg, words, ne, ctx, 16)
    # request 4 has no entries: no occurrence
    assert plan["req_ref_begin"][4] == plan["req_ref_begin"][5]
    # a request's entries held by no other request: one item with one occurrence
    own = [(list(range(10, 40)), [16] * 10 + [5] + [16] * 18 + [7]), ([1, 2], [16, 3]), ([1, 2], [16, 3])]
    words, ne, ctx = _tables([b for b, _ in own], [l for _, l in own])
    plan = _check_plan(cfg, words, ne, ctx, 64)
    req0 = [it for it in plan["items"] if it[1] > 0 and plan["refs"][it[2], 0] == 0]
    assert len(req0) == 1 and req0[0][1] == 30 and req0[0][3] == 1
    # many occurrences of one run split over items of at most 16 / G
    many = [([1, 2], [16, 4])] * 23
    words, ne, ctx = _tables([b for b, _ in many], [l for _, l in many])
    plan = _check_plan(cfg, words, ne, ctx, 4)
    assert sum(1 for it in plan["items"] if it[1] > 0) == (23 + 3) // 4
    # a long shared run is cut into pieces of at most 64 entries
    long = [(list(range(150)), [16] * 149 + [9])] * 2
    words, ne, ctx = _tables([b for b, _ in long], [l for _, l in long])
    plan = _check_plan(cfg, words, ne, ctx, 200)
    assert sorted(int(it[1]) for it in plan["items"] if it[1] > 0) == [22, 64, 64]


def test_plan_errors():
    words, ne, ctx = _tables([[1, 2]], [[16, 3]])
    with pytest.raises(_abi.LazyAttnError) as e:
        _abi.decode_runs_plan(_cfg(32, 1), words, ne, ctx, 4)           # G = 32
    assert e.value.status == _abi.EUNSUPPORTED
    with pytest.raises(_abi.LazyAttnError) as e:
        _abi.decode_runs_plan(_cfg(), words, ne, ctx, 2)                # block 2 outside a 2-block pool
    assert e.value.status == _abi.EINVAL
    bad = words.copy()
    bad[0, 1] = _abi.pack_entries(np.array([2], np.uint32), np.array([20], np.uint32))[0]   # length 20 > 16
    with pytest.raises(_abi.LazyAttnError):
        _abi.decode_runs_plan(_cfg(), bad, ne, ctx, 4)
    # capacities too small: sizes come back, arrays untouched
    import ctypes
    ni, nw, nr = ctypes.c_int32(-1), ctypes.c_int32(-1), ctypes.c_int32(-1)
    st = _abi.lib().lazyattn_decode_runs_plan(ctypes.byref(_cfg()), words.ctypes.data, 1, words.shape[1],
                                             ne.ctypes.data, ctx.ctypes.data, 4, 0, 0, 0, None, None, None, None,
                                             None, ctypes.byref(ni), ctypes.byref(nw), ctypes.byref(nr))
    assert st == _abi.EWORKSPACE and ni.value == 32 and nw.value == 2 and nr.value == 1
    assert _abi.decode_runs_workspace_size(_cfg(), 3) == 3 * 32 * (128 * 2 + 8)


def test_decode_runs_rejects_bad_arguments_before_launch():
    import ctypes
    lib = _abi.lib()
    P = ctypes.c_void_p(64)
    plan = _abi.RunPlan()
    plan.num_items, plan.num_words, plan.num_refs = 32, 4, 2
    plan.items = plan.words = plan.refs = plan.req_ref_begin = plan.req_refs = 64   # never dereferenced on the host
    c = _cfg()
    call = lambda cfg, pl, ws, nws: lib.lazyattn_decode_runs(ctypes.byref(cfg), P, P, P, 8, 2, pl, P, ws, nws, None)
    need = _abi.decode_runs_workspace_size(c, 2)
    assert call(c, None, P, need) == _abi.EINVAL                                   # no plan
    assert call(c, ctypes.byref(plan), None, 0) == _abi.EWORKSPACE                 # no room for the partials
    assert call(c, ctypes.byref(plan), P, need - 1) == _abi.EWORKSPACE
    assert call(_cfg(32, 1), ctypes.byref(plan), P, need) == _abi.EUNSUPPORTED      # G = 32
    odd = _abi.RunPlan()
    odd.num_items, odd.num_words, odd.num_refs = 8, 4, 2                          # not a multiple of 32
    odd.items = odd.words = odd.refs = odd.req_ref_begin = odd.req_refs = 64
    assert call(c, ctypes.byref(odd), P, need) == _abi.EINVAL
    plan.req_ref_begin = None
    assert call(c, ctypes.byref(plan), P, need) == _abi.EINVAL
    empty = _abi.RunPlan()                                                        # no requests: nothing to do
    assert lib.lazyattn_decode_runs(ctypes.byref(c), P, P, P, 8, 0, ctypes.byref(empty), P, None, 0, None) == _abi.OK
