"""The block pool manager (native, through the C interface) against the oracle's cache model (CPU only)."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from position_agnostic_kv_pool_amd import _abi

POLICIES = ("agnostic", "aware", "prefix")


def _requests(ids, lens, offs):
    return [(ids[offs[i]:offs[i + 1]], lens[offs[i]:offs[i + 1]]) for i in range(offs.size - 1)]


# ---------------------------------------------------------------------------
# pins of the oracle's cache model
# ---------------------------------------------------------------------------
def test_oracle_hand_trace_lru():
    # budget 2 blocks, one-block documents A B A C B A:
    # A miss, B miss, A hit (LRU order B, A), C evicts B, B evicts A, A evicts C
    c = O.BlockCache(2, "agnostic")
    got = []
    for d in "ABACBA":
        st, bl, _, t = c.admit([ord(d)], [16])
        got.append((st[0], bl))
        c.release(t)
    assert [g[0] for g in got] == [0, 0, 1, 0, 0, 0]
    assert [g[1] for g in got] == [[0], [1], [0], [1], [0], [1]]
    assert c.stats["doc_hits"] == 1 and c.stats["evictions"] == 3


def test_oracle_unlimited_budget_closed_form():
    ids, lens, offs = W.cache_trace(200, 300, (2, 6), 1.1, seed=3)
    reqs = _requests(ids, lens, offs)
    big = int(((lens + 15) // 16).sum()) + 1
    distinct = {"agnostic": len(set(ids.tolist())), "aware": set(), "prefix": set()}
    for d, l in reqs:
        pos = 0
        for k in range(len(d)):
            distinct["aware"].add((int(d[k]), pos))
            distinct["prefix"].add(tuple(int(x) for x in d[:k + 1]))
            pos += int(l[k])
    for pol in POLICIES:
        st = O.BlockCache(big, pol).run(reqs)
        n_keys = distinct[pol] if isinstance(distinct[pol], int) else len(distinct[pol])
        assert st["doc_hits"] == ids.size - n_keys, pol
        assert st["evictions"] == 0 and st["bypasses"] == 0


def test_oracle_zero_budget_and_single_document_requests():
    ids, lens, offs = W.cache_trace(50, 100, (1, 1), 1.0, seed=4)
    reqs = _requests(ids, lens, offs)
    st = O.BlockCache(0, "agnostic").run(reqs)
    assert st["doc_hits"] == 0 and st["bypasses"] == ids.size
    # a document alone at offset 0: the three keys coincide
    runs = [O.BlockCache(64, p).run(reqs) for p in POLICIES]
    assert runs[0] == runs[1] == runs[2]


def test_oracle_agnostic_beats_aware_and_prefix_under_skew():
    ids, lens, offs = W.cache_trace(400, 600, (4, 8), 1.2, seed=5)
    reqs = _requests(ids, lens, offs)
    hits = {p: O.BlockCache(2048, p).run(reqs)["token_hits"] for p in POLICIES}
    assert hits["agnostic"] > 2 * hits["aware"] > 0
    assert hits["aware"] >= hits["prefix"]


# ---------------------------------------------------------------------------
# the native pool manager: bit-exact with the oracle
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("policy", POLICIES)
@pytest.mark.parametrize("budget", [0, 7, 96, 1024])
def test_pool_admit_matches_oracle(policy, budget):
    ids, lens, offs = W.cache_trace(60, 120, (1, 5), 1.0, seed=6, doc_len_lognormal=(40, 0.8, 5, 200))
    orc = O.BlockCache(budget, policy)
    pool = _abi.Pool(budget, policy)
    held = []
    for i, (d, l) in enumerate(_requests(ids, lens, offs)):
        st, bl, sta, t = pool.admit(d, l)
        ost, obl, osta, ot = orc.admit(d, l)
        assert st.tolist() == ost and bl.tolist() == obl and sta.tolist() == osta, i
        held.append((t, ot))
        if i % 3 != 2:                       # keep up to three requests open at a time
            for a, b in held:
                pool.release(a)
                orc.release(b)
            held = []
    for a, b in held:
        pool.release(a)
        orc.release(b)
    s = pool.stats()
    for k, v in orc.stats.items():
        assert s[k] == v, k
    assert s["blocks_in_use"] == orc.blocks_in_use() and s["open_requests"] == 0


@pytest.mark.parametrize("policy", POLICIES)
def test_pool_trace_runner_matches_oracle(policy):
    ids, lens, offs = W.cache_trace(500, 1500, (4, 10), 1.2, seed=7)
    for budget in (256, 2048):
        pool = _abi.Pool(budget, policy)
        pool.run_trace(ids, lens, offs)
        ref = O.BlockCache(budget, policy).run(_requests(ids, lens, offs))
        s = pool.stats()
        for k, v in ref.items():
            assert s[k] == v, (policy, budget, k)


def test_pool_rejects_bad_arguments():
    lib = _abi.lib()
    import ctypes
    h = ctypes.c_void_p()
    assert lib.lazyattn_pool_create(-1, 0, ctypes.byref(h)) == _abi.EINVAL
    assert lib.lazyattn_pool_create(8, 3, ctypes.byref(h)) == _abi.EINVAL
    pool = _abi.Pool(8)
    with pytest.raises(_abi.LazyAttnError):
        pool.admit([1, -2], [16, 16])
    with pytest.raises(_abi.LazyAttnError):
        pool.admit([1], [0])
    with pytest.raises(_abi.LazyAttnError):
        pool.release(12345)
    # entries that do not fit max_entries leave the pool unchanged
    ids = np.array([1, 2], dtype=np.int64)
    lens = np.array([40, 40], dtype=np.int32)
    b = np.empty(8, np.uint32)
    s = np.empty(8, np.uint32)
    st = np.empty(2, np.uint8)
    ne, t = ctypes.c_int32(), ctypes.c_int64()
    assert lib.lazyattn_pool_admit(pool._h, ids.ctypes.data, lens.ctypes.data, 2, b.ctypes.data, s.ctypes.data, 5,
                                   ctypes.byref(ne), st.ctypes.data, ctypes.byref(t)) == _abi.EWORKSPACE
    assert pool.stats()["doc_accesses"] == 0
