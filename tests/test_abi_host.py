"""The C interface on the host: exports, codec, validator, sizing and argument errors (CPU only).

Only entry points that return before touching a GPU are called here.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from position_agnostic_kv_pool_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lazyattn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lazyattn_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 15
    L = _abi.lib()
    for n in names:
        assert hasattr(L, n), n
        getattr(L, n)          # resolves the symbol


def test_version_and_status_strings():
    assert _abi.lib().lazyattn_abi_version() == 9
    for s in range(5):
        assert len(_abi.status_string(s)) > 0
    assert _abi.status_string(99) == "unknown status"


def test_codec_matches_oracle_bit_exact():
    L = _abi.lib()
    rng = np.random.default_rng(0)
    b = np.concatenate([[0, 0xFFFFFFFF, 1, 0], rng.integers(0, 2**32, 5000)]).astype(np.uint32)
    s = np.concatenate([[0, 0xFFFFFFFF, 0, 1], rng.integers(0, 2**32, 5000)]).astype(np.uint32)
    lib_words = _abi.pack_entries(b, s)
    orc_words = O.pack_table(b, s)
    assert np.array_equal(lib_words, orc_words)
    for i in range(0, b.size, 251):
        w = int(lib_words[i])
        assert L.lazyattn_pack(int(b[i]), int(s[i])) == w
        assert (L.lazyattn_entry_block(w), L.lazyattn_entry_start(w)) == O.unpack_entry(w)


def _cfg(**kw):
    d = dict(num_q_heads=4, num_kv_heads=2, head_dim=128, dtype="bf16", pe="rope", rope_theta=10000.0)
    d.update(kw)
    return _abi.make_config(**d)


def _tables(rows):
    """rows: list of lists of (block, start)."""
    E = max(len(r) for r in rows)
    t = np.zeros((len(rows), E), dtype=np.uint64)
    for i, r in enumerate(rows):
        for e, (b, s) in enumerate(r):
            t[i, e] = O.pack_entry(b, s)
    return t


def test_validator_accepts_dense_tables():
    t = _tables([[(3, 0), (1, 16), (2, 20)], [(0, 0)]])
    st, br, be = _abi.validate_tables(_cfg(), t, [3, 1], [30, 5], 4)
    assert (st, br, be) == (_abi.OK, -1, -1)


@pytest.mark.parametrize("case,want", [
    ("start0", (1, 0)), ("too_long", (1, 1)), ("empty_entry", (1, 1)), ("block_oob", (1, 1)),
    ("descending", (1, 1)), ("ctx_short", (1, 2)), ("count_too_big", (1, -1)), ("empty_with_ctx", (1, -1)),
])
def test_validator_rejects_with_location(case, want):
    good = [(0, 0), (1, 16), (2, 20)]
    L, n = 30, 3
    if case == "start0":
        good[0] = (0, 1)
    elif case == "too_long":
        good[2] = (2, 33); L = 50
    elif case == "empty_entry":
        good[2] = (2, 16)
    elif case == "block_oob":
        good[1] = (10, 16)
    elif case == "descending":
        good[2] = (2, 10)
    elif case == "ctx_short":
        L = 20
    elif case == "count_too_big":
        n = 4
    elif case == "empty_with_ctx":
        n = 0
    t = _tables([[(0, 0)], good])
    st, br, be = _abi.validate_tables(_cfg(), t, [1, n], [5, L], 10)
    assert st == _abi.EINVAL
    assert (br, be) == want
    # the oracle's decoder agrees that the table is malformed
    if n <= 3 and n > 0:
        with pytest.raises(O.TableError):
            O.decode_table([int(w) for w in t[1]], n, L, 16, 10)


def test_validator_on_generated_workloads():
    import workloads as W
    for cfg_id in (1, 2, 5):
        wl = W.build_workload(W.spec(cfg_id))
        pb = wl.prefill_batch()
        words = _abi.pack_entries(pb["table_blocks"], pb["table_starts"])
        cfg = _abi.make_config(wl.spec.num_q_heads, wl.spec.num_kv_heads, wl.spec.head_dim, wl.spec.dtype)
        st, _, _ = _abi.validate_tables(cfg, words, pb["num_entries"], pb["ctx_lens"], wl.num_blocks)
        assert st == _abi.OK


def test_config_errors():
    C = _cfg
    lib = _abi.lib()
    check = lambda c: lib.lazyattn_validate_tables(ctypes.byref(c), None, 0, 0, None, None, 0, None, None)
    assert check(C()) == _abi.OK
    assert check(C(num_q_heads=6, num_kv_heads=4)) == _abi.EINVAL
    assert check(C(num_kv_heads=0)) == _abi.EINVAL
    assert check(C(head_dim=64)) == _abi.EUNSUPPORTED            # bf16 kernels are built for D = 128
    assert check(C(head_dim=64, dtype="f32")) == _abi.OK
    assert check(C(block_size=32)) == _abi.EUNSUPPORTED
    assert check(C(rope_theta=0.0)) == _abi.EINVAL
    assert check(C(rope_theta=0.0, pe="none")) == _abi.OK
    c = C(); c.flags = _abi.FLAG_EXACT_MAX
    assert check(c) == _abi.OK
    c = C(); c.flags = _abi.FLAG_KEYS_FUSED | _abi.FLAG_EXACT_MAX
    assert check(c) == _abi.OK
    c = C(); c.flags = _abi.FLAG_KEYS_FUSED | _abi.FLAG_KEYS_ONCE
    assert check(c) == _abi.EINVAL
    c = C(); c.flags = 8
    assert check(c) == _abi.EINVAL
    c = C(); c.dtype = 7
    assert check(c) == _abi.EINVAL
    c = C(); c.pe = 9
    assert check(c) == _abi.EINVAL
    assert check(C(softmax_scale=-1.0)) == _abi.EINVAL


def test_split_heuristics_and_workspace_sizes():
    c = _cfg(num_q_heads=32, num_kv_heads=8)
    # 16 requests x 8 KV heads of one 64-position tile -> too few work-groups: split the keys
    s = _abi.prefill_splits(c, 16, 64, 260)
    assert s == 2
    assert _abi.prefill_workspace_size(c, 16, 1024, 64, 260) == s * 1024 * 32 * (128 * 2 + 8)
    assert _abi.prefill_workspace_size(c, 16, 1024, 64, 260, 1) == 0
    # 128 requests x 8 KV heads is plenty for decode
    assert _abi.decode_splits(c, 128, 274) == 1
    assert _abi.decode_workspace_size(c, 128, 274) == 0
    # the 70B shape: 32 (request, KV head) units -> one round of 16 splits (137 entries each)
    c70 = _cfg(num_q_heads=64, num_kv_heads=8)
    s = _abi.decode_splits(c70, 4, 2184)
    assert s == 16
    assert _abi.decode_workspace_size(c70, 4, 2184) == s * 4 * 64 * (128 * 2 + 8)
    assert _abi.decode_workspace_size(_cfg(dtype="f32", head_dim=64), 4, 100, 8) == 0
    # groups of more than 16 heads decode as two work-groups per (request, KV head,
    # split): 96 MQA requests make 192 of them, so 3 splits fill one round of 512
    # work-groups; 1300 entries would leave splits of 434 entries, so whole rounds
    # more until they hold at most 160: 9
    assert _abi.decode_splits(_cfg(num_q_heads=32, num_kv_heads=1), 96, 1300) == 9
    assert _abi.decode_splits(_cfg(num_q_heads=32, num_kv_heads=1), 96, 600) == 6
    assert _abi.decode_splits(_cfg(num_q_heads=16, num_kv_heads=1), 96, 300) == 6
    assert _abi.decode_splits(_cfg(num_q_heads=16, num_kv_heads=1), 96, 100) == 3   # 6 capped at 100 / 32


def test_keys_once_route_and_its_workspace():
    """The RoPE prefill turns the keys once when a request spans >= 8 query tiles of 256 rows
    (or when asked to); its workspace then holds the turned keys after the partials."""
    turned = lambda R, E, hkv: R * E * hkv * 16 * 128 * 2
    c70 = _cfg(num_q_heads=64, num_kv_heads=8)
    # the 70B chunk: 2048 positions x 8 heads = 64 query tiles per (request, KV head), 1 split
    assert _abi.prefill_splits(c70, 4, 2048, 2176) == 1
    assert _abi.prefill_workspace_size(c70, 4, 8192, 2048, 2176) == turned(4, 2176, 8)
    # 8 tiles (256 positions x 8 heads) turn once, 7 do not
    assert _abi.prefill_workspace_size(c70, 4, 1024, 256, 100, 1) == turned(4, 100, 8)
    assert _abi.prefill_workspace_size(c70, 4, 1024, 224, 100, 1) == 0
    # split partials first, the turned keys from the next 256-byte boundary
    part = 3 * 5 * 64 * (128 * 2 + 8)
    assert _abi.prefill_workspace_size(c70, 1, 5, 256, 300, 3) == (part + 255) // 256 * 256 + turned(1, 300, 8)
    # the flags force either route; other encodings, FP8 pools and f32 never turn once
    fused = _abi.make_config(64, 8, 128, pe="rope", rope_theta=5e5, keys="fused")
    once = _abi.make_config(64, 8, 128, pe="rope", rope_theta=5e5, keys="once")
    assert _abi.prefill_workspace_size(fused, 4, 8192, 2048, 2176) == 0
    assert _abi.prefill_workspace_size(once, 2, 10, 5, 7, 1) == turned(2, 7, 8)
    for kw in (dict(pe="none"), dict(pe="alibi"), dict(kv_format="fp8")):
        c = _abi.make_config(64, 8, 128, rope_theta=5e5, keys="once", **kw)
        assert _abi.prefill_workspace_size(c, 2, 10, 5, 7, 1) == 0
    # MQA (G = 32): 8 positions per tile, so 64 positions make 8 tiles
    cm = _cfg(num_q_heads=32, num_kv_heads=1)
    assert _abi.prefill_workspace_size(cm, 2, 128, 64, 40, 1) == turned(2, 40, 1)
    assert _abi.prefill_workspace_size(cm, 2, 112, 56, 40, 1) == 0
    # both flags at once is no valid config
    both = _abi.make_config(64, 8, 128, rope_theta=5e5)
    both.flags = _abi.FLAG_KEYS_FUSED | _abi.FLAG_KEYS_ONCE
    assert _abi.lib().lazyattn_prefill_splits(ctypes.byref(both), 1, 1, 1) == 0
    assert _abi.prefill_workspace_size(both, 1, 1, 1, 1) == 0
    bad = _abi.make_config(64, 8, 128, rope_theta=5e5)
    bad.flags = 8
    assert _abi.lib().lazyattn_prefill_splits(ctypes.byref(bad), 1, 1, 1) == 0
    # a call on the turned route checks that the workspace holds the turned keys
    lib = _abi.lib()
    b = _abi.Batch()
    b.num_reqs, b.max_entries = 2, 4
    b.block_tables = b.num_entries = b.ctx_lens = 16   # never dereferenced on the host
    P = ctypes.c_void_p(64)
    need = turned(2, 4, 8)
    assert lib.lazyattn_prefill(ctypes.byref(once), P, P, 2, 1, P, P, 1, ctypes.byref(b), 1, P, P, need - 1,
                                None) == _abi.EWORKSPACE
    assert lib.lazyattn_prefill_attend(ctypes.byref(once), P, P, 2, 1, P, P, 1, ctypes.byref(b), 1, P, None, 0,
                                       None) == _abi.EWORKSPACE


def test_gpu_entry_points_reject_bad_arguments_before_launch():
    lib = _abi.lib()
    c = _cfg()
    b = _abi.Batch()
    b.num_reqs, b.max_entries = 2, 4
    b.block_tables = b.num_entries = b.ctx_lens = 16   # never dereferenced on the host
    P = ctypes.c_void_p(64)
    # null config / batch
    assert lib.lazyattn_prefill(None, P, P, 1, 1, P, P, 1, ctypes.byref(b), 0, P, None, 0, None) == _abi.EINVAL
    assert lib.lazyattn_decode(ctypes.byref(c), P, P, P, 1, None, 0, P, None, 0, None) == _abi.EINVAL
    # null data pointers
    assert lib.lazyattn_prefill(ctypes.byref(c), None, P, 1, 1, P, P, 1, ctypes.byref(b), 0, P, None, 0, None) == _abi.EINVAL
    assert lib.lazyattn_decode(ctypes.byref(c), P, None, P, 1, ctypes.byref(b), 0, P, None, 0, None) == _abi.EINVAL
    assert lib.lazyattn_append_kv(ctypes.byref(c), P, P, 1, P, None, P, 3, None) == _abi.EINVAL
    # out-of-range sizes
    assert lib.lazyattn_prefill(ctypes.byref(c), P, P, -1, 1, P, P, 1, ctypes.byref(b), 0, P, None, 0, None) == _abi.EINVAL
    assert lib.lazyattn_prefill(ctypes.byref(c), P, P, 1, 1, P, P, 1, ctypes.byref(b), 65, P, None, 0, None) == _abi.EINVAL
    assert lib.lazyattn_decode(ctypes.byref(c), P, P, P, 1, ctypes.byref(b), 257, P, None, 0, None) == _abi.EINVAL
    assert lib.lazyattn_prefill(ctypes.byref(c), P, P, 1, 1, P, P, 0, ctypes.byref(b), 0, P, None, 0, None) == _abi.EINVAL
    # unsupported shapes
    c33 = _cfg(num_q_heads=66, num_kv_heads=2)
    assert lib.lazyattn_decode(ctypes.byref(c33), P, P, P, 1, ctypes.byref(b), 0, P, None, 0, None) == _abi.EUNSUPPORTED
    # a split call without its workspace
    assert lib.lazyattn_decode(ctypes.byref(c), P, P, P, 1, ctypes.byref(b), 8, P, None, 0, None) == _abi.EWORKSPACE
    assert lib.lazyattn_prefill(ctypes.byref(c), P, P, 1, 1, P, P, 1, ctypes.byref(b), 4, P, P, 16, None) == _abi.EWORKSPACE
    assert lib.lazyattn_prefill_attend(ctypes.byref(c), P, P, 1, 1, P, P, 1, ctypes.byref(b), 4, P, P, 16, None) == _abi.EWORKSPACE
    assert lib.lazyattn_decode_attend(ctypes.byref(c), P, P, P, 1, ctypes.byref(b), 8, P, None, 0, None) == _abi.EWORKSPACE
    # merge: bad counts, short workspace, and the no-op cases
    assert lib.lazyattn_merge_splits(ctypes.byref(c), 4, 0, P, 1 << 20, P, None) == _abi.EINVAL
    assert lib.lazyattn_merge_splits(ctypes.byref(c), -1, 2, P, 1 << 20, P, None) == _abi.EINVAL
    assert lib.lazyattn_merge_splits(ctypes.byref(c), 4, 2, P, 2 * 4 * 4 * (128 * 2 + 8) - 1, P, None) == _abi.EWORKSPACE
    assert lib.lazyattn_merge_splits(ctypes.byref(c), 4, 1, None, 0, None, None) == _abi.OK
    assert lib.lazyattn_merge_splits(ctypes.byref(c), 0, 3, None, 0, None, None) == _abi.OK
    # document-local frames: RoPE and bf16 only; the framed append needs its indices
    bf = _abi.Batch()
    bf.num_reqs, bf.max_entries = 2, 4
    bf.block_tables = bf.num_entries = bf.ctx_lens = bf.frame_starts = 16
    c32 = _cfg(dtype="f32", head_dim=64)
    assert lib.lazyattn_prefill(ctypes.byref(c32), P, P, 1, 1, P, P, 1, ctypes.byref(bf), 0, P, None, 0, None) == _abi.EUNSUPPORTED
    assert lib.lazyattn_decode(ctypes.byref(_cfg(pe="alibi")), P, P, P, 1, ctypes.byref(bf), 0, P, None, 0, None) == _abi.EUNSUPPORTED
    assert lib.lazyattn_decode(ctypes.byref(_cfg(pe="none")), P, P, P, 1, ctypes.byref(bf), 0, P, None, 0, None) == _abi.EUNSUPPORTED
    assert lib.lazyattn_materialize_kv(ctypes.byref(c), P, P, 1, ctypes.byref(bf), P, P, P, 1, None) == _abi.EUNSUPPORTED
    assert lib.lazyattn_append_kv_framed(ctypes.byref(c), P, P, 1, P, P, P, None, 3, None) == _abi.EINVAL
    assert lib.lazyattn_append_kv_framed(ctypes.byref(c), P, P, 1, P, P, P, P, -1, None) == _abi.EINVAL
    assert lib.lazyattn_append_kv_framed(ctypes.byref(_cfg(pe="none")), P, P, 1, P, P, P, P, 3, None) == _abi.EUNSUPPORTED
    assert lib.lazyattn_append_kv_framed(ctypes.byref(c32), P, P, 1, P, P, P, P, 3, None) == _abi.EUNSUPPORTED
    assert lib.lazyattn_append_kv_framed(ctypes.byref(c), None, None, 0, None, None, None, None, 0, None) == _abi.OK
    # malformed batch
    b2 = _abi.Batch()
    b2.num_reqs, b2.max_entries = 1, 0
    assert lib.lazyattn_decode(ctypes.byref(c), P, P, P, 1, ctypes.byref(b2), 0, P, None, 0, None) == _abi.EINVAL
    assert lib.lazyattn_debug_decode_tables(ctypes.byref(b2), P, None) == _abi.EINVAL
    # empty work is a no-op that succeeds without a launch
    b0 = _abi.Batch()
    assert lib.lazyattn_decode(ctypes.byref(c), None, None, None, 0, ctypes.byref(b0), 0, None, None, 0, None) == _abi.OK
    assert lib.lazyattn_prefill(ctypes.byref(c), None, None, 0, 0, None, None, 0, ctypes.byref(b), 0, None, None, 0, None) == _abi.OK
    assert lib.lazyattn_append_kv(ctypes.byref(c), None, None, 0, None, None, None, 0, None) == _abi.OK


def test_rope_frequency_tables_match_the_oracle():
    import oracle as O
    for D, rd, th in ((128, 128, 5e5), (128, 64, 1e4), (64, 32, 1e4), (128, 2, 10.0)):
        np.testing.assert_allclose(_abi.rope_inv_freq(D, rd, th), O.rope_inv_freq_partial(D, rd, th), rtol=1e-14)
    for args in ((128, 5e5, 8.0, 1.0, 4.0, 8192), (128, 5e5, 1.0, 1.0, 4.0, 8192), (64, 1e4, 4.0, 2.0, 8.0, 2048)):
        np.testing.assert_allclose(_abi.rope_inv_freq_llama31(*args), O.rope_inv_freq_llama31(*args), rtol=1e-14)
    lib = _abi.lib()
    out = np.empty(64)
    bad = [(128, 0, 1e4), (128, 3, 1e4), (128, 130, 1e4), (128, 64, 0.0), (127, 64, 1e4)]
    for D, rd, th in bad:
        assert lib.lazyattn_rope_inv_freq(D, rd, th, out.ctypes.data) == _abi.EINVAL
    assert lib.lazyattn_rope_inv_freq(128, 64, 1e4, None) == _abi.EINVAL
    assert lib.lazyattn_rope_inv_freq_llama31(128, 5e5, 0.5, 1.0, 4.0, 8192, out.ctypes.data) == _abi.EINVAL
    assert lib.lazyattn_rope_inv_freq_llama31(128, 5e5, 8.0, 4.0, 4.0, 8192, out.ctypes.data) == _abi.EINVAL
    assert lib.lazyattn_rope_inv_freq_llama31(128, 5e5, 8.0, 1.0, 4.0, 0, out.ctypes.data) == _abi.EINVAL


def test_config_frequency_table_checks():
    lib = _abi.lib()
    check = lambda c: lib.lazyattn_prefill_splits(ctypes.byref(c), 1, 1, 1) > 0
    good = _cfg(rope_theta=0.0, inv_freq=np.linspace(1.0, 0.0, 64))     # theta unused with a table
    assert check(good)
    assert not check(_cfg(rope_theta=0.0))
    assert not check(_cfg(inv_freq=np.full(64, -1.0)))
    assert not check(_cfg(inv_freq=np.full(64, np.inf)))
    assert not check(_cfg(inv_freq=np.full(64, np.nan)))


def test_balanced_prefill_splits():
    c = _cfg(num_q_heads=32, num_kv_heads=1)
    # equal lengths: the plain heuristic (one 128-token query tile per request gives 512 work-groups)
    assert _abi.prefill_splits_balanced(c, 32, 128, 651, 32 * 651) == _abi.prefill_splits(c, 32, 128, 651) == 1
    # the longest request 2.2x the mean: three splits bring its share per work-group to the mean's
    assert _abi.prefill_splits_balanced(c, 32, 128, 1445, 20832) == 3
    assert _abi.prefill_splits_balanced(c, 32, 128, 969, 16000) == 2
    # a ratio just above a whole number takes no extra split (70B: 2176 entries each, a table stride of 2184)
    c70 = _cfg(num_q_heads=64, num_kv_heads=8)
    assert _abi.prefill_splits_balanced(c70, 4, 2048, 2184, 4 * 2176) == 1
    assert _abi.prefill_splits_balanced(c, 32, 128, 1100, 32 * 1000) == 1
    assert _abi.prefill_splits_balanced(c, 32, 128, 1150, 32 * 1000) == 2
    # never fewer than the plain heuristic (8B shape: too few work-groups, 2 splits)
    c8 = _cfg(num_q_heads=32, num_kv_heads=8)
    assert _abi.prefill_splits_balanced(c8, 16, 64, 260, 16 * 260) == _abi.prefill_splits(c8, 16, 64, 260) == 2
    # at most one split per 64 entries of the longest request, and at most 64
    assert _abi.prefill_splits_balanced(c, 100, 4096, 100, 100) == 1
    assert _abi.prefill_splits_balanced(c, 1000, 4096, 100000, 100000) == 64
    # no lengths given, or an invalid config
    assert _abi.prefill_splits_balanced(c, 32, 128, 1445, 0) == _abi.prefill_splits(c, 32, 128, 1445)
    assert _abi.prefill_splits_balanced(_cfg(num_q_heads=3, num_kv_heads=2), 1, 1, 1, 1) == 0
