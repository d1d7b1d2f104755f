"""Pins of the fp64 oracle to facts fixed outside itself (CPU only).

Each test checks the oracle against something other than its own formula:
printed values of the LazyAttention pages, closed forms, hand-derived
vectors, an independent library routine (torch SDPA on CPU), brute-force
loops, and invariants the pages state (RoPE scores depend only on the
relative offset; deferred and materialised attention are identical; one
physical copy serves any logical position).
"""
import cmath
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([float(x) for x in line.split()])
    return rows


# ---------------------------------------------------------------------------
# table words
# ---------------------------------------------------------------------------
def test_codec_boundaries_and_hand_values():
    assert O.pack_entry(0, 0) == 0
    assert O.pack_entry(5, 144) == 144 * 2**32 + 5
    assert O.pack_entry(2**32 - 1, 2**32 - 1) == 2**64 - 1
    assert O.unpack_entry(2**64 - 1) == (2**32 - 1, 2**32 - 1)
    assert O.unpack_entry(0x0000_0090_0000_0005) == (5, 144)
    rng = np.random.default_rng(0)
    b = rng.integers(0, 2**32, size=1000, dtype=np.uint64)
    s = rng.integers(0, 2**32, size=1000, dtype=np.uint64)
    w = O.pack_table(b, s)
    for i in range(0, 1000, 97):
        assert O.unpack_entry(int(w[i])) == (int(b[i]), int(s[i]))
        assert int(w[i]) == O.pack_entry(int(b[i]), int(s[i]))


def test_decode_table_dense_contract_tiny_config():
    # tiny fp32 case: 4 documents of 2 blocks each at 0..112, query block at 128,
    # decode block at 144 (hand-derived from the config text)
    blocks = [6, 1, 4, 7, 2, 5, 3, 0, 8, 9]
    starts = [0, 16, 32, 48, 64, 80, 96, 112, 128, 144]
    words = [O.pack_entry(b, s) for b, s in zip(blocks, starts)]
    bb, ss, ll = O.decode_table(words, 9, 144, 16, 10)     # after the 16-token prefill
    assert list(bb) == blocks[:9] and list(ss) == starts[:9] and list(ll) == [16] * 9
    bb, ss, ll = O.decode_table(words, 10, 147, 16, 10)    # after 3 decode tokens
    assert list(ll) == [16] * 9 + [3]


@pytest.mark.parametrize("case", ["start0", "too_long", "empty_entry", "block_oob", "descending"])
def test_decode_table_rejects(case):
    good = [(0, 0), (1, 16), (2, 20)]
    L = 30
    if case == "start0":
        good[0] = (0, 1)
    elif case == "too_long":
        good[2] = (2, 33)
        L = 50
    elif case == "empty_entry":
        good[2] = (2, 16)
    elif case == "block_oob":
        good[1] = (10, 16)
    elif case == "descending":
        good[2] = (2, 10)
    words = [O.pack_entry(b, s) for b, s in good]
    with pytest.raises(O.TableError):
        O.decode_table(words, 3, L, 16, 10)


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------
def test_inv_freq_closed_form():
    assert np.array_equal(O.rope_inv_freq(4, 10000.0), np.array([1.0, 0.01]))
    f = O.rope_inv_freq(128, 500000.0)
    assert f[0] == 1.0
    assert math.isclose(f[64 // 2], 500000.0 ** -0.5, rel_tol=1e-15)
    assert math.isclose(f[-1], 500000.0 ** (-126 / 128), rel_tol=1e-15)


def test_rope_hand_vectors():
    for row in _golden_rows("rope_unit_vectors.txt"):
        D, theta, pos = int(row[0]), row[1], row[2]
        x = np.array(row[3:3 + D])
        y = np.array(row[3 + D:3 + 2 * D])
        got = O.rope_rotate(x, pos, O.rope_inv_freq(D, theta))
        np.testing.assert_allclose(got, y, rtol=0, atol=1e-15)


def test_rope_group_properties():
    rng = np.random.default_rng(1)
    D = 64
    f = O.rope_inv_freq(D, 10000.0)
    x = rng.standard_normal(D)
    np.testing.assert_array_equal(O.rope_rotate(x, 0, f), x)                  # R(0) = I
    for n in (1, 17, -300, 35000):
        y = O.rope_rotate(x, n, f)
        assert math.isclose(np.linalg.norm(y), np.linalg.norm(x), rel_tol=1e-13)
    a, b = 123, -4567
    np.testing.assert_allclose(O.rope_rotate(O.rope_rotate(x, a, f), b, f),
                               O.rope_rotate(x, a + b, f), atol=1e-11)       # R(a)R(b) = R(a+b)
    # R(n)^T = R(-n): <R(n)u, v> = <u, R(-n)v>
    u, v = rng.standard_normal(D), rng.standard_normal(D)
    assert math.isclose(O.rope_rotate(u, 77, f) @ v, u @ O.rope_rotate(v, -77, f), rel_tol=1e-12)


def test_rope_d2_is_complex_multiplication():
    theta0 = O.rope_inv_freq(2, 10000.0)[0]
    for n in (0, 1, 5, -9, 1000):
        x = np.array([0.3, -1.7])
        z = complex(x[0], x[1]) * cmath.exp(1j * n * theta0)
        y = O.rope_rotate(x, n, O.rope_inv_freq(2, 10000.0))
        assert abs(y[0] - z.real) < 1e-12 and abs(y[1] - z.imag) < 1e-12


# ---------------------------------------------------------------------------
# attention for one request: small random contexts
# ---------------------------------------------------------------------------
def _rand_ctx(rng, L=40, M=5, Hq=4, Hkv=2, D=16):
    K = rng.standard_normal((L, Hkv, D))
    V = rng.standard_normal((L, Hkv, D))
    q = rng.standard_normal((M, Hq, D))
    kp = np.arange(L)
    qp = np.arange(L - M, L)
    return q, qp, K, V, kp


def test_shift_invariance_of_rope_scores():
    # the pages: RoPE attention depends only on the offset n - m
    rng = np.random.default_rng(2)
    q, qp, K, V, kp = _rand_ctx(rng)
    o1, w1 = O.attend(q, qp, K, V, kp, pe="rope", rope_theta=10000.0, return_weights=True)
    for c in (1, 1000, 34567):
        o2, w2 = O.attend(q, qp + c, K, V, kp + c, pe="rope", rope_theta=10000.0, return_weights=True)
        np.testing.assert_allclose(w2, w1, rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(o2, o1, rtol=1e-9, atol=1e-12)


def test_deferred_equals_materialized():
    rng = np.random.default_rng(3)
    for theta in (10000.0, 500000.0):
        q, qp, K, V, kp = _rand_ctx(rng, L=70, M=7)
        qp = qp + 30000
        kp = kp + 30000
        a = O.attend(q, qp, K, V, kp, pe="rope", rope_theta=theta, formulation="materialized")
        b = O.attend(q, qp, K, V, kp, pe="rope", rope_theta=theta, formulation="deferred")
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def test_no_pe_equals_torch_sdpa():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    q, qp, K, V, kp = _rand_ctx(rng, L=33, M=9, Hq=4, Hkv=4, D=8)
    out = O.attend(q, qp, K, V, kp, pe="none")
    mask = torch.from_numpy(kp[None, :] <= qp[:, None])
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(K).permute(1, 0, 2)
    vt = torch.from_numpy(V).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_softmax_rows_sum_to_one_and_causal_zeros():
    rng = np.random.default_rng(5)
    q, qp, K, V, kp = _rand_ctx(rng)
    for pe in ("rope", "none", "alibi"):
        _, w = O.attend(q, qp, K, V, kp, pe=pe, rope_theta=10000.0, return_weights=True)
        np.testing.assert_allclose(w.sum(axis=-1), 1.0, atol=1e-13)
        for m, p in enumerate(qp):
            assert np.all(w[m, :, kp > p] == 0.0)
            assert np.all(w[m, :, kp <= p] > 0.0)


def test_gqa_equals_mha_with_repeated_heads():
    rng = np.random.default_rng(6)
    q, qp, K, V, kp = _rand_ctx(rng, Hq=8, Hkv=2)
    g = O.attend(q, qp, K, V, kp, pe="rope", rope_theta=500000.0)
    Kr = np.repeat(K, 4, axis=1)
    Vr = np.repeat(V, 4, axis=1)
    m = O.attend(q, qp, Kr, Vr, kp, pe="rope", rope_theta=500000.0)
    np.testing.assert_allclose(g, m, atol=1e-14)
    # MQA: one kv-head serves all
    g1 = O.attend(q, qp, K[:, :1], V[:, :1], kp, pe="rope", rope_theta=500000.0)
    m1 = O.attend(q, qp, np.repeat(K[:, :1], 8, 1), np.repeat(V[:, :1], 8, 1), kp, pe="rope", rope_theta=500000.0)
    np.testing.assert_allclose(g1, m1, atol=1e-14)


def test_alibi_slopes_closed_form_and_shift_invariance():
    # Press et al.: for 8 heads the slopes are 1/2, 1/4, ..., 1/256
    np.testing.assert_allclose(O.alibi_slopes(8), [2.0 ** -(i + 1) for i in range(8)], rtol=0, atol=0)
    s32 = O.alibi_slopes(32)
    assert s32[0] == 2.0 ** -0.25 and s32[-1] == 2.0 ** -8
    rng = np.random.default_rng(7)
    q, qp, K, V, kp = _rand_ctx(rng)
    a = O.attend(q, qp, K, V, kp, pe="alibi")
    b = O.attend(q, qp + 999, K, V, kp + 999, pe="alibi")
    np.testing.assert_allclose(a, b, atol=1e-12)
    # the bias is not a no-op
    c = O.attend(q, qp, K, V, kp, pe="none")
    assert np.max(np.abs(a - c)) > 1e-3


# ---------------------------------------------------------------------------
# the full path through tables and pools, against brute force
# ---------------------------------------------------------------------------
def _tiny_pool(rng, docs, B, Hkv, D, extra_blocks=0):
    """Dense pool holding documents (lists of token counts) in fresh blocks; NaN padding."""
    nblk = sum((n + B - 1) // B for n in docs) + extra_blocks
    kp = np.full((nblk, Hkv, B, D), np.nan)
    vp = np.full((nblk, Hkv, D, B), np.nan)
    perm = rng.permutation(nblk)
    doc_entries, cur = [], 0
    for n in docs:
        k = rng.standard_normal((n, Hkv, D))
        v = rng.standard_normal((n, Hkv, D))
        ents = []
        for j in range(0, n, B):
            b = int(perm[cur]); cur += 1
            rows = min(B, n - j)
            kp[b, :, :rows, :] = k[j:j + rows].transpose(1, 0, 2)
            vp[b, :, :, :rows] = v[j:j + rows].transpose(1, 2, 0)
            ents.append((b, rows))
        doc_entries.append(ents)
    free = [int(x) for x in perm[cur:]]
    return kp.astype(np.float32), vp.astype(np.float32), doc_entries, free


def _words_for(order, doc_entries, priv_entries=()):
    words, pos = [], 0
    for d in order:
        for b, rows in doc_entries[d]:
            words.append(O.pack_entry(b, pos))
            pos += rows
    for b, rows in priv_entries:
        words.append(O.pack_entry(b, pos))
        pos += rows
    return words, pos


@pytest.mark.parametrize("pe,Hq,Hkv", [("rope", 1, 1), ("rope", 2, 1), ("alibi", 2, 1), ("none", 2, 2)])
def test_brute_force_tiny(pe, Hq, Hkv):
    # D=4, B=2, two 3-token documents and one 2-token query
    rng = np.random.default_rng(8)
    B, D = 2, 4
    kp, vp, doc_entries, free = _tiny_pool(rng, [3, 3], B, Hkv, D, extra_blocks=1)
    qb = free[0]
    knew = rng.standard_normal((2, Hkv, D)).astype(np.float32)
    vnew = rng.standard_normal((2, Hkv, D)).astype(np.float32)
    O.append_kv(kp, vp, knew, vnew, [qb * B, qb * B + 1], B)
    words, L = _words_for([1, 0], doc_entries, [(qb, 2)])
    q = rng.standard_normal((2, Hq, D)).astype(np.float32)
    got = O.prefill(q=q, cu_q_lens=[0, 2], ctx_lens=[L], num_entries=[len(words)],
                    table_words=[words], k_pool=kp, v_pool=vp, num_kv_heads=Hkv, block_size=B,
                    dtype="f32", pe=pe, rope_theta=10.0)[0]
    bf = O.brute_force_attention(q.astype(np.float64).tolist(), [L - 2, L - 1], words, len(words), L,
                                 kp.astype(np.float64).tolist(), vp.astype(np.float64).tolist(),
                                 B, Hq, Hkv, 10.0, pe=pe)
    np.testing.assert_allclose(got, np.array(bf), rtol=1e-12, atol=1e-13)


def test_reuse_one_physical_copy_equals_private_copies():
    # the pages' core claim: a single physical KV copy serves requests at any offset
    rng = np.random.default_rng(9)
    B, Hkv, Hq, D = 4, 2, 4, 8
    kp, vp, de, free = _tiny_pool(rng, [9, 7, 5], B, Hkv, D)
    qs = rng.standard_normal((2, 3, Hq, D)).astype(np.float32)
    shared = []
    for order, qq in (([0, 1, 2], qs[0]), ([2, 1, 0], qs[1])):
        w, L = _words_for(order, de)
        shared.append(O.decode(q=qq[-1:], ctx_lens=[L], num_entries=[len(w)], table_words=[w],
                               k_pool=kp, v_pool=vp, num_kv_heads=Hkv, block_size=B, dtype="f32",
                               pe="rope", rope_theta=100.0)[0])
    # same contents, but each request gets its own copies of every block
    nb = kp.shape[0]
    kp2 = np.concatenate([kp, kp])
    vp2 = np.concatenate([vp, vp])
    de2 = [[(b + nb, r) for b, r in ents] for ents in de]
    w1, L1 = _words_for([0, 1, 2], de)
    w2, L2 = _words_for([2, 1, 0], de2)
    priv = [O.decode(q=qs[0][-1:], ctx_lens=[L1], num_entries=[len(w1)], table_words=[w1], k_pool=kp2,
                     v_pool=vp2, num_kv_heads=Hkv, block_size=B, dtype="f32", pe="rope", rope_theta=100.0)[0],
            O.decode(q=qs[1][-1:], ctx_lens=[L2], num_entries=[len(w2)], table_words=[w2], k_pool=kp2,
                     v_pool=vp2, num_kv_heads=Hkv, block_size=B, dtype="f32", pe="rope", rope_theta=100.0)[0]]
    np.testing.assert_array_equal(shared[0], priv[0])
    np.testing.assert_array_equal(shared[1], priv[1])
    # and the two requests do see the document at different positions
    assert np.max(np.abs(shared[0] - shared[1])) > 1e-3


def test_reblocking_invariance():
    # splitting the same documents into blocks of 2, 4 or 16 tokens does not change the result
    outs = []
    for B in (2, 4, 16):
        rng = np.random.default_rng(10)          # same values each time
        Hkv, Hq, D = 1, 2, 8
        docs = [rng.standard_normal((n, Hkv, D)) for n in (5, 11)]
        vals = [rng.standard_normal((n, Hkv, D)) for n in (5, 11)]
        q = rng.standard_normal((3, Hq, D))
        nblk = sum((d.shape[0] + B - 1) // B for d in docs)
        kp = np.full((nblk, Hkv, B, D), np.nan)
        vp = np.full((nblk, Hkv, D, B), np.nan)
        words, pos, b = [], 0, nblk - 1          # fill blocks from the tail, descending ids
        for k, v in zip(docs, vals):
            for j in range(0, k.shape[0], B):
                rows = min(B, k.shape[0] - j)
                kp[b, :, :rows] = k[j:j + rows].transpose(1, 0, 2)
                vp[b, :, :, :rows] = v[j:j + rows].transpose(1, 2, 0)
                words.append(O.pack_entry(b, pos))
                pos += rows
                b -= 1
        outs.append(O.prefill(q=q, cu_q_lens=[0, 3], ctx_lens=[pos], num_entries=[len(words)],
                              table_words=[words], k_pool=kp, v_pool=vp, num_kv_heads=Hkv,
                              block_size=B, dtype="f32", pe="rope", rope_theta=1000.0)[0])
    np.testing.assert_allclose(outs[1], outs[0], atol=1e-13)
    np.testing.assert_allclose(outs[2], outs[0], atol=1e-13)


def test_decode_equals_last_row_of_prefill():
    rng = np.random.default_rng(11)
    B, Hkv, Hq, D = 4, 2, 4, 8
    kp, vp, de, free = _tiny_pool(rng, [6, 9], B, Hkv, D, extra_blocks=2)
    n_new = 5
    knew = rng.standard_normal((n_new, Hkv, D)).astype(np.float32)
    vnew = rng.standard_normal((n_new, Hkv, D)).astype(np.float32)
    O.append_kv(kp, vp, knew, vnew, [free[i // B] * B + i % B for i in range(n_new)], B)
    w, L = _words_for([1, 0], de, [(free[0], 4), (free[1], 1)])
    q = rng.standard_normal((n_new, Hq, D)).astype(np.float32)
    pre = O.prefill(q=q, cu_q_lens=[0, n_new], ctx_lens=[L], num_entries=[len(w)], table_words=[w],
                    k_pool=kp, v_pool=vp, num_kv_heads=Hkv, block_size=B, dtype="f32", pe="rope",
                    rope_theta=500.0)[0]
    dec = O.decode(q=q[-1:], ctx_lens=[L], num_entries=[len(w)], table_words=[w], k_pool=kp,
                   v_pool=vp, num_kv_heads=Hkv, block_size=B, dtype="f32", pe="rope",
                   rope_theta=500.0)[0]
    # equal up to BLAS summation order (M=1 vs M=5 products)
    np.testing.assert_allclose(dec, pre[-1], rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# appends: what the content-only pool holds after new tokens arrive
# ([gist:Methodology]: the cache stores content only, no rotation).  Checked
# against the documented layout, K [block][head][row][d] and V [block][head][d][row],
# by reading every written element back with explicit indices, and against a
# NaN-poisoned pool: every slot not written must still be NaN (np.isnan, since
# assert_allclose would take NaN == NaN as a match).
# ---------------------------------------------------------------------------
_APPEND_SLOTS = [(1, 15), (2, 0), (2, 7), (0, 3), (3, 15)]     # (block, row): a last row, a partial block


def _poisoned_pools(nb, Hkv, B, D, dtype=np.float64):
    return np.full((nb, Hkv, B, D), np.nan, dtype=dtype), np.full((nb, Hkv, D, B), np.nan, dtype=dtype)


def _hand_kv(n, Hkv, D):
    # value i*1000 + h*100 + d (K) and its negative minus 0.5 (V): every element distinct
    i, h, d = np.meshgrid(np.arange(n), np.arange(Hkv), np.arange(D), indexing="ij")
    k = (1000.0 * i + 100.0 * h + d).astype(np.float64)
    return k, -k - 0.5


def test_append_kv_layout_and_untouched_slots():
    B, Hkv, D, nb = 16, 2, 4, 5
    kp, vp = _poisoned_pools(nb, Hkv, B, D)
    k, v = _hand_kv(len(_APPEND_SLOTS), Hkv, D)
    O.append_kv(kp, vp, k, v, [b * B + r for b, r in _APPEND_SLOTS], B)
    written_k = np.zeros(kp.shape, dtype=bool)
    written_v = np.zeros(vp.shape, dtype=bool)
    for i, (b, r) in enumerate(_APPEND_SLOTS):
        for h in range(Hkv):
            for d in range(D):
                assert kp[b, h, r, d] == 1000 * i + 100 * h + d
                assert vp[b, h, d, r] == -(1000 * i + 100 * h + d) - 0.5
                written_k[b, h, r, d] = True
                written_v[b, h, d, r] = True
    assert np.isnan(kp[~written_k]).all() and np.isnan(vp[~written_v]).all()
    assert not np.isnan(kp[written_k]).any() and not np.isnan(vp[written_v]).any()


def test_append_kv_bf16_bit_patterns_and_overwrite():
    # bf16 pools are uint16 bit patterns: the append copies them unchanged; a second
    # append to the same slot replaces it and leaves its neighbours alone
    B, Hkv, D, nb = 16, 1, 2, 3
    nan_bits = np.uint16(0x7FC0)
    kp = np.full((nb, Hkv, B, D), nan_bits, dtype=np.uint16)
    vp = np.full((nb, Hkv, D, B), nan_bits, dtype=np.uint16)
    k = np.array([[[0x3F80, 0xBF80]], [[0x4000, 0x0001]]], dtype=np.uint16)   # 1, -1 ; 2, smallest subnormal
    v = np.array([[[0x4040, 0x8000]], [[0x7F7F, 0xC000]]], dtype=np.uint16)   # 3, -0 ; max finite, -2
    O.append_kv(kp, vp, k, v, [2 * B + 15, 0 * B + 0], B)
    assert kp[2, 0, 15].tolist() == [0x3F80, 0xBF80] and vp[2, 0, :, 15].tolist() == [0x4040, 0x8000]
    assert kp[0, 0, 0].tolist() == [0x4000, 0x0001] and vp[0, 0, :, 0].tolist() == [0x7F7F, 0xC000]
    assert int((kp != nan_bits).sum()) == 4 and int((vp != nan_bits).sum()) == 4
    O.append_kv(kp, vp, v[:1], k[:1], [2 * B + 15], B)
    assert kp[2, 0, 15].tolist() == [0x4040, 0x8000] and vp[2, 0, :, 15].tolist() == [0x3F80, 0xBF80]
    assert kp[2, 0, 14].tolist() == [nan_bits] * 2 and vp[2, 0, 0, 14] == nan_bits
    assert int((kp != nan_bits).sum()) == 4 and int((vp != nan_bits).sum()) == 4


def test_append_kv_framed_layout_and_quarter_turns():
    # one channel pair at angular frequency pi/2 per position: frame index j turns a
    # key by j quarter turns, (x, y) -> (-y, x) -> (-x, -y) -> (y, -x), values hand-derived;
    # V is stored unrotated
    B, Hkv, D, nb = 16, 2, 2, 4
    kp, vp = _poisoned_pools(nb, Hkv, B, D)
    k, v = _hand_kv(len(_APPEND_SLOTS), Hkv, D)
    frames = [1, 2, 3, 0, 5]
    O.append_kv_framed(kp, vp, k.astype(np.float32), v.astype(np.float32), [b * B + r for b, r in _APPEND_SLOTS],
                       frames, B, np.array([math.pi / 2]), "f32")
    turns = {0: lambda x, y: (x, y), 1: lambda x, y: (-y, x), 2: lambda x, y: (-x, -y), 3: lambda x, y: (y, -x)}
    written_k = np.zeros(kp.shape, dtype=bool)
    written_v = np.zeros(vp.shape, dtype=bool)
    for i, (b, r) in enumerate(_APPEND_SLOTS):
        for h in range(Hkv):
            x, y = 1000.0 * i + 100.0 * h, 1000.0 * i + 100.0 * h + 1.0
            ex = turns[frames[i] % 4](x, y)
            assert abs(kp[b, h, r, 0] - ex[0]) <= 1e-9 * 1e4 and abs(kp[b, h, r, 1] - ex[1]) <= 1e-9 * 1e4
            assert vp[b, h, 0, r] == -x - 0.5 and vp[b, h, 1, r] == -y - 0.5
            written_k[b, h, r, :] = True
            written_v[b, h, :, r] = True
    assert np.isnan(kp[~written_k]).all() and np.isnan(vp[~written_v]).all()


def test_bf16_conversion_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x3F81, 0x7F7F, 0x0001], dtype=np.uint16)
    want = [1.0, -1.0, 0.0, -0.0, 1.0 + 2.0 ** -7, (2 - 2.0 ** -7) * 2.0 ** 127, 2.0 ** -133]
    np.testing.assert_array_equal(O.bf16_to_f64(bits), want)


# ---------------------------------------------------------------------------
# cost model printed on the pages
# ---------------------------------------------------------------------------
def test_rotation_cost_model_matches_printed_value():
    for M, pct, dec in _golden_rows("cost_model.txt"):
        frac = O.rotation_flop_fraction(int(M))
        assert round(100 * frac, int(dec)) == pct
        assert math.isclose(frac, 3.0 / (4.0 * M), rel_tol=1e-15)
    for M in (1, 16, 64, 256, 1024):
        assert math.isclose(O.rotation_flop_fraction(M, N=32, D=64), 3.0 / (4.0 * M), rel_tol=1e-15)


# ---------------------------------------------------------------------------
# negative controls: plausible mistakes must move the result beyond the bf16 bar
# ---------------------------------------------------------------------------
def test_plausible_mistakes_exceed_bf16_tolerance_at_long_context():
    rng = np.random.default_rng(12)
    L, M, Hq, Hkv, D = 4160, 4, 4, 1, 128
    K = rng.standard_normal((L, Hkv, D))
    V = rng.standard_normal((L, Hkv, D))
    q = rng.standard_normal((M, Hq, D))
    kp, qp = np.arange(L), np.arange(L - M, L)
    ref = O.attend(q, qp, K, V, kp, pe="rope", rope_theta=500000.0)
    off_by_one = O.attend(q, qp + 1, K, V, kp, pe="rope", rope_theta=500000.0)
    no_rot = O.attend(q, qp, K, V, kp, pe="none")
    half = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])   # half-split pair layout
    swapped = O.attend(q[..., half], qp, K[..., half], V, kp, pe="rope", rope_theta=500000.0)
    for bad in (off_by_one, no_rot, swapped):
        assert np.max(np.abs(bad - ref)) > 1e-2 or np.mean(np.abs(bad - ref)) > 1e-3


# ---------------------------------------------------------------------------
# document-local frames: the framed pool gives the content-only results
# ---------------------------------------------------------------------------
def _framed_pools(wl, inv_freq, extra=None):
    """fp64 framed pools of a workload: every referenced document written with
    its in-document indices, then ``extra`` new tokens with their frame_index."""
    kp, vp = wl.pools()
    k64 = np.full(kp.shape, np.nan)
    v64 = np.full(vp.shape, np.nan)
    for d in wl.referenced_docs:
        k, v = wl.doc_kv(int(d))
        slots, j = wl.doc_frame_tokens(int(d))
        O.append_kv_framed(k64, v64, k, v, slots, j, wl.B, inv_freq, wl.spec.dtype)
    if extra is not None:
        O.append_kv_framed(k64, v64, extra["k_new"], extra["v_new"], extra["slots"], extra["frame_index"],
                           wl.B, inv_freq, wl.spec.dtype)
    return k64, v64


def test_framed_pool_equals_content_pool_tiny():
    import workloads as W
    wl = W.build_workload(W.spec(1))
    s = wl.spec
    inv_freq = O.rope_inv_freq(s.head_dim, s.rope_theta)
    pb = wl.prefill_batch()
    kc, vc = wl.pools()
    kc, vc = kc.dense(), vc.dense()
    O.append_kv(kc, vc, pb["k_new"], pb["v_new"], pb["slots"], wl.B)
    kf, vf = _framed_pools(wl, inv_freq, pb)
    words = O.pack_table(pb["table_blocks"], pb["table_starts"])
    common = dict(q=pb["q"], cu_q_lens=pb["cu_q_lens"], ctx_lens=pb["ctx_lens"],
                  num_entries=pb["num_entries"], table_words=words, block_size=wl.B, dtype=s.dtype,
                  rope_theta=s.rope_theta)
    ref = O.prefill(k_pool=kc, v_pool=vc, num_kv_heads=s.num_kv_heads, pe="rope", **common)
    got = O.prefill_framed(k_pool=kf, v_pool=vf, frame_starts=pb["frame_starts"], **common)
    for r in ref:
        np.testing.assert_allclose(got[r], ref[r], rtol=0, atol=1e-12)
    # the frames differ from 0 and from the positions: the check is not vacuous
    fs = pb["frame_starts"][0, :int(pb["num_entries"][0])]
    assert len(set(fs.tolist())) > 2 and fs[0] == 0
    # one decode step (its token appended with frame index q_len)
    ds = wl.decode_step(0)
    O.append_kv(kc, vc, ds["k_new"], ds["v_new"], ds["slots"], wl.B)
    O.append_kv_framed(kf, vf, ds["k_new"], ds["v_new"], ds["slots"], ds["frame_index"], wl.B, inv_freq, s.dtype)
    words = O.pack_table(ds["table_blocks"], ds["table_starts"])
    common = dict(q=ds["q"], ctx_lens=ds["ctx_lens"], num_entries=ds["num_entries"], table_words=words,
                  block_size=wl.B, dtype=s.dtype, rope_theta=s.rope_theta)
    ref = O.decode(k_pool=kc, v_pool=vc, num_kv_heads=s.num_kv_heads, pe="rope", **common)
    got = O.decode_framed(k_pool=kf, v_pool=vf, frame_starts=ds["frame_starts"], **common)
    for r in ref:
        np.testing.assert_allclose(got[r], ref[r], rtol=0, atol=1e-12)


def test_framed_planted_frame_mistakes_are_seen():
    # a frame start off by one for one document, or the frames ignored (every
    # key read as if stored at its absolute position), moves the output far
    # beyond the bf16 tolerance
    import workloads as W
    wl = W.build_workload(W.spec(1))
    s = wl.spec
    inv_freq = O.rope_inv_freq(s.head_dim, s.rope_theta)
    pb = wl.prefill_batch()
    kf, vf = _framed_pools(wl, inv_freq, pb)
    words = O.pack_table(pb["table_blocks"], pb["table_starts"])
    common = dict(q=pb["q"], cu_q_lens=pb["cu_q_lens"], ctx_lens=pb["ctx_lens"],
                  num_entries=pb["num_entries"], table_words=words, k_pool=kf, v_pool=vf,
                  block_size=wl.B, dtype=s.dtype, rope_theta=s.rope_theta, requests=[0])
    good = O.prefill_framed(frame_starts=pb["frame_starts"], **common)[0]
    fs = pb["frame_starts"].copy()
    fs[0, 2:4] += 1                          # the second document's two entries
    bad = O.prefill_framed(frame_starts=fs, **common)[0]
    assert np.max(np.abs(bad - good)) > 2e-2
    ignored = O.prefill_framed(frame_starts=np.zeros_like(pb["frame_starts"]), **common)[0]
    assert np.max(np.abs(ignored - good)) > 2e-2


def test_framed_two_channel_closed_form():
    # D = 2, inv_freq = 1: a key stored at frame index j = t - F and a query at
    # p give the score cos/sin of (t - p) exactly as the unframed rotation does
    q = np.array([[[0.7, -0.2]]])                      # [M=1][H=1][D=2]
    k = np.array([[[1.0, 0.5]], [[-0.3, 0.8]]])       # two keys
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    t = np.array([3, 9])
    F = np.array([1, 6])                               # two different frames
    kf = O.rotate_into_frames(k, t - F, np.array([1.0]))
    out = O.attend_framed(q, np.array([9]), kf, v, t, F, rope_theta=1.0, softmax_scale=1.0)
    # hand: score_t = q . R(t - p) k with R(a) = [[cos a, -sin a], [sin a, cos a]]
    z = []
    for tt, kk in zip(t, k[:, 0]):
        a = float(tt - 9)
        rk = np.array([math.cos(a) * kk[0] - math.sin(a) * kk[1], math.sin(a) * kk[0] + math.cos(a) * kk[1]])
        z.append(float(q[0, 0] @ rk))
    w = np.exp(np.array(z) - max(z))
    w /= w.sum()
    np.testing.assert_allclose(out[0, 0], w, rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# RoPE variants: partial rotary and the Llama 3.1 frequency rescaling
# ---------------------------------------------------------------------------
def test_partial_rotary_table_and_identity_pairs():
    full = O.rope_inv_freq(128, 5e5)
    np.testing.assert_array_equal(O.rope_inv_freq_partial(128, 128, 5e5), full)
    part = O.rope_inv_freq_partial(128, 64, 1e4)
    assert np.all(part[32:] == 0.0)
    np.testing.assert_allclose(part[:32], O.rope_inv_freq(64, 1e4), rtol=1e-15)
    # zero-frequency pairs are left exactly as they are
    x = np.random.default_rng(12).standard_normal((5, 128))
    y = O.rope_rotate(x, np.arange(5) * 1000 + 3, part)
    np.testing.assert_array_equal(y[:, 64:], x[:, 64:])
    assert np.max(np.abs(y[:, :64] - x[:, :64])) > 0.1


def test_all_zero_frequencies_equal_no_positional_encoding():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((4, 4, 8))
    K = rng.standard_normal((9, 2, 8))
    V = rng.standard_normal((9, 2, 8))
    a = O.attend(q, np.arange(5, 9), K, V, np.arange(9), pe="rope", inv_freq=np.zeros(4))
    b = O.attend(q, np.arange(5, 9), K, V, np.arange(9), pe="none")
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-15)


def test_llama31_rescaling_structure():
    D, theta, L = 128, 5e5, 8192
    base = O.rope_inv_freq(D, theta)
    # factor 1 changes nothing
    np.testing.assert_allclose(O.rope_inv_freq_llama31(D, theta, 1.0, 1.0, 4.0, L), base, rtol=1e-15)
    f = O.rope_inv_freq_llama31(D, theta, 8.0, 1.0, 4.0, L)
    wl = 2 * np.pi / base
    short, long_ = wl < L / 4.0, wl > L / 1.0
    assert short.sum() > 0 and long_.sum() > 0 and (~short & ~long_).sum() > 0
    np.testing.assert_array_equal(f[short], base[short])
    np.testing.assert_allclose(f[long_], base[long_] / 8.0, rtol=1e-15)
    mid = ~short & ~long_
    assert np.all(f[mid] < base[mid]) and np.all(f[mid] > base[mid] / 8.0)
    assert np.all(np.diff(f) < 0)                    # still strictly decreasing with the pair index
    # continuity across both region boundaries: with pairs dense in frequency, neighbours stay close
    # (a blend running the wrong way, or swapped regions, jumps by up to the factor there)
    fd = O.rope_inv_freq_llama31(1 << 16, theta, 8.0, 1.0, 4.0, L)
    bd = O.rope_inv_freq(1 << 16, theta)
    assert np.max(np.abs(np.diff(np.log(fd)) - np.diff(np.log(bd)))) < 1e-3


# ---------------------------------------------------------------------------
# FP8 (OCP e4m3) pool: the format's definition and the quantisation rule
# ---------------------------------------------------------------------------
def test_e4m3_values_from_the_format():
    assert O.e4m3_value(0x38) == 1.0 and O.e4m3_value(0x7E) == 448.0 and O.e4m3_value(0xFE) == -448.0
    assert O.e4m3_value(0x08) == 2.0 ** -6 and O.e4m3_value(0x01) == 2.0 ** -9 and O.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert O.e4m3_value(0x40) == 2.0 and O.e4m3_value(0x3F) == 1.875
    assert math.isnan(O.e4m3_value(0x7F)) and math.isnan(O.e4m3_value(0xFF))
    assert O.e4m3_value(0x80) == 0.0 and math.copysign(1.0, O.e4m3_value(0x80)) == -1.0
    finite = [c for c in range(256) if not math.isnan(O.e4m3_value(c))]
    assert len(finite) == 254
    assert len({O.e4m3_value(c) for c in finite}) == 253           # +0 and -0 compare equal


def test_e4m3_encode_round_trip_ties_and_saturation():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = np.array([O.e4m3_value(int(c)) for c in codes])
    np.testing.assert_array_equal(O.e4m3_encode(vals), codes)
    # midpoints round to the even code
    assert O.e4m3_encode(np.array([1.0625]))[0] == 0x38             # between 1 (0x38) and 1.125 (0x39)
    assert O.e4m3_encode(np.array([1.1875]))[0] == 0x3A             # between 1.125 and 1.25
    assert O.e4m3_encode(np.array([-1.1875]))[0] == 0xBA
    assert O.e4m3_encode(np.array([2.0 ** -10]))[0] == 0x00         # between 0 and the first subnormal
    assert O.e4m3_encode(np.array([3 * 2.0 ** -10]))[0] == 0x02
    assert O.e4m3_encode(np.array([1.0625 + 1e-6]))[0] == 0x39
    # saturation instead of overflow to NaN
    np.testing.assert_array_equal(O.e4m3_encode(np.array([448.0, 460.0, 1e6, -1e6])), [0x7E, 0x7E, 0x7E, 0xFE])


def test_fp8_row_exponent_rule_and_quantisation_error():
    assert O.fp8_row_exponent(0.0) == 0
    assert O.fp8_row_exponent(448.0) == 0 and O.fp8_row_exponent(448.0 * (1 + 2 ** -20)) == 1
    assert O.fp8_row_exponent(224.0) == -1 and O.fp8_row_exponent(1.0) == -8
    assert O.fp8_row_exponent(1.75) == -8 and O.fp8_row_exponent(1.75 * (1 + 2 ** -20)) == -7
    assert O.fp8_row_exponent(1e-45) == -127
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((200, 128)) * np.exp(rng.uniform(-8, 8, (200, 1)))).astype(np.float32)
    codes, exps = O.quantize_fp8_rows(x)
    table = np.array([O.e4m3_value(c) for c in range(256)])
    deq = table[codes] * np.ldexp(1.0, exps.astype(np.int32))[:, None]
    amax = np.abs(x).max(axis=1)
    assert np.all(amax <= 448.0 * np.ldexp(1.0, exps.astype(np.int32)))
    assert np.all(amax > 224.0 * np.ldexp(1.0, exps.astype(np.int32)))       # the smallest such exponent
    # relative error of a normal e4m3 value: at most 2^-4 (half of the 3-bit mantissa step)
    big = np.abs(x) >= 2.0 ** -6 * np.ldexp(1.0, exps.astype(np.int32))[:, None]
    rel = np.abs(deq - x) / np.abs(x)
    assert rel[big].max() <= 2.0 ** -4 + 1e-12


def test_fp8_pool_view_dequantises_the_chunk_layout():
    rng = np.random.default_rng(15)
    kc, vc = O.fp8_empty_pools(3, 2)
    k = rng.standard_normal((5, 2, 128)).astype(np.float32)
    v = rng.standard_normal((5, 2, 128)).astype(np.float32)
    slots = np.array([16 * 2 + 3, 16 * 2 + 4, 16 * 0 + 15, 16 * 1 + 0, 16 * 2 + 5])
    O.append_kv_fp8(kc, vc, k, v, slots, "f32")
    K = O.Fp8PoolView(kc, "k")[np.array([0, 1, 2])]
    V = O.Fp8PoolView(vc, "v")[np.array([0, 1, 2])]
    # within half a mantissa step (2^-4 relative), or half a subnormal step (2^-10 x the row's
    # scale) for the values that fall below the smallest normal
    _, ke = O.quantize_fp8_rows(k)
    _, ve = O.quantize_fp8_rows(v)
    for i, sl in enumerate(slots):
        b, r = divmod(int(sl), 16)
        for got, want, e in ((K[b, :, r, :], k[i], ke[i]), (V[b, :, :, r], v[i], ve[i])):
            bound = np.maximum(2.0 ** -4 * np.abs(want), np.ldexp(1.0, e.astype(np.int32) - 10)[:, None])
            assert np.all(np.abs(got - want) <= bound)
    assert np.isnan(K[0, :, 0, :]).all()                                # never written
