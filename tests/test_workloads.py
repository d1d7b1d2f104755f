"""The seeded input generator: distributions, table structure and pool layout (CPU only)."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from workloads.synth import _zipf_draw


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -2.5, np.inf, np.nan],
                 dtype=np.float32)
    b = W.f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 ties -> 1 + 2^-6 (even)
    assert list(b[:6]) == [0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xC020, 0x7F80]
    assert np.isnan(W.bf16_bits_to_f32(b[6:7]))[0]
    y = W.bf16_bits_to_f32(b[:6])
    assert list(y) == [1.0, 1.0, 1.0 + 2.0 ** -6, 1.0, -2.5, np.inf]


def test_zipf_first_draw_matches_closed_form():
    # first draw of a request follows P(k) ~ k^-s exactly; chi-square over many draws
    rng = np.random.default_rng(123)
    n_pool, s, trials = 20, 1.2, 20000
    counts = np.zeros(n_pool)
    for _ in range(trials):
        w = np.arange(1, n_pool + 1, dtype=np.float64) ** -s
        cdf = np.cumsum(w)
        k = int(np.searchsorted(cdf, rng.random() * cdf[-1], side="right"))
        counts[k] += 1
    p = np.arange(1, n_pool + 1, dtype=np.float64) ** -s
    p /= p.sum()
    exp = trials * p
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    assert chi2 < 45.3   # chi-square 0.999 quantile, 19 dof
    # and the generator's sampler (order destroyed by its final shuffle) has the same marginal
    rng = np.random.default_rng(7)
    hits = np.zeros(n_pool)
    for _ in range(4000):
        hits[_zipf_draw(rng, n_pool, 1, s)] += 1
    exp = 4000 * p
    assert float(((hits - exp) ** 2 / exp).sum()) < 45.3


def test_zipf_draws_are_distinct():
    rng = np.random.default_rng(3)
    for s in (0.0, 0.8, 1.6):
        d = _zipf_draw(rng, 50, 32, s)
        assert len(set(d.tolist())) == 32


def test_lognormal_lengths():
    wl = W.build_workload(W.spec(5))
    L = wl.doc_lens
    assert L.min() >= 64 and L.max() <= 2048
    assert 270 <= np.median(L) <= 330
    # most documents end mid-block
    assert np.mean(L % 16 != 0) > 0.8


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_tables_obey_dense_contract(cfg):
    wl = W.build_workload(W.spec(cfg))
    for q in wl.requests:
        words = O.pack_table(q.entry_blocks, q.entry_starts)
        n_new = q.q_len + q.n_decode
        L = q.ctx_docs + n_new
        blocks, starts, lens = O.decode_table(words, q.num_entries_after(n_new), L, 16, wl.num_blocks)
        assert lens.sum() == L
        assert np.all(q.entry_blocks[:q.n_doc_entries] < wl.n_doc_blocks)
        assert np.all(q.private_blocks >= wl.n_doc_blocks)
    # private blocks are not shared between requests
    priv = np.concatenate([q.private_blocks for q in wl.requests])
    assert np.unique(priv).size == priv.size


def test_known_sizes():
    assert W.build_workload(W.spec(1)).num_blocks == 10
    wl2 = W.build_workload(W.spec(2))
    assert wl2.n_doc_blocks == 8192
    assert max(q.entry_blocks.size for q in wl2.requests) == 260
    wl4 = W.build_workload(W.spec(4, requests=[1]))
    assert wl4.n_doc_blocks == 131072
    assert wl4.requests[0].entry_blocks.size == 2048 + 136


def test_pool_layout_round_trip_tiny():
    # token t of the assembled context equals the document's own K/V row
    wl = W.build_workload(W.spec(1))
    kp, vp = wl.pools()
    q = wl.requests[0]
    words = O.pack_table(q.entry_blocks, q.entry_starts)
    K, V, pos = O.gather_context(words, q.n_doc_entries, q.ctx_docs, kp, vp, 16, "f32")
    off = 0
    for d in q.doc_ids:
        k, v = wl.doc_kv(int(d))
        np.testing.assert_array_equal(K[off:off + k.shape[0]], k.astype(np.float64))
        np.testing.assert_array_equal(V[off:off + k.shape[0]], v.astype(np.float64))
        off += k.shape[0]
    assert off == q.ctx_docs


def test_pool_layout_round_trip_partial_blocks():
    wl = W.build_workload(W.spec(5, requests=[2, 2], skew=0.8))
    kp, vp = wl.pools()
    for q in wl.requests:
        words = O.pack_table(q.entry_blocks, q.entry_starts)
        K, V, pos = O.gather_context(words, q.n_doc_entries, q.ctx_docs, kp, vp, 16, "bf16")
        assert not np.isnan(K).any() and not np.isnan(V).any()
        off = 0
        for d in q.doc_ids:
            k, v = wl.doc_kv(int(d))
            np.testing.assert_array_equal(K[off:off + k.shape[0]], O.bf16_to_f64(k))
            np.testing.assert_array_equal(V[off:off + k.shape[0]], O.bf16_to_f64(v))
            off += k.shape[0]


def test_padding_and_unwritten_blocks_are_nan():
    wl = W.build_workload(W.spec(5, requests=[1, 1]))
    kp, vp = wl.pools()
    d = int(wl.referenced_docs[0])
    L = int(wl.doc_lens[d])
    last = wl.doc_blocks(d)[-1]
    rows = L % 16
    if rows:
        blk = kp[np.array([last])][0]
        assert np.all(blk[:, rows:, :] == 0x7FC0)
        assert np.all(blk[:, :rows, :] != 0x7FC0)
    unref = np.setdiff1d(np.arange(wl.n_doc_blocks), kp.ids)
    if unref.size:
        assert np.all(kp[unref[:3]] == 0x7FC0)


def test_streams_are_reproducible_and_sweep_dependent():
    a = W.build_workload(W.spec(5, skew=1.2, pe="rope"))
    b = W.build_workload(W.spec(5, skew=1.2, pe="rope"))
    c = W.build_workload(W.spec(5, skew=1.6, pe="rope"))
    assert all(np.array_equal(x.entry_blocks, y.entry_blocks) for x, y in zip(a.requests, b.requests))
    assert any(not np.array_equal(x.doc_ids, y.doc_ids) for x, y in zip(a.requests, c.requests))
    pa, pb = a.prefill_batch(), b.prefill_batch()
    assert np.array_equal(pa["q"], pb["q"])


def test_decode_step_bookkeeping():
    wl = W.build_workload(W.spec(3, requests=[3], n_decode=20))
    q = wl.requests[0]
    for step in (0, 15, 16, 19):
        d = wl.decode_step(step)
        n_new = q.q_len + step + 1
        assert d["ctx_lens"][0] == q.ctx_docs + n_new
        assert d["num_entries"][0] == q.n_doc_entries + (n_new + 15) // 16
        b, row = wl.new_token_slot(q, q.q_len + step)
        assert d["slots"][0] == b * 16 + row
    hist = wl.tokens_before_step(5)
    assert hist["slots"].size == 3 * (q.q_len + 5)


def test_tokens_before_every_step_cover_each_step_token():
    # before step s: each decode request's suffix and steps 0..s-1, the same
    # values and slots as decode_step writes; s may be the number of decode steps
    # (every token written), where no decode step remains
    n = 6
    wl = W.build_workload(W.spec(3, requests=[3], n_decode=n))
    for s in (0, 1, n - 1, n, n + 3):
        hist = wl.tokens_before_step(s)
        q_len = wl.requests[0].q_len
        assert hist["slots"].size == 3 * (q_len + min(s, n))
        assert np.unique(hist["slots"]).size == hist["slots"].size
        for step in range(min(s, n)):
            d = wl.decode_step(step)
            for r in range(3):
                i = int(np.flatnonzero(hist["slots"] == d["slots"][r])[0])
                np.testing.assert_array_equal(hist["k_new"][i], d["k_new"][r])
                np.testing.assert_array_equal(hist["v_new"][i], d["v_new"][r])
    assert wl.decode_step(n) is None
