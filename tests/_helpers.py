"""Shared test plumbing: oracle-side state for a workload, and the parity bar."""
from __future__ import annotations

import numpy as np

import oracle as O

# Parity bar.  bf16: max |d| <= 1e-2 and mean |d| <= 1e-3; fp32: within 1e-4.
# A bf16 output cannot be closer to the exact value than half a bf16 ulp of
# that value (0.0156 once |value| >= 4), so the bf16 max bar is applied to the
# error beyond the output's own rounding: |d| - ulp_bf16(ref)/2 <= 1e-2.  For
# the diffuse outputs of long contexts (|ref| ~ 0.02) the allowance is < 1e-4.
TOL = {"bf16": (1e-2, 1e-3), "f32": (1e-4, 1e-4)}


def half_ulp(ref: np.ndarray, dtype: str) -> np.ndarray:
    if dtype != "bf16":
        return np.zeros_like(ref, dtype=np.float64)
    a = np.abs(np.asarray(ref, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)        # bf16 keeps 8 significant bits


def diff_stats(got: np.ndarray, ref: np.ndarray, dtype: str = None):
    """(max excess over the output rounding allowance, mean |d|); plain max |d| when dtype is None."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    d = np.abs(g - r)
    if d.size == 0:
        return 0.0, 0.0
    ex = d - half_ulp(r, dtype) if dtype else d
    return float(ex.max()), float(d.mean())


def within(got, ref, dtype) -> bool:
    mx, mn = diff_stats(got, ref, dtype)
    tmax, tmean = TOL[dtype]
    return bool(np.all(np.isfinite(got))) and mx <= tmax and mn <= tmean


# every assert_parity call appends (case, dtype, elements, raw max |d|, max excess
# over the rounding allowance, mean |d|, max |ref|); conftest writes them out
PARITY_RECORDS = []


def write_parity_records(path):
    with open(path, "a") as f:
        for r in PARITY_RECORDS:
            f.write("%-58s %-4s n=%-9d raw_max=%.3e excess_max=%.3e mean=%.3e ref_absmax=%.3g\n" % r)


def assert_parity(got, ref, dtype, what=""):
    mx, mn = diff_stats(got, ref, dtype)
    raw = float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)))) if np.size(got) else 0.0
    amax = float(np.max(np.abs(np.asarray(ref, np.float64)))) if np.size(ref) else 0.0
    PARITY_RECORDS.append((what[:58], dtype, int(np.size(got)), raw, mx, mn, amax))
    tmax, tmean = TOL[dtype]
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert mx <= tmax and mn <= tmean, (f"{what}: max |d| {raw:.3e} (beyond output rounding {mx:.3e}, bar {tmax}), "
                                        f"mean |d| {mn:.3e} (bar {tmean})")
    return raw, mn


class OracleState:
    """The oracle's own copy of a workload's pools, grown by its own appends."""

    def __init__(self, wl):
        self.wl = wl
        kp, vp = wl.pools()
        self.k, self.v = kp.copy(), vp.copy()

    def append(self, inputs):
        if inputs is not None:
            O.append_kv(self.k, self.v, inputs["k_new"], inputs["v_new"], inputs["slots"], self.wl.B)

    def words(self, inputs):
        return O.pack_table(inputs["table_blocks"], inputs["table_starts"])

    def prefill(self, inputs, token_subset=None, requests=None, pe=None, heads=None, q_shift=0,
                pair_perm=None, inv_freq=None):
        """Oracle prefill outputs {r: [tokens][heads][D]}; q_shift / pair_perm plant mistakes (controls)."""
        s = self.wl.spec
        words = self.words(inputs)
        q = inputs["q"]
        kp, vp = self.k, self.v
        ctx = inputs["ctx_lens"]
        if q_shift:                  # every query |q_shift| positions off, keys unchanged
            return self._shifted_prefill(inputs, token_subset, requests, pe, heads, q_shift)
        if pair_perm is not None:
            return self._permuted_prefill(inputs, token_subset, requests, pe, heads, pair_perm)
        return O.prefill(q=q, cu_q_lens=inputs["cu_q_lens"], ctx_lens=ctx, num_entries=inputs["num_entries"],
                         table_words=words, k_pool=kp, v_pool=vp, num_kv_heads=s.num_kv_heads,
                         block_size=s.block_size, dtype=s.dtype, pe=pe or s.pe, rope_theta=s.rope_theta,
                         requests=requests, heads=heads, token_subset=token_subset, inv_freq=inv_freq)

    def _contexts(self, inputs, r):
        s = self.wl.spec
        words = self.words(inputs)
        return O.gather_context(words[r], int(inputs["num_entries"][r]), int(inputs["ctx_lens"][r]),
                                self.k, self.v, s.block_size, s.dtype)

    def _shifted_prefill(self, inputs, token_subset, requests, pe, heads, shift):
        s = self.wl.spec
        res = {}
        reqs = range(len(inputs["ctx_lens"])) if requests is None else requests
        qf = O.to_f64(inputs["q"], s.dtype)
        for r in reqs:
            K, V, kp = self._contexts(inputs, r)
            a, b = int(inputs["cu_q_lens"][r]), int(inputs["cu_q_lens"][r + 1])
            local = np.arange(b - a) if token_subset is None else np.asarray(token_subset[r])
            qpos = int(inputs["ctx_lens"][r]) - (b - a) + local
            res[r] = O.attend(qf[a + local], qpos + shift, K, V, kp, pe=pe or s.pe, rope_theta=s.rope_theta,
                              heads=heads)
        return res

    def _permuted_prefill(self, inputs, token_subset, requests, pe, heads, perm):
        s = self.wl.spec
        res = {}
        reqs = range(len(inputs["ctx_lens"])) if requests is None else requests
        qf = O.to_f64(inputs["q"], s.dtype)
        for r in reqs:
            K, V, kp = self._contexts(inputs, r)
            a, b = int(inputs["cu_q_lens"][r]), int(inputs["cu_q_lens"][r + 1])
            local = np.arange(b - a) if token_subset is None else np.asarray(token_subset[r])
            qpos = int(inputs["ctx_lens"][r]) - (b - a) + local
            res[r] = O.attend(qf[a + local][..., perm], qpos, K[..., perm], V, kp, pe=pe or s.pe,
                              rope_theta=s.rope_theta, heads=heads)
        return res

    def decode(self, inputs, requests=None, pe=None, inv_freq=None):
        s = self.wl.spec
        return O.decode(q=inputs["q"], ctx_lens=inputs["ctx_lens"], num_entries=inputs["num_entries"],
                        table_words=self.words(inputs), k_pool=self.k, v_pool=self.v,
                        num_kv_heads=s.num_kv_heads, block_size=s.block_size, dtype=s.dtype, pe=pe or s.pe,
                        rope_theta=s.rope_theta, requests=requests, inv_freq=inv_freq)


def gpu_f64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


class OracleFp8State:
    """The oracle's own FP8 pools for a workload: every referenced document quantised by the
    oracle, grown by its own quantising appends; attention over the dequantised values.
    ``framed``: keys in document-local frames (attention through the framed definition)."""

    def __init__(self, wl, framed=False):
        self.wl = wl
        self.framed = framed
        s = wl.spec
        self.inv_freq = O.rope_inv_freq(s.head_dim, s.rope_theta)
        self.kc, self.vc = O.fp8_empty_pools(wl.num_blocks, s.num_kv_heads)
        for d in wl.referenced_docs:
            k, v = wl.doc_kv(int(d))
            slots, j = wl.doc_frame_tokens(int(d))
            O.append_kv_fp8(self.kc, self.vc, k, v, slots, s.dtype, frame_index=j if framed else None,
                            inv_freq=self.inv_freq)

    def append(self, inputs):
        if inputs is not None:
            O.append_kv_fp8(self.kc, self.vc, inputs["k_new"], inputs["v_new"], inputs["slots"], self.wl.spec.dtype,
                            frame_index=inputs["frame_index"] if self.framed else None, inv_freq=self.inv_freq)

    def _common(self, inputs):
        s = self.wl.spec
        return dict(ctx_lens=inputs["ctx_lens"], num_entries=inputs["num_entries"],
                    table_words=O.pack_table(inputs["table_blocks"], inputs["table_starts"]),
                    k_pool=O.Fp8PoolView(self.kc, "k"), v_pool=O.Fp8PoolView(self.vc, "v"),
                    num_kv_heads=s.num_kv_heads, block_size=s.block_size, dtype=s.dtype, pool_dtype="f64",
                    rope_theta=s.rope_theta)

    def prefill(self, inputs, token_subset=None, requests=None, pe=None):
        if self.framed:
            c = self._common(inputs)
            for key in ("num_kv_heads", "pool_dtype"):
                c.pop(key)
            c["dtype"] = self.wl.spec.dtype
            return O.prefill_framed(q=inputs["q"], cu_q_lens=inputs["cu_q_lens"], frame_starts=inputs["frame_starts"],
                                    token_subset=token_subset, requests=requests, **c)
        return O.prefill(q=inputs["q"], cu_q_lens=inputs["cu_q_lens"], pe=pe or self.wl.spec.pe,
                         token_subset=token_subset, requests=requests, **self._common(inputs))

    def decode(self, inputs, requests=None, pe=None):
        if self.framed:
            c = self._common(inputs)
            for key in ("num_kv_heads", "pool_dtype"):
                c.pop(key)
            return O.decode_framed(q=inputs["q"], frame_starts=inputs["frame_starts"], requests=requests, **c)
        return O.decode(q=inputs["q"], pe=pe or self.wl.spec.pe, requests=requests, **self._common(inputs))
