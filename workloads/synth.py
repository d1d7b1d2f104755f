"""Seeded synthetic workloads: a document pool, Zipf-skewed retrieval and new tokens.

The LazyAttention pages measure on RAG question-answering suites with
Llama-3.1-8B/70B; none of that is used here.  Instead every input is drawn
from seeded numpy streams with the attention-layer shapes of those models:

* documents hold K/V ~ N(0, 1), rounded to bfloat16 (or kept in float32 for the
  tiny fp32 case), stored **unrotated** (content only);
* each document occupies whole physical blocks of ``block_size`` tokens, its
  last block possibly partial (padding rows hold NaN as a poison check);
* each request retrieves distinct documents drawn with Zipf skew
  (P(rank k) proportional to k**-s, sequential renormalised sampling without
  replacement, then a uniform random order) and concatenates them densely at
  logical positions 0, len0, len0+len1, ...;
* the request's new tokens (query suffix and decode tokens) get private
  blocks taken from the tail of the pool, the first one starting at the end
  of the documents, whatever its alignment.

Streams (``numpy.random.SeedSequence`` entropy lists):
  [cfg, 1]               document lengths
  [cfg, 3]               physical placement of document blocks
  [cfg, 6, doc]          one document's K then V
  [cfg, sweep, 2]        documents per request, draws and order
  [cfg, sweep, 7]        physical placement of private blocks
  [cfg, sweep, 4, r, ph] request r's queries; phase 0 = prefill, 1+s = decode step s
  [cfg, sweep, 5, r, ph] request r's new-token K then V, same phases

Nothing here computes attention, rotates a vector or packs a table word.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


# ----------------------------------------------------------------------------
# bfloat16 as 16-bit patterns (numpy has no bfloat16 dtype)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    out = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    out[np.isnan(x)] = BF16_NAN
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# specifications
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class GroupSpec:
    """A group of requests sharing a shape of work."""
    n_requests: int
    docs_lo: int          # documents per request, uniform on [docs_lo, docs_hi]
    docs_hi: int
    q_len: int            # new tokens prefilled in one call (0: decode-only)
    n_decode: int         # single-token decode steps after the prefill


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    name: str
    cfg_id: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str                      # "bf16" or "f32"
    rope_theta: float
    pe: str                         # "rope", "none" or "alibi"
    n_docs_pool: int
    doc_len: Optional[int]          # fixed document length, or None for lognormal
    doc_len_lognormal: Optional[tuple] = None   # (median, sigma, lo, hi)
    zipf_s: float = 0.0             # 0 means uniform
    groups: tuple = ()
    sweep: int = 0

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def _cfg(cfg_id: int) -> WorkloadSpec:
    if cfg_id == 1:
        # tiny single-head fp32 case: 4 documents of 32 tokens in shuffled order,
        # a 16-token causal prefill, then 8 decode steps
        return WorkloadSpec("tiny-f32-d64", 1, 1, 1, 64, 16, "f32", 10000.0, "rope",
                            n_docs_pool=4, doc_len=32, zipf_s=0.0,
                            groups=(GroupSpec(1, 4, 4, 16, 8),))
    if cfg_id == 2:
        # Llama-3.1-8B attention shape, bf16 prefill over ~4.2k tokens
        return WorkloadSpec("llama8b-prefill-16x(8x512)+64", 2, 32, 8, 128, 16, "bf16", 500000.0, "rope",
                            n_docs_pool=256, doc_len=512, zipf_s=1.0,
                            groups=(GroupSpec(16, 8, 8, 64, 0),))
    if cfg_id == 3:
        # Llama-3.1-8B shape decode: 128 requests, 32-token suffix then 256 steps
        return WorkloadSpec("llama8b-decode-128x(8x512)+32+256", 3, 32, 8, 128, 16, "bf16", 500000.0, "rope",
                            n_docs_pool=1024, doc_len=512, zipf_s=1.2,
                            groups=(GroupSpec(128, 8, 8, 32, 256),))
    if cfg_id == 4:
        # Llama-3.1-70B single-layer shape, 32k context, 2048-token chunk then 128 steps
        return WorkloadSpec("llama70b-32k-4x(64x512)+2048+128", 4, 64, 8, 128, 16, "bf16", 500000.0, "rope",
                            n_docs_pool=4096, doc_len=512, zipf_s=1.0,
                            groups=(GroupSpec(4, 64, 64, 2048, 128),))
    if cfg_id == 5:
        # MQA stress: lognormal documents, 32 prefill requests + 96 decode requests
        return WorkloadSpec("mqa-stress-lognormal", 5, 32, 1, 128, 16, "bf16", 10000.0, "rope",
                            n_docs_pool=1024, doc_len=None,
                            doc_len_lognormal=(300.0, 1.0, 64, 2048), zipf_s=1.2,
                            groups=(GroupSpec(32, 4, 32, 128, 0), GroupSpec(96, 4, 32, 0, 8)))
    raise ValueError(f"unknown config {cfg_id}")


CONFIGS = (1, 2, 3, 4, 5)
CFG5_SKEWS = (0.0, 0.8, 1.2, 1.6)
CFG5_PES = ("rope", "alibi")


def spec(cfg_id: int, *, skew: Optional[float] = None, pe: Optional[str] = None,
         requests: Optional[Sequence[int]] = None, n_decode: Optional[int] = None,
         q_len: Optional[int] = None, dtype: Optional[str] = None,
         n_docs_pool: Optional[int] = None, docs: Optional[tuple] = None,
         doc_len: Optional[int] = None) -> WorkloadSpec:
    """A config's spec, optionally with a sweep point or a reduced size.

    ``skew``/``pe`` select a sweep point (used by the MQA stress case; the
    sweep index is derived from them so that streams differ per point).
    ``requests`` gives the request count per group, ``n_decode``/``q_len``
    override every group's, ``docs`` = (lo, hi) documents per request.
    """
    s = _cfg(cfg_id)
    changes = {}
    sweep = 0
    if skew is not None:
        changes["zipf_s"] = float(skew)
        sweep += 1 + int(round(skew * 10))
    if pe is not None:
        changes["pe"] = pe
        sweep += 100 * (("rope", "none", "alibi").index(pe))
    if dtype is not None:
        changes["dtype"] = dtype
    if n_docs_pool is not None:
        changes["n_docs_pool"] = n_docs_pool
    if doc_len is not None:
        changes["doc_len"] = doc_len
        changes["doc_len_lognormal"] = None
    groups = list(s.groups)
    for i, g in enumerate(groups):
        kw = {}
        if requests is not None:
            kw["n_requests"] = int(requests[i])
        if n_decode is not None:
            kw["n_decode"] = int(n_decode)
        if q_len is not None and g.q_len > 0:
            kw["q_len"] = int(q_len)
        if docs is not None:
            kw["docs_lo"], kw["docs_hi"] = int(docs[0]), int(docs[1])
        groups[i] = dataclasses.replace(g, **kw)
    changes["groups"] = tuple(g for g in groups if g.n_requests > 0)
    changes["sweep"] = sweep
    return dataclasses.replace(s, **changes)


# ----------------------------------------------------------------------------
# pool storage
# ----------------------------------------------------------------------------
class SparsePool:
    """A block pool of which only some blocks were ever written.

    Indexing along axis 0 with physical block ids returns whole blocks; blocks
    never written read as NaN.  ``dense()`` materialises the full array.
    Layout of one block: ``block_shape`` (K: [Hkv][B][D], V: [Hkv][D][B]).
    """

    def __init__(self, num_blocks: int, block_shape: tuple, ids: np.ndarray, data: np.ndarray, nan_bits):
        self.num_blocks = int(num_blocks)
        self.block_shape = tuple(block_shape)
        self.ids = np.asarray(ids, dtype=np.int64)
        self.data = data
        self.nan = nan_bits
        self.lookup = np.full(self.num_blocks, -1, dtype=np.int64)
        self.lookup[self.ids] = np.arange(self.ids.size)

    @property
    def shape(self):
        return (self.num_blocks,) + self.block_shape

    @property
    def dtype(self):
        return self.data.dtype

    def _rows(self, ids):
        ids = np.asarray(ids, dtype=np.int64)
        if np.any(ids < 0) or np.any(ids >= self.num_blocks):
            raise IndexError("physical block id out of range")
        return ids, self.lookup[ids]

    def __getitem__(self, ids):
        ids, rows = self._rows(ids)
        out = np.empty(ids.shape + self.block_shape, dtype=self.data.dtype)
        out[...] = self.nan
        have = rows >= 0
        out[have] = self.data[rows[have]]
        return out

    def __setitem__(self, ids, values):
        ids, rows = self._rows(ids)
        if np.any(rows < 0):
            raise KeyError("block was not allocated in this sparse pool")
        self.data[rows] = values

    def copy(self) -> "SparsePool":
        return SparsePool(self.num_blocks, self.block_shape, self.ids.copy(), self.data.copy(), self.nan)

    def dense(self) -> np.ndarray:
        out = np.empty(self.shape, dtype=self.data.dtype)
        out[...] = self.nan
        out[self.ids] = self.data
        return out


# ----------------------------------------------------------------------------
# the workload
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class RequestLayout:
    index: int
    doc_ids: np.ndarray        # documents in context order
    doc_lens: np.ndarray
    entry_blocks: np.ndarray   # uint32, every entry including all private blocks
    entry_starts: np.ndarray   # uint32 logical start of each entry
    n_doc_entries: int
    ctx_docs: int              # tokens of retrieved documents
    q_len: int
    n_decode: int
    private_blocks: np.ndarray

    def num_entries_after(self, n_new: int) -> int:
        """Entries in use once ``n_new`` private tokens have been written."""
        return self.n_doc_entries + (n_new + self.block_size - 1) // self.block_size

    block_size: int = 16


def _zipf_draw(rng: np.random.Generator, n_pool: int, n: int, s: float) -> np.ndarray:
    """n distinct documents, sequentially renormalised P(rank k) ~ k^-s, then shuffled."""
    w = np.arange(1, n_pool + 1, dtype=np.float64) ** (-float(s))
    taken = np.zeros(n_pool, dtype=bool)
    out = np.empty(n, dtype=np.int64)
    for i in range(n):
        p = np.where(taken, 0.0, w)
        cdf = np.cumsum(p)
        u = rng.random() * cdf[-1]
        k = int(np.searchsorted(cdf, u, side="right"))
        k = min(k, n_pool - 1)
        while taken[k]:          # guard against u landing on a zero-width bin edge
            k -= 1
        taken[k] = True
        out[i] = k
    return out[rng.permutation(n)]


class Workload:
    """All inputs of one config, generated lazily from seeded streams."""

    def __init__(self, s: WorkloadSpec):
        self.spec = s
        B, Hkv, D = s.block_size, s.num_kv_heads, s.head_dim
        self.B, self.Hkv, self.D, self.Hq = B, Hkv, D, s.num_q_heads
        self.is_bf16 = s.dtype == "bf16"

        # document lengths
        rl = np.random.default_rng(np.random.SeedSequence([s.cfg_id, 1]))
        if s.doc_len is not None:
            doc_lens = np.full(s.n_docs_pool, s.doc_len, dtype=np.int64)
        else:
            med, sig, lo, hi = s.doc_len_lognormal
            raw = np.exp(rl.normal(np.log(med), sig, size=s.n_docs_pool))
            doc_lens = np.clip(np.rint(raw), lo, hi).astype(np.int64)
        self.doc_lens = doc_lens
        doc_nblk = (doc_lens + B - 1) // B
        self.doc_first = np.concatenate([[0], np.cumsum(doc_nblk)[:-1]])
        n_doc_blocks = int(doc_nblk.sum())
        rp = np.random.default_rng(np.random.SeedSequence([s.cfg_id, 3]))
        self.doc_block_perm = rp.permutation(n_doc_blocks).astype(np.int64)
        self.doc_nblk = doc_nblk

        # requests
        rd = np.random.default_rng(np.random.SeedSequence([s.cfg_id, s.sweep, 2]))
        self.requests: list[RequestLayout] = []
        n_private_total = 0
        req_specs = []
        for g in s.groups:
            for _ in range(g.n_requests):
                n = int(rd.integers(g.docs_lo, g.docs_hi + 1))
                docs = _zipf_draw(rd, s.n_docs_pool, n, s.zipf_s)
                n_priv = (g.q_len + g.n_decode + B - 1) // B
                req_specs.append((docs, g, n_priv))
                n_private_total += n_priv
        rpp = np.random.default_rng(np.random.SeedSequence([s.cfg_id, s.sweep, 7]))
        priv_ids = n_doc_blocks + rpp.permutation(n_private_total).astype(np.int64)
        self.num_blocks = n_doc_blocks + n_private_total
        self.n_doc_blocks = n_doc_blocks

        cursor = 0
        for r, (docs, g, n_priv) in enumerate(req_specs):
            blocks, starts = [], []
            pos = 0
            for d in docs:
                L = int(doc_lens[d])
                phys = self.doc_blocks(int(d))
                for j in range(phys.size):
                    blocks.append(int(phys[j]))
                    starts.append(pos + j * B)
                pos += L
            n_doc_entries = len(blocks)
            priv = priv_ids[cursor:cursor + n_priv]
            cursor += n_priv
            for j in range(n_priv):
                blocks.append(int(priv[j]))
                starts.append(pos + j * B)
            self.requests.append(RequestLayout(
                index=r, doc_ids=np.asarray(docs), doc_lens=doc_lens[docs],
                entry_blocks=np.asarray(blocks, dtype=np.uint32),
                entry_starts=np.asarray(starts, dtype=np.uint32),
                n_doc_entries=n_doc_entries, ctx_docs=pos, q_len=g.q_len,
                n_decode=g.n_decode, private_blocks=priv, block_size=B))

        self.referenced_docs = np.unique(np.concatenate([q.doc_ids for q in self.requests])) \
            if self.requests else np.zeros(0, dtype=np.int64)
        self._pools = None

    # ------------------------------------------------------------------
    def doc_blocks(self, d: int) -> np.ndarray:
        f = int(self.doc_first[d])
        return self.doc_block_perm[f:f + int(self.doc_nblk[d])]

    def _values(self, rng: np.random.Generator, shape) -> np.ndarray:
        x = rng.standard_normal(size=shape, dtype=np.float32)
        return f32_to_bf16_bits(x) if self.is_bf16 else x

    @property
    def nan_value(self):
        return BF16_NAN if self.is_bf16 else np.float32(np.nan)

    def doc_kv(self, d: int):
        """Document d's K and V, each [len][Hkv][D] (bf16 bits or float32)."""
        rng = np.random.default_rng(np.random.SeedSequence([self.spec.cfg_id, 6, int(d)]))
        L = int(self.doc_lens[d])
        k = self._values(rng, (L, self.Hkv, self.D))
        v = self._values(rng, (L, self.Hkv, self.D))
        return k, v

    def pools(self):
        """(K pool, V pool) as SparsePool: referenced documents written, private blocks NaN.

        K block layout [Hkv][B][D] (token rows, channels contiguous);
        V block layout [Hkv][D][B] (channel rows, tokens contiguous).
        """
        if self._pools is not None:
            return self._pools
        B, Hkv, D = self.B, self.Hkv, self.D
        dt = np.uint16 if self.is_bf16 else np.float32
        ids = [self.doc_blocks(int(d)) for d in self.referenced_docs]
        ids += [q.private_blocks for q in self.requests]
        ids = np.concatenate(ids).astype(np.int64) if ids else np.zeros(0, np.int64)
        kd = np.empty((ids.size, Hkv, B, D), dtype=dt)
        vd = np.empty((ids.size, Hkv, D, B), dtype=dt)
        kd[...] = self.nan_value
        vd[...] = self.nan_value
        row = 0
        for d in self.referenced_docs:
            k, v = self.doc_kv(int(d))
            L = k.shape[0]
            nb = (L + B - 1) // B
            kp = np.empty((nb * B, Hkv, D), dtype=dt)
            vp = np.empty((nb * B, Hkv, D), dtype=dt)
            kp[...] = self.nan_value
            vp[...] = self.nan_value
            kp[:L] = k
            vp[:L] = v
            kd[row:row + nb] = kp.reshape(nb, B, Hkv, D).transpose(0, 2, 1, 3)
            vd[row:row + nb] = vp.reshape(nb, B, Hkv, D).transpose(0, 2, 3, 1)
            row += nb
        kpool = SparsePool(self.num_blocks, (Hkv, B, D), ids, kd, self.nan_value)
        vpool = SparsePool(self.num_blocks, (Hkv, D, B), ids, vd, self.nan_value)
        self._pools = (kpool, vpool)
        return self._pools

    # ------------------------------------------------------------------
    def _phase_rng(self, kind: int, r: int, phase: int):
        s = self.spec
        return np.random.default_rng(np.random.SeedSequence([s.cfg_id, s.sweep, kind, r, phase]))

    def new_token_slot(self, req: RequestLayout, i: int) -> tuple:
        """(physical block, row) of the request's i-th new token."""
        return int(req.private_blocks[i // self.B]), i % self.B

    def table_arrays(self, reqs: Sequence[RequestLayout]):
        """Per-request entry lists padded to a common width: (blocks, starts) uint32 [R][E_max].

        Padding entries hold block 0 and start 0x7fffffff; they are never in use.
        """
        e_max = max(int(q.entry_blocks.size) for q in reqs)
        blocks = np.zeros((len(reqs), e_max), dtype=np.uint32)
        starts = np.full((len(reqs), e_max), 0x7FFFFFFF, dtype=np.uint32)
        for i, q in enumerate(reqs):
            blocks[i, :q.entry_blocks.size] = q.entry_blocks
            starts[i, :q.entry_starts.size] = q.entry_starts
        return blocks, starts

    def frame_arrays(self, reqs: Sequence[RequestLayout]) -> np.ndarray:
        """Frame start of every table entry, int32 [R][E_max], for a pool in
        document-local frames: a document's entries carry the document's first
        logical position in that request, the request's private entries carry
        the first position after its documents (ctx_docs).  Padding: 0."""
        e_max = max(int(q.entry_blocks.size) for q in reqs)
        out = np.zeros((len(reqs), e_max), dtype=np.int32)
        for i, q in enumerate(reqs):
            col, pos = 0, 0
            for L in q.doc_lens:
                nb = (int(L) + self.B - 1) // self.B
                out[i, col:col + nb] = pos
                col += nb
                pos += int(L)
            out[i, col:q.entry_blocks.size] = q.ctx_docs
        return out

    def doc_frame_tokens(self, d: int):
        """(slots, frame_index) of document d's tokens: pool slot block * B + row, and
        the token's index within the document."""
        L = int(self.doc_lens[d])
        j = np.arange(L, dtype=np.int64)
        return self.doc_blocks(int(d))[j // self.B] * self.B + j % self.B, j.astype(np.int32)

    def prefill_batch(self) -> dict:
        """Inputs of one prefill call over every request with a query suffix."""
        reqs = [q for q in self.requests if q.q_len > 0]
        if not reqs:
            return None
        qs, ks, vs, slots, fidx = [], [], [], [], []
        for q in reqs:
            rq = self._phase_rng(4, q.index, 0)
            qs.append(self._values(rq, (q.q_len, self.Hq, self.D)))
            rk = self._phase_rng(5, q.index, 0)
            ks.append(self._values(rk, (q.q_len, self.Hkv, self.D)))
            vs.append(self._values(rk, (q.q_len, self.Hkv, self.D)))
            for i in range(q.q_len):
                b, row = self.new_token_slot(q, i)
                slots.append(b * self.B + row)
                fidx.append(i)
        q_lens = np.array([q.q_len for q in reqs], dtype=np.int32)
        blocks, starts = self.table_arrays(reqs)
        return dict(
            requests=reqs,
            q=np.concatenate(qs), k_new=np.concatenate(ks), v_new=np.concatenate(vs),
            slots=np.asarray(slots, dtype=np.int64), frame_index=np.asarray(fidx, dtype=np.int32),
            cu_q_lens=np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32),
            ctx_lens=np.array([q.ctx_docs + q.q_len for q in reqs], dtype=np.int32),
            num_entries=np.array([q.num_entries_after(q.q_len) for q in reqs], dtype=np.int32),
            table_blocks=blocks, table_starts=starts, frame_starts=self.frame_arrays(reqs),
            max_q_len=int(q_lens.max()), total_q=int(q_lens.sum()),
        )

    def tokens_before_step(self, step: int) -> Optional[dict]:
        """Every new token of the decode requests written before decode step ``step``:
        their prefill suffix and their decode steps 0..step-1 (a request with fewer
        decode steps contributes all of its own; ``step`` may be the number of decode
        steps, i.e. every token written), as one batch of (k, v, slots)."""
        reqs = [q for q in self.requests if q.n_decode > 0]
        ks, vs, slots, fidx = [], [], [], []
        for q in reqs:
            if q.q_len > 0:
                rk = self._phase_rng(5, q.index, 0)
                ks.append(self._values(rk, (q.q_len, self.Hkv, self.D)))
                vs.append(self._values(rk, (q.q_len, self.Hkv, self.D)))
                for i in range(q.q_len):
                    b, row = self.new_token_slot(q, i)
                    slots.append(b * self.B + row)
                    fidx.append(i)
            for s in range(min(step, q.n_decode)):
                rk = self._phase_rng(5, q.index, 1 + s)
                ks.append(self._values(rk, (1, self.Hkv, self.D)))
                vs.append(self._values(rk, (1, self.Hkv, self.D)))
                b, row = self.new_token_slot(q, q.q_len + s)
                slots.append(b * self.B + row)
                fidx.append(q.q_len + s)
        if not slots:
            return None
        return dict(k_new=np.concatenate(ks), v_new=np.concatenate(vs),
                    slots=np.asarray(slots, dtype=np.int64), frame_index=np.asarray(fidx, dtype=np.int32))

    def decode_requests(self, step: int) -> list:
        return [q for q in self.requests if q.n_decode > step]

    def decode_step(self, step: int) -> dict:
        """Inputs of decode step ``step`` (0-based): the new token is appended, then attends."""
        reqs = self.decode_requests(step)
        if not reqs:
            return None
        qs, ks, vs, slots = [], [], [], []
        for q in reqs:
            rq = self._phase_rng(4, q.index, 1 + step)
            qs.append(self._values(rq, (self.Hq, self.D)))
            rk = self._phase_rng(5, q.index, 1 + step)
            ks.append(self._values(rk, (self.Hkv, self.D)))
            vs.append(self._values(rk, (self.Hkv, self.D)))
            b, row = self.new_token_slot(q, q.q_len + step)
            slots.append(b * self.B + row)
        blocks, starts = self.table_arrays(reqs)
        n_new = [q.q_len + step + 1 for q in reqs]
        return dict(
            requests=reqs,
            q=np.stack(qs), k_new=np.stack(ks), v_new=np.stack(vs),
            slots=np.asarray(slots, dtype=np.int64),
            frame_index=np.array([q.q_len + step for q in reqs], dtype=np.int32),
            ctx_lens=np.array([q.ctx_docs + n for q, n in zip(reqs, n_new)], dtype=np.int32),
            num_entries=np.array([q.num_entries_after(n) for q, n in zip(reqs, n_new)], dtype=np.int32),
            table_blocks=blocks, table_starts=starts, frame_starts=self.frame_arrays(reqs),
        )


def build_workload(s: WorkloadSpec) -> Workload:
    return Workload(s)


# ----------------------------------------------------------------------------
# request traces for the block-pool hit-ratio simulation
# ----------------------------------------------------------------------------
def cache_trace(n_docs_pool: int, n_requests: int, docs_per_request: tuple, zipf_s: float, seed: int,
                doc_len: int = 512, doc_len_lognormal: Optional[tuple] = None):
    """A seeded stream of retrieval requests: (doc_ids int64 [N], doc_lens int32 [N], req_offsets int64 [R+1]).

    Each request retrieves between docs_per_request[0] and [1] distinct documents, Zipf(zipf_s) over
    the pool's popularity ranks (sequentially renormalised, without replacement), in random order.
    Document lengths are fixed, or lognormal (median, sigma, lo, hi) per document.
    """
    rl = np.random.default_rng(np.random.SeedSequence([seed, 1]))
    if doc_len_lognormal is None:
        lens = np.full(n_docs_pool, doc_len, dtype=np.int32)
    else:
        med, sig, lo, hi = doc_len_lognormal
        lens = np.clip(np.rint(np.exp(rl.normal(np.log(med), sig, size=n_docs_pool))), lo, hi).astype(np.int32)
    rd = np.random.default_rng(np.random.SeedSequence([seed, 2]))
    ids, offs = [], [0]
    for _ in range(n_requests):
        n = int(rd.integers(docs_per_request[0], docs_per_request[1] + 1))
        d = _zipf_draw(rd, n_docs_pool, n, zipf_s)
        ids.append(d)
        offs.append(offs[-1] + n)
    doc_ids = np.concatenate(ids).astype(np.int64) if ids else np.zeros(0, np.int64)
    return doc_ids, lens[doc_ids].astype(np.int32), np.asarray(offs, dtype=np.int64)
