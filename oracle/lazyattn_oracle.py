"""fp64 CPU oracle for attention over a position-agnostic (content-only) KV pool.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the package smoke check and the
benchmark's CPU-baseline leg may import or call this module; the library
never does, and this module imports nothing from the library (numpy only).

Sources.  The method is LazyAttention (arXiv 2606.04302).  Citations name the
web page and its section:
  [abstract]  shd-paper.top digest of "LazyAttention: Efficient Retrieval-
              Augmented Generation with Deferred Positional Encoding", the
              original English abstract;
  [gist:X]    gist.science explainer of the same paper, Technical Summary,
              section X (Methodology, Technical Implementation / Prefilling,
              Technical Implementation / Decoding, Mathematical Equivalence,
              Key Contributions).

What is computed (the definition).  A request's context is a dense run of
logical positions 0..L-1 assembled from cached documents and the request's
own new tokens.  The cache holds content-only keys and values: no position
is baked into them [gist:Methodology].  The result of attention must be the
same as if every key had been rotated with RoPE at its logical position and
stored that way ("materialised"), which is what the pages prove the deferred
kernel equals [gist:Mathematical Equivalence].  So the definition used here
is the materialised one:

  1. decode each table word into (physical block, logical start) and derive
     each entry's valid length from the next entry's start (or L);
  2. gather k_t, v_t of every logical token t from the pool;
  3. rotate every key at its own position t and every query at its position p
     (RoPE, interleaved channel pairs, inv_freq_i = theta^(-2i/D));
  4. score z_t = scale * <q'_p, k'_t> for t <= p, softmax over t, output the
     softmax-weighted sum of v_t.

A second, separate formulation (``formulation="deferred"``) never rotates
the query and rotates each stored key by the relative offset t - p only,
z_t = scale * q_p^T R(t - p) k_t, which is the deferred scheme the pages
describe; the tests require the two to agree to ~1e-12.

Readings where the pages are silent (each is listed in the design notes):
  * RoPE channel pairs are interleaved (2i, 2i+1); frequencies are the plain
    theta^(-2i/D) without any long-context rescaling;
  * the pool stores keys unrotated (content only);
  * a query at logical position p sees keys t <= p (itself included); the
    new tokens of a call are the last positions of the context and their
    K/V are appended to private blocks before the call;
  * query head h reads kv-head h // G (contiguous GQA groups);
  * table word = (logical start << 32) | physical block id;
  * ALiBi: no rotation and bias -slope_h * (p - t), slope_h = 2^(-8(h+1)/Hq);
  * softmax scale defaults to 1/sqrt(D).

Pool layouts (the library's documented input format):
  K pool [num_blocks][Hkv][B][D]   token rows, channels contiguous
  V pool [num_blocks][Hkv][D][B]   channel rows, tokens contiguous
Values are bfloat16 bit patterns (uint16) or float32.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "pack_entry", "unpack_entry", "pack_table", "decode_table", "TableError",
    "bf16_to_f64", "to_f64", "rope_inv_freq", "rope_rotate", "alibi_slopes",
    "gather_context", "attend", "prefill", "decode", "append_kv",
    "brute_force_attention", "rotation_flop_fraction", "tile_flop_counts",
    "rotate_into_frames", "append_kv_framed", "token_frames", "attend_framed", "prefill_framed",
    "decode_framed", "rope_inv_freq_partial", "rope_inv_freq_llama31", "BlockCache",
    "e4m3_value", "e4m3_encode", "fp8_row_exponent", "quantize_fp8_rows", "fp8_empty_pools",
    "append_kv_fp8", "Fp8PoolView", "FP8_CHUNK",
]


# ---------------------------------------------------------------------------
# 1. block-table words
#    [gist:Technical Implementation / Decoding]: per-block metadata
#    (block ID, offset) is bit-packed into one register-sized word.
#    Reading: a 64-bit word, logical start in the high 32 bits, block id in
#    the low 32 bits, so a request's words ascend with position.
# ---------------------------------------------------------------------------
class TableError(ValueError):
    """A block table that breaks the dense contract."""

    def __init__(self, msg, entry=None):
        super().__init__(msg)
        self.entry = entry


def pack_entry(block_id: int, start: int) -> int:
    if not (0 <= block_id < 2**32 and 0 <= start < 2**32):
        raise ValueError("block id and start must fit in 32 bits")
    return (int(start) << 32) | int(block_id)


def unpack_entry(word: int) -> tuple:
    w = int(word)
    return w & 0xFFFFFFFF, (w >> 32) & 0xFFFFFFFF


def pack_table(blocks: np.ndarray, starts: np.ndarray) -> np.ndarray:
    """Element-wise pack of uint32 arrays into uint64 words."""
    b = np.asarray(blocks, dtype=np.uint64)
    s = np.asarray(starts, dtype=np.uint64)
    return (s << np.uint64(32)) | b


def decode_table(words: Sequence[int], n_entries: int, ctx_len: int, block_size: int,
                 num_blocks: int):
    """(blocks, starts, lens) of a request's first ``n_entries`` words.

    Dense contract: the first start is 0; every entry holds 1..block_size
    valid tokens, its length being the next start minus its own (the last
    one runs to ``ctx_len``); every block id is below ``num_blocks``.
    """
    blocks, starts = [], []
    for e in range(int(n_entries)):
        b, s = unpack_entry(words[e])
        blocks.append(b)
        starts.append(s)
    if n_entries <= 0:
        if ctx_len != 0:
            raise TableError("empty table with a non-empty context")
        return np.zeros(0, np.int64), np.zeros(0, np.int64), np.zeros(0, np.int64)
    ends = starts[1:] + [int(ctx_len)]
    lens = [e - s for s, e in zip(starts, ends)]
    if starts[0] != 0:
        raise TableError("first entry must start at logical position 0", 0)
    for e in range(len(blocks)):
        if not (1 <= lens[e] <= block_size):
            raise TableError(f"entry {e} holds {lens[e]} tokens", e)
        if blocks[e] >= num_blocks:
            raise TableError(f"entry {e} names block {blocks[e]} >= {num_blocks}", e)
    return (np.asarray(blocks, np.int64), np.asarray(starts, np.int64), np.asarray(lens, np.int64))


# ---------------------------------------------------------------------------
# 2. value conversion
# ---------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64, exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# 3. RoPE  ([gist:Methodology] names RoPE as the encoding that is deferred)
# ---------------------------------------------------------------------------
def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """inv_freq_i = theta^(-2i/D), i = 0..D/2-1, in float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / head_dim)


def rope_inv_freq_partial(head_dim: int, rotary_dim: int, theta: float) -> np.ndarray:
    """Partial rotary: the first rotary_dim/2 pairs use theta^(-2i/rotary_dim), the rest do not turn.

    ([gist:Key Contributions] names RoPE variants as compatible.)  rotary_dim == head_dim is plain RoPE.
    """
    f = np.zeros(head_dim // 2, dtype=np.float64)
    i = np.arange(rotary_dim // 2, dtype=np.float64)
    f[:rotary_dim // 2] = np.power(float(theta), -2.0 * i / rotary_dim)
    return f


def rope_inv_freq_llama31(head_dim: int, theta: float, factor: float, low_freq_factor: float,
                          high_freq_factor: float, original_max_position: int) -> np.ndarray:
    """The frequency rescaling published with the Llama 3.1 models, written per pair from its definition.

    A base frequency f (wavelength 2 pi / f) is kept when its wavelength is shorter than
    original_max_position / high_freq_factor, divided by ``factor`` when longer than
    original_max_position / low_freq_factor, and otherwise blended linearly between f / factor and f
    with weight s = (original_max_position / wavelength - low_freq_factor) / (high_freq_factor - low_freq_factor).
    """
    base = rope_inv_freq(head_dim, theta)
    out = np.empty_like(base)
    for i, f in enumerate(base):
        wavelength = 2.0 * math.pi / f
        if wavelength < original_max_position / high_freq_factor:
            out[i] = f
        elif wavelength > original_max_position / low_freq_factor:
            out[i] = f / factor
        else:
            s = (original_max_position / wavelength - low_freq_factor) / (high_freq_factor - low_freq_factor)
            out[i] = (1.0 - s) * f / factor + s * f
    return out


def rope_rotate(x: np.ndarray, pos, inv_freq: np.ndarray) -> np.ndarray:
    """Rotate each interleaved channel pair (2i, 2i+1) of x[..., D] by pos * inv_freq_i.

    ``pos`` broadcasts against x's leading axes (it may be negative or
    fractional).  x'_{2i} = x_{2i} cos - x_{2i+1} sin,
    x'_{2i+1} = x_{2i} sin + x_{2i+1} cos.
    """
    x = np.asarray(x, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    even, odd = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, c.shape[:-1] + (x.shape[-1],)), dtype=np.float64)
    out[..., 0::2] = even * c - odd * s
    out[..., 1::2] = even * s + odd * c
    return out


def alibi_slopes(num_heads: int) -> np.ndarray:
    """ALiBi head slopes 2^(-8(h+1)/H), h = 0..H-1 ([gist:Key Contributions] names ALiBi)."""
    h = np.arange(num_heads, dtype=np.float64)
    return np.power(2.0, -8.0 * (h + 1.0) / num_heads)


# ---------------------------------------------------------------------------
# 4. gather a request's context through its table
# ---------------------------------------------------------------------------
def gather_context(words, n_entries, ctx_len, k_pool, v_pool, block_size, dtype):
    """K, V [L][Hkv][D] in float64 and the logical position of each row.

    Logical token t with start_e <= t < start_e + len_e lives in pool slot
    (block_e, t - start_e).  ``k_pool``/``v_pool`` index by physical block id
    along axis 0 (numpy arrays or any object doing so).
    """
    num_blocks = k_pool.shape[0]
    blocks, starts, lens = decode_table(words, n_entries, ctx_len, block_size, num_blocks)
    if blocks.size == 0:
        hk = k_pool.shape[1]
        d = k_pool.shape[3]
        return np.zeros((0, hk, d)), np.zeros((0, hk, d)), np.zeros(0, np.int64)
    kb = to_f64(k_pool[blocks], dtype)   # [E][Hkv][B][D]
    vb = to_f64(v_pool[blocks], dtype)   # [E][Hkv][D][B]
    ks, vs, pos = [], [], []
    for e in range(blocks.size):
        n = int(lens[e])
        ks.append(kb[e, :, :n, :].transpose(1, 0, 2))   # [n][Hkv][D]
        vs.append(vb[e, :, :, :n].transpose(2, 0, 1))   # [n][Hkv][D]
        pos.append(starts[e] + np.arange(n))
    K = np.concatenate(ks)
    V = np.concatenate(vs)
    P = np.concatenate(pos)
    if P.size != ctx_len or np.any(P != np.arange(ctx_len)):
        raise TableError("table does not cover positions 0..L-1 densely")
    return K, V, P


# ---------------------------------------------------------------------------
# 5. attention for one request
# ---------------------------------------------------------------------------
def attend(q: np.ndarray, q_pos: np.ndarray, K: np.ndarray, V: np.ndarray, k_pos: np.ndarray, *,
           pe: str, rope_theta: float = 10000.0, softmax_scale: Optional[float] = None,
           slopes: Optional[np.ndarray] = None, formulation: str = "materialized",
           heads: Optional[Sequence[int]] = None, return_weights: bool = False,
           inv_freq: Optional[np.ndarray] = None):
    """Causal attention of queries q [M][Hq][D] at positions q_pos over keys K, V [L][Hkv][D].

    Returns out [M][Hq][D] (only ``heads`` if given, in that order along
    axis 1) and, if asked, the weights [M][H][L].  ``inv_freq`` [D/2]
    replaces the theta^(-2i/D) table (RoPE variants).
    """
    q = np.asarray(q, dtype=np.float64)
    M, Hq, D = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if not softmax_scale else float(softmax_scale)
    heads = list(range(Hq)) if heads is None else list(heads)
    inv_freq = rope_inv_freq(D, rope_theta) if inv_freq is None else np.asarray(inv_freq, dtype=np.float64)
    if pe == "alibi" and slopes is None:
        slopes = alibi_slopes(Hq)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    visible = k_pos[None, :] <= q_pos[:, None]                    # [M][L], causal incl. self

    if pe == "rope" and formulation == "materialized":
        Kr = rope_rotate(K, k_pos[:, None], inv_freq)             # every key at its position
        Qr = rope_rotate(q, q_pos[:, None], inv_freq)             # every query at its position
    else:
        Kr, Qr = K, q

    out = np.zeros((M, len(heads), D), dtype=np.float64)
    weights = np.zeros((M, len(heads), K.shape[0]), dtype=np.float64) if return_weights else None
    for j, h in enumerate(heads):
        kvh = h // G
        if pe == "rope" and formulation == "deferred":
            z = np.empty((M, K.shape[0]), dtype=np.float64)
            for m in range(M):
                # keys rotated by the relative offset t - p only; query untouched
                krel = rope_rotate(K[:, kvh, :], k_pos - q_pos[m], inv_freq)
                z[m] = scale * (krel @ q[m, h, :])
        else:
            z = scale * (Qr[:, h, :] @ Kr[:, kvh, :].T)               # [M][L]
            if pe == "alibi":
                z = z - slopes[h] * (q_pos[:, None] - k_pos[None, :]).astype(np.float64)
            elif pe not in ("rope", "none"):
                raise ValueError(pe)
        z = np.where(visible, z, -np.inf)
        zmax = z.max(axis=1, keepdims=True)
        e = np.where(visible, np.exp(z - zmax), 0.0)
        a = e / e.sum(axis=1, keepdims=True)
        out[:, j, :] = a @ V[:, kvh, :]
        if return_weights:
            weights[:, j, :] = a
    return (out, weights) if return_weights else out


# ---------------------------------------------------------------------------
# 6. the library's two calls, batch level
# ---------------------------------------------------------------------------
def _request_args(table_words, num_entries, ctx_lens, r):
    return table_words[r], int(num_entries[r]), int(ctx_lens[r])


def prefill(*, q, cu_q_lens, ctx_lens, num_entries, table_words, k_pool, v_pool,
            num_kv_heads: int, block_size: int, dtype: str, pe: str, rope_theta: float,
            softmax_scale: Optional[float] = None, slopes=None, formulation: str = "materialized",
            requests: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None,
            token_subset: Optional[dict] = None, inv_freq: Optional[np.ndarray] = None,
            pool_dtype: Optional[str] = None) -> dict:
    """Causal prefill of each request's new tokens over its whole context.

    q [total_q][Hq][D]; request r owns rows cu_q_lens[r]..cu_q_lens[r+1]-1,
    its j-th new token sitting at logical position ctx_lens[r] - q_len_r + j
    (the new tokens are the context's last positions).  Returns
    {r: out [q_len_r (or the subset)][len(heads)][D]} in float64.
    ``token_subset`` optionally maps r to the local token indices to compute.
    """
    qf = to_f64(q, dtype)
    reqs = range(len(ctx_lens)) if requests is None else requests
    res = {}
    for r in reqs:
        words, n_ent, L = _request_args(table_words, num_entries, ctx_lens, r)
        K, V, kp = gather_context(words, n_ent, L, k_pool, v_pool, block_size, pool_dtype or dtype)
        a, b = int(cu_q_lens[r]), int(cu_q_lens[r + 1])
        M = b - a
        local = np.arange(M) if token_subset is None or r not in token_subset \
            else np.asarray(token_subset[r], dtype=np.int64)
        qpos = L - M + local
        res[r] = attend(qf[a + local], qpos, K, V, kp, pe=pe, rope_theta=rope_theta,
                        softmax_scale=softmax_scale, slopes=slopes,
                        formulation=formulation, heads=heads, inv_freq=inv_freq)
    return res


def decode(*, q, ctx_lens, num_entries, table_words, k_pool, v_pool,
           num_kv_heads: int, block_size: int, dtype: str, pe: str, rope_theta: float,
           softmax_scale: Optional[float] = None, slopes=None, formulation: str = "materialized",
           requests: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None,
           inv_freq: Optional[np.ndarray] = None, pool_dtype: Optional[str] = None) -> dict:
    """One decode step: request r's single query q[r] [Hq][D] sits at position ctx_lens[r]-1."""
    qf = to_f64(q, dtype)
    reqs = range(len(ctx_lens)) if requests is None else requests
    res = {}
    for r in reqs:
        words, n_ent, L = _request_args(table_words, num_entries, ctx_lens, r)
        K, V, kp = gather_context(words, n_ent, L, k_pool, v_pool, block_size, pool_dtype or dtype)
        res[r] = attend(qf[r][None], np.array([L - 1]), K, V, kp, pe=pe, rope_theta=rope_theta,
                        softmax_scale=softmax_scale, slopes=slopes,
                        formulation=formulation, heads=heads, inv_freq=inv_freq)[0]
    return res


def append_kv(k_pool, v_pool, k_new, v_new, slots, block_size: int):
    """Write new tokens' unrotated K/V [n][Hkv][D] into pool slots (block * B + row), in place."""
    slots = np.asarray(slots, dtype=np.int64)
    for i, sl in enumerate(slots):
        b, row = int(sl) // block_size, int(sl) % block_size
        kb = k_pool[np.array([b])]
        vb = v_pool[np.array([b])]
        kb[0, :, row, :] = k_new[i]
        vb[0, :, :, row] = v_new[i]
        k_pool[np.array([b])] = kb
        v_pool[np.array([b])] = vb


# ---------------------------------------------------------------------------
# 6b. the document-local-frame pool variant
#     [gist:Technical Implementation / Decoding]: the query is rotated only
#     when the offset changes, i.e. when attention moves on to another
#     document; [gist:Technical Implementation / Prefilling]: one relative
#     rotation per key tile.  Both only save work if the cached keys already
#     carry their positions inside their own document.  Reading: a document
#     block stores R(j) k for the key's index j inside its document (its
#     "frame"); entry e of a request carries the frame start F_e (the
#     document's first logical position there).  Since R(a)^T R(b) = R(b - a)
#     [gist:Mathematical Equivalence], with t = F + j
#         q^T R(t - p) k = (R(p - F) q)^T (R(t - F) k),
#     so the framed scores equal the content-only ones.
# ---------------------------------------------------------------------------
def rotate_into_frames(k_new: np.ndarray, frame_index, inv_freq: np.ndarray) -> np.ndarray:
    """Keys [n][Hkv][D] as a framed pool stores them: token i turned by R(frame_index[i])."""
    return rope_rotate(k_new, np.asarray(frame_index, dtype=np.float64)[:, None], inv_freq)


def append_kv_framed(k_pool, v_pool, k_new, v_new, slots, frame_index, block_size: int, inv_freq,
                     dtype: str):
    """append_kv of the framed keys into float64 pools; k_new, v_new in ``dtype``."""
    append_kv(k_pool, v_pool, rotate_into_frames(to_f64(k_new, dtype), frame_index, inv_freq),
              to_f64(v_new, dtype), slots, block_size)


def token_frames(words, n_entries, ctx_len, frame_starts, block_size, num_blocks) -> np.ndarray:
    """Frame start of each logical token 0..L-1: that of the entry holding it."""
    _, starts, lens = decode_table(words, n_entries, ctx_len, block_size, num_blocks)
    f = np.empty(ctx_len, dtype=np.int64)
    for e in range(starts.size):
        f[int(starts[e]):int(starts[e]) + int(lens[e])] = int(frame_starts[e])
    return f


def attend_framed(q, q_pos, K, V, k_pos, k_frame, *, rope_theta: float, softmax_scale=None, heads=None):
    """Causal attention over framed keys: z_t = scale * <R(p - F_t) q_p, K_t>.

    q [M][Hq][D] unrotated; K [L][Hkv][D] holds R(t - F_t) k_t; V content.
    The query is turned separately for every key's frame (no grouping by
    document: the plain definition).
    """
    q = np.asarray(q, dtype=np.float64)
    M, Hq, D = q.shape
    G = Hq // K.shape[1]
    scale = 1.0 / math.sqrt(D) if not softmax_scale else float(softmax_scale)
    heads = list(range(Hq)) if heads is None else list(heads)
    inv_freq = rope_inv_freq(D, rope_theta)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    k_frame = np.asarray(k_frame, dtype=np.int64)
    out = np.zeros((M, len(heads), D), dtype=np.float64)
    for j, h in enumerate(heads):
        kvh = h // G
        for m in range(M):
            qt = rope_rotate(np.broadcast_to(q[m, h], (K.shape[0], D)), q_pos[m] - k_frame, inv_freq)
            z = scale * np.sum(qt * K[:, kvh, :], axis=1)
            vis = k_pos <= q_pos[m]
            z = np.where(vis, z, -np.inf)
            e = np.where(vis, np.exp(z - z.max()), 0.0)
            out[m, j] = (e / e.sum()) @ V[:, kvh, :]
    return out


def prefill_framed(*, q, cu_q_lens, ctx_lens, num_entries, table_words, frame_starts, k_pool, v_pool,
                   block_size: int, dtype: str, rope_theta: float, softmax_scale=None,
                   requests=None, heads=None, token_subset=None) -> dict:
    """prefill over a framed pool (k_pool, v_pool float64; q in ``dtype``); results as prefill's."""
    qf = to_f64(q, dtype)
    reqs = range(len(ctx_lens)) if requests is None else requests
    res = {}
    for r in reqs:
        words, n_ent, L = _request_args(table_words, num_entries, ctx_lens, r)
        K, V, kp = gather_context(words, n_ent, L, k_pool, v_pool, block_size, "f64")
        fr = token_frames(words, n_ent, L, frame_starts[r], block_size, k_pool.shape[0])
        a, b = int(cu_q_lens[r]), int(cu_q_lens[r + 1])
        M = b - a
        local = np.arange(M) if token_subset is None or r not in token_subset \
            else np.asarray(token_subset[r], dtype=np.int64)
        res[r] = attend_framed(qf[a + local], L - M + local, K, V, kp, fr, rope_theta=rope_theta,
                               softmax_scale=softmax_scale, heads=heads)
    return res


def decode_framed(*, q, ctx_lens, num_entries, table_words, frame_starts, k_pool, v_pool,
                  block_size: int, dtype: str, rope_theta: float, softmax_scale=None,
                  requests=None, heads=None) -> dict:
    """One decode step over a framed pool (float64 pools); results as decode's."""
    qf = to_f64(q, dtype)
    reqs = range(len(ctx_lens)) if requests is None else requests
    res = {}
    for r in reqs:
        words, n_ent, L = _request_args(table_words, num_entries, ctx_lens, r)
        K, V, kp = gather_context(words, n_ent, L, k_pool, v_pool, block_size, "f64")
        fr = token_frames(words, n_ent, L, frame_starts[r], block_size, k_pool.shape[0])
        res[r] = attend_framed(qf[r][None], np.array([L - 1]), K, V, kp, fr, rope_theta=rope_theta,
                               softmax_scale=softmax_scale, heads=heads)[0]
    return res

# ---------------------------------------------------------------------------
def brute_force_attention(q_rows, q_positions, words, n_entries, ctx_len, k_pool, v_pool,
                          block_size, num_q_heads, num_kv_heads, theta, pe="rope", scale=None):
    """out[m][h][:] for nested-list queries, written with Python loops only."""
    D = len(q_rows[0][0])
    G = num_q_heads // num_kv_heads
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    # table walk
    slot_of = {}
    ents = []
    for e in range(n_entries):
        w = int(words[e])
        ents.append((w & 0xFFFFFFFF, w >> 32))
    for e, (b, s) in enumerate(ents):
        nxt = ents[e + 1][1] if e + 1 < len(ents) else ctx_len
        for r in range(nxt - s):
            slot_of[s + r] = (b, r)

    def rot(vec, n):
        outv = list(vec)
        for i in range(D // 2):
            ang = n * theta ** (-2.0 * i / D)
            c, s = math.cos(ang), math.sin(ang)
            x0, x1 = vec[2 * i], vec[2 * i + 1]
            outv[2 * i] = x0 * c - x1 * s
            outv[2 * i + 1] = x0 * s + x1 * c
        return outv

    out = []
    for m, p in enumerate(q_positions):
        rows = []
        for h in range(num_q_heads):
            g = h // G
            qv = [float(x) for x in q_rows[m][h]]
            if pe == "rope":
                qv = rot(qv, p)
            zs, vs = [], []
            for t in range(p + 1):
                b, r = slot_of[t]
                kv = [float(k_pool[b][g][r][d]) for d in range(D)]
                if pe == "rope":
                    kv = rot(kv, t)
                z = scale * sum(qv[d] * kv[d] for d in range(D))
                if pe == "alibi":
                    z -= 2.0 ** (-8.0 * (h + 1) / num_q_heads) * (p - t)
                zs.append(z)
                vs.append([float(v_pool[b][g][d][r]) for d in range(D)])
            mx = max(zs)
            ex = [math.exp(z - mx) for z in zs]
            tot = sum(ex)
            rows.append([sum(ex[t] * vs[t][d] for t in range(len(zs))) / tot for d in range(D)])
        out.append(rows)
    return out


# ---------------------------------------------------------------------------
# 8. prefill rotation cost model  ([gist:Technical Implementation / Prefilling])
# ---------------------------------------------------------------------------
def tile_flop_counts(M: int, N: int, D: int) -> dict:
    """Operation counts of one (query tile M x key tile N) step with head dim D.

    QK^T and PV each cost M*N*D multiplies and as many adds; rotating the N
    keys of the tile once costs, per channel of each pair, two multiplies and
    one add.  Counted element by element over the tile.
    """
    qk = pv = 0
    for _ in range(M):
        qk += N * D * 2
        pv += N * D * 2
    rot = 0
    for _ in range(N):
        for _ in range(D // 2):
            rot += 2 * 3
    return {"qk": qk, "pv": pv, "rotation": rot}


def rotation_flop_fraction(M: int, N: int = 64, D: int = 128) -> float:
    """Rotation FLOPs as a fraction of the tile's matmul FLOPs."""
    c = tile_flop_counts(M, N, D)
    return c["rotation"] / (c["qk"] + c["pv"])


# ---------------------------------------------------------------------------
# 9. which documents a block budget keeps: three cache keys under LRU
#    [gist:Problem Statement]: a position-aware cache can reuse a document
#    only at the position it was cached at, so it stores several variants of
#    one document; prefix reuse needs an identical prefix; under a limited
#    HBM budget and skewed (Zipf) access this lowers the hit ratio.
#    [gist:Key Contributions], [gist:Experimental Results] report the ratios.
#    Readings (the pages leave the mechanics open): documents are cached
#    whole, ceil(len/16) blocks each; least-recently-used eviction of entries
#    no admitted request is using; a document that cannot get blocks is
#    served uncached ("bypass"); a request's documents become most recently
#    used when it finishes, in context order; under the prefix key a
#    document counts as a hit only if all earlier documents of the request
#    hit.  Blocks are handed out lowest id first and come back on eviction so
#    that they are handed out again in their old order.
# ---------------------------------------------------------------------------
class BlockCache:
    """Plain Python model of a document cache over ``num_blocks`` blocks.

    policy "agnostic": key = document; "aware": key = (document, logical start);
    "prefix": key = the tuple of documents up to and including this one.
    """

    MISS, HIT, BYPASS = 0, 1, 2

    def __init__(self, num_blocks: int, policy: str):
        from collections import OrderedDict
        if policy not in ("agnostic", "aware", "prefix"):
            raise ValueError(policy)
        self.policy = policy
        self.num_blocks = int(num_blocks)
        self.free = list(range(self.num_blocks))      # free[0] is handed out next
        self.entries = {}                             # key -> [blocks, pins]
        self.lru = OrderedDict()                      # unpinned keys, oldest first
        self.open = {}
        self.next_ticket = 1
        self.stats = dict(doc_accesses=0, doc_hits=0, token_accesses=0, token_hits=0, inserts=0,
                          evictions=0, bypasses=0)

    def _key(self, docs, k, start):
        if self.policy == "agnostic":
            return docs[k]
        if self.policy == "aware":
            return (docs[k], start)
        return tuple(docs[:k + 1])

    def admit(self, docs, lens):
        docs = [int(d) for d in docs]
        status, blocks, starts, used = [], [], [], []
        start = 0
        all_hit_so_far = True
        for k, n in enumerate(int(x) for x in lens):
            nb = -(-n // 16)
            key = self._key(docs, k, start)
            self.stats["doc_accesses"] += 1
            self.stats["token_accesses"] += n
            if key in self.entries:
                ent = self.entries[key]
                s = self.HIT if (self.policy != "prefix" or all_hit_so_far) else self.MISS
                if ent[1] == 0:
                    del self.lru[key]
                ent[1] += 1
            else:
                while len(self.free) < nb and self.lru:
                    old, _ = self.lru.popitem(last=False)
                    self.free = self.entries.pop(old)[0] + self.free
                    self.stats["evictions"] += 1
                if len(self.free) >= nb:
                    ent = [self.free[:nb], 1]
                    self.free = self.free[nb:]
                    self.entries[key] = ent
                    self.stats["inserts"] += 1
                    s = self.MISS
                else:
                    ent = None
                    self.stats["bypasses"] += 1
                    s = self.BYPASS
            if s == self.HIT:
                self.stats["doc_hits"] += 1
                self.stats["token_hits"] += n
            else:
                all_hit_so_far = False
            if ent is not None:
                used.append(key)
                for j, b in enumerate(ent[0]):
                    blocks.append(b)
                    starts.append(start + 16 * j)
            status.append(s)
            start += n
        t = self.next_ticket
        self.next_ticket += 1
        self.open[t] = used
        return status, blocks, starts, t

    def release(self, ticket):
        for key in self.open.pop(ticket):
            ent = self.entries[key]
            ent[1] -= 1
            if ent[1] == 0:
                self.lru[key] = None

    def blocks_in_use(self):
        return self.num_blocks - len(self.free)

    def run(self, requests):
        """requests: iterable of (docs, lens); each admitted and released in turn."""
        for docs, lens in requests:
            _, _, _, t = self.admit(docs, lens)
            self.release(t)
        return self.stats


# ---------------------------------------------------------------------------
# 10. an FP8 (e4m3) pool with per-row power-of-two scales
#     Not described by the pages (their pool is bf16); a narrower format for
#     the same content-only cache.  Readings: OCP e4m3 (1 sign, 4 exponent
#     bits with bias 7, 3 mantissa bits; exponent 15 with mantissa 7 is NaN,
#     largest finite 448, subnormals below 2^-6); each 128-value row (one
#     token's K, or its V) gets the smallest exponent e >= -127 with
#     max|x| <= 448 * 2^e (0 for an all-zero row) and codes = nearest e4m3
#     value of x * 2^-e, ties to the even code, saturating at 448.
#     Chunk per (block, KV head): K codes [16 rows][128], then 16 int8
#     exponents (rows); V codes [128][16 tokens], then 16 int8 exponents.
# ---------------------------------------------------------------------------
FP8_CHUNK = 16 * 128 + 16


def e4m3_value(code: int) -> float:
    """The value of one e4m3 code, from the format's definition."""
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_MAGNITUDES = np.array([e4m3_value(c) for c in range(127)])       # codes 0..126, increasing


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Nearest e4m3 code of each value (ties to the even code, saturating at 448; the sign of
    zero kept), by search over the 127 non-negative finite magnitudes."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    hi = np.clip(np.searchsorted(_E4M3_MAGNITUDES, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = np.abs(a - _E4M3_MAGNITUDES[lo])
    d_hi = np.abs(_E4M3_MAGNITUDES[hi] - a)
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a >= 448.0, 126, pick)
    return (pick | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def fp8_row_exponent(amax: float) -> int:
    """Smallest e >= -127 with amax <= 448 * 2^e (0 when amax is 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    e = max(-127, math.ceil(math.log2(amax / 448.0)))
    while amax > 448.0 * 2.0 ** e:
        e += 1
    while e > -127 and amax <= 448.0 * 2.0 ** (e - 1):
        e -= 1
    return e


def quantize_fp8_rows(x: np.ndarray):
    """Rows x [..., D] (float32 values) -> (codes uint8 [..., D], exponents int8 [...])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    exps = np.vectorize(fp8_row_exponent, otypes=[np.int64])(amax)
    y = np.ldexp(x, -exps[..., None].astype(np.int32))              # float32, exact scaling
    return e4m3_encode(y), exps.astype(np.int8)


def fp8_empty_pools(num_blocks: int, num_kv_heads: int):
    """Chunked K and V pools, every byte 0xFF (NaN codes) until written."""
    shape = (num_blocks, num_kv_heads, FP8_CHUNK)
    return np.full(shape, 0xFF, dtype=np.uint8), np.full(shape, 0xFF, dtype=np.uint8)


def append_kv_fp8(k_chunks, v_chunks, k_new, v_new, slots, dtype: str, block_size: int = 16,
                  frame_index=None, inv_freq=None):
    """Quantise new tokens' K/V [n][Hkv][D] (in ``dtype``) row by row into pool slots, in place.
    With ``frame_index`` the keys are first turned into their document-local frames (section 6b),
    exactly, then rounded to float32 and quantised."""
    k = to_f64(k_new, dtype)
    if frame_index is not None:
        k = rotate_into_frames(k, frame_index, inv_freq)
    k = k.astype(np.float32)
    v = to_f64(v_new, dtype).astype(np.float32)
    kc, ke = quantize_fp8_rows(k)
    vc, ve = quantize_fp8_rows(v)
    D = k.shape[-1]
    for i, sl in enumerate(np.asarray(slots, dtype=np.int64)):
        b, row = int(sl) // block_size, int(sl) % block_size
        k_chunks[b, :, row * D:(row + 1) * D] = kc[i]
        k_chunks[b, :, block_size * D + row] = ke[i].view(np.uint8)
        v_chunks[b, :, row:block_size * D:block_size] = vc[i]
        v_chunks[b, :, block_size * D + row] = ve[i].view(np.uint8)


class Fp8PoolView:
    """Dequantised float64 blocks of a chunked pool, in the plain layouts, on indexing:
    kind "k" -> [n][Hkv][16][D], kind "v" -> [n][Hkv][D][16]."""

    _table = np.array([e4m3_value(c) for c in range(256)])

    def __init__(self, chunks: np.ndarray, kind: str, head_dim: int = 128, block_size: int = 16):
        self.chunks, self.kind, self.D, self.B = chunks, kind, head_dim, block_size

    @property
    def shape(self):
        nb, hkv = self.chunks.shape[:2]
        return (nb, hkv, self.B, self.D) if self.kind == "k" else (nb, hkv, self.D, self.B)

    def __getitem__(self, ids):
        c = self.chunks[ids]
        vals = self._table[c[..., :self.B * self.D]]
        scale = np.ldexp(1.0, c[..., self.B * self.D:].view(np.int8).astype(np.int32))   # [n][Hkv][16]
        if self.kind == "k":
            return vals.reshape(c.shape[:2] + (self.B, self.D)) * scale[..., :, None]
        return vals.reshape(c.shape[:2] + (self.D, self.B)) * scale[..., None, :]
