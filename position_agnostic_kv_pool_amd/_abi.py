"""ctypes binding of liblazyattn.so (argument marshalling only).

Every computation happens in the library's HIP kernels; this module turns
torch tensors into device pointers and the current HIP stream, and numpy
arrays into host pointers.  If the built library is missing the import of
any GPU entry point raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# LAZYATTN_LIBRARY names another build of the same library to load (the tests'
# host-sanitizer build); by default the in-tree build
LIB_PATH = os.environ.get("LAZYATTN_LIBRARY") or os.path.join(_PKG, "liblazyattn.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, 1, 2, 3, 4
FLAG_EXACT_MAX = 1          # LAZYATTN_FLAG_EXACT_MAX
FLAG_KEYS_FUSED = 2         # LAZYATTN_FLAG_KEYS_FUSED: the prefill turns keys inside the attention kernel
FLAG_KEYS_ONCE = 4          # LAZYATTN_FLAG_KEYS_ONCE: the prefill turns each key once first
KEYS_ONCE_TILES = 8         # LAZYATTN_KEYS_ONCE_TILES
_KEYS = {None: 0, "auto": 0, "fused": FLAG_KEYS_FUSED, "once": FLAG_KEYS_ONCE}
F32, BF16 = 0, 1
PE_ROPE, PE_NONE, PE_ALIBI = 0, 1, 2
_PE = {"rope": PE_ROPE, "none": PE_NONE, "alibi": PE_ALIBI}
_DT = {"f32": F32, "bf16": BF16}


class LazyAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


KV_FORMATS = {"plain": 0, "fp8": 1}
FP8_CHUNK_BYTES = 2064


class Config(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("pe", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("softmax_scale", ctypes.c_float),
        ("flags", ctypes.c_int32),
        ("alibi_slopes", ctypes.c_void_p),
        ("rope_inv_freq", ctypes.c_void_p),
        ("kv_format", ctypes.c_int32),
    ]


class PoolStats(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in (
        "num_blocks", "blocks_in_use", "doc_accesses", "doc_hits", "token_accesses", "token_hits",
        "inserts", "evictions", "bypasses", "open_requests")]

    def as_dict(self) -> dict:
        return {name: int(getattr(self, name)) for name, _ in self._fields_}


class Batch(ctypes.Structure):
    _fields_ = [
        ("num_reqs", ctypes.c_int32),
        ("max_entries", ctypes.c_int32),
        ("block_tables", ctypes.c_void_p),
        ("num_entries", ctypes.c_void_p),
        ("ctx_lens", ctypes.c_void_p),
        ("frame_starts", ctypes.c_void_p),
        ("req_order", ctypes.c_void_p),
    ]


RUN_ITEM_INTS = 4


class RunPlan(ctypes.Structure):
    """lazyattn_run_plan: the device arrays of a shared-run decode plan."""
    _fields_ = [
        ("num_items", ctypes.c_int32),
        ("num_words", ctypes.c_int32),
        ("num_refs", ctypes.c_int32),
        ("items", ctypes.c_void_p),
        ("words", ctypes.c_void_p),
        ("refs", ctypes.c_void_p),
        ("req_ref_begin", ctypes.c_void_p),
        ("req_refs", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m position_agnostic_kv_pool_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, U32, U64, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                      ctypes.c_uint64, ctypes.c_size_t)
        CP, BP = ctypes.POINTER(Config), ctypes.POINTER(Batch)
        sig = {
            "lazyattn_abi_version": (I32, []),
            "lazyattn_status_string": (ctypes.c_char_p, [I32]),
            "lazyattn_pack": (U64, [U32, U32]),
            "lazyattn_entry_block": (U32, [U64]),
            "lazyattn_entry_start": (U32, [U64]),
            "lazyattn_pack_entries": (I32, [P, P, I64, P]),
            "lazyattn_validate_tables": (I32, [CP, P, I32, I32, P, P, I64, P, P]),
            "lazyattn_prefill_splits": (I32, [CP, I32, I32, I32]),
            "lazyattn_prefill_splits_balanced": (I32, [CP, I32, I32, I32, I64]),
            "lazyattn_decode_splits": (I32, [CP, I32, I32]),
            "lazyattn_prefill_workspace_size": (SZ, [CP, I32, I32, I32, I32, I32]),
            "lazyattn_decode_workspace_size": (SZ, [CP, I32, I32, I32]),
            "lazyattn_prefill": (I32, [CP, P, P, I32, I32, P, P, I64, BP, I32, P, P, SZ, P]),
            "lazyattn_decode": (I32, [CP, P, P, P, I64, BP, I32, P, P, SZ, P]),
            "lazyattn_decode_noalloc": (I32, [CP, P, P, P, I64, BP, I32, P, P]),
            "lazyattn_decode_runs_plan": (I32, [CP, P, I32, I32, P, P, I64, I32, I32, I32, P, P, P, P, P,
                                                ctypes.POINTER(I32), ctypes.POINTER(I32), ctypes.POINTER(I32)]),
            "lazyattn_decode_runs_workspace_size": (SZ, [CP, I32]),
            "lazyattn_decode_runs": (I32, [CP, P, P, P, I64, I32, ctypes.POINTER(RunPlan), P, P, SZ, P]),
            "lazyattn_prefill_attend": (I32, [CP, P, P, I32, I32, P, P, I64, BP, I32, P, P, SZ, P]),
            "lazyattn_decode_attend": (I32, [CP, P, P, P, I64, BP, I32, P, P, SZ, P]),
            "lazyattn_merge_splits": (I32, [CP, I32, I32, P, SZ, P, P]),
            "lazyattn_append_kv": (I32, [CP, P, P, I64, P, P, P, I32, P]),
            "lazyattn_append_kv_framed": (I32, [CP, P, P, I64, P, P, P, P, I32, P]),
            "lazyattn_debug_decode_tables": (I32, [BP, P, P]),
            "lazyattn_materialize_kv": (I32, [CP, P, P, I64, BP, P, P, P, I64, P]),
            "lazyattn_rotate_queries": (I32, [CP, P, P, I32, I32, BP, P, P]),
            "lazyattn_rope_inv_freq": (I32, [I32, I32, ctypes.c_double, P]),
            "lazyattn_pool_create": (I32, [I64, I32, ctypes.POINTER(P)]),
            "lazyattn_pool_destroy": (None, [P]),
            "lazyattn_pool_admit": (I32, [P, P, P, I32, P, P, I32, P, P, P]),
            "lazyattn_pool_release": (I32, [P, I64]),
            "lazyattn_pool_get_stats": (I32, [P, ctypes.POINTER(PoolStats)]),
            "lazyattn_pool_run_trace": (I32, [P, P, P, P, I64]),
            "lazyattn_rope_inv_freq_llama31": (I32, [I32, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                                     ctypes.c_double, I32, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().lazyattn_status_string(int(s)).decode()


def _check(status: int, where: str):
    if status != OK:
        raise LazyAttnError(status, where)


# ---------------------------------------------------------------------------
# host helpers
# ---------------------------------------------------------------------------
def make_config(num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: str = "bf16", pe: str = "rope",
                rope_theta: float = 10000.0, softmax_scale: float = 0.0, alibi_slopes=None,
                block_size: int = 16, exact_max: bool = False, inv_freq: np.ndarray = None,
                kv_format: str = "plain", keys: str = None) -> Config:
    """inv_freq: optional host float64 [head_dim/2] RoPE frequency table (kept alive by the config);
    kv_format "plain" or "fp8" (e4m3 chunks of FP8_CHUNK_BYTES per block and KV head);
    keys: where the RoPE prefill turns the keys, "fused" (in the attention kernel), "once" (one
    pass over each request's keys first) or None / "auto" (the library's choice)."""
    c = Config()
    c.num_q_heads, c.num_kv_heads, c.head_dim, c.block_size = num_q_heads, num_kv_heads, head_dim, block_size
    c.dtype = _DT[dtype] if isinstance(dtype, str) else int(dtype)
    c.pe = _PE[pe] if isinstance(pe, str) else int(pe)
    c.rope_theta = float(rope_theta)
    c.softmax_scale = float(softmax_scale)
    c.flags = (FLAG_EXACT_MAX if exact_max else 0) | _KEYS[keys]
    c.alibi_slopes = _ptr(alibi_slopes) if alibi_slopes is not None else None
    f = None
    if inv_freq is not None:
        f = np.ascontiguousarray(inv_freq, dtype=np.float64)
        if f.shape != (head_dim // 2,):
            raise ValueError(f"inv_freq must hold head_dim/2 = {head_dim // 2} values")
    c.rope_inv_freq = f.ctypes.data if f is not None else None
    c.kv_format = KV_FORMATS[kv_format]
    c._keep = (alibi_slopes, f)
    return c


def rope_inv_freq(head_dim: int, rotary_dim: int, theta: float) -> np.ndarray:
    """Partial-rotary frequency table from the library (pairs past rotary_dim/2 are 0)."""
    out = np.empty(head_dim // 2, dtype=np.float64)
    _check(lib().lazyattn_rope_inv_freq(int(head_dim), int(rotary_dim), float(theta), out.ctypes.data),
           "rope_inv_freq")
    return out


def rope_inv_freq_llama31(head_dim: int, theta: float, factor: float, low_freq_factor: float,
                          high_freq_factor: float, original_max_position: int) -> np.ndarray:
    """Llama 3.1 rescaled frequency table from the library."""
    out = np.empty(head_dim // 2, dtype=np.float64)
    _check(lib().lazyattn_rope_inv_freq_llama31(int(head_dim), float(theta), float(factor), float(low_freq_factor),
                                                float(high_freq_factor), int(original_max_position),
                                                out.ctypes.data), "rope_inv_freq_llama31")
    return out


def pack_entries(blocks: np.ndarray, starts: np.ndarray) -> np.ndarray:
    """Pack uint32 arrays (any shape) into uint64 words with the library's host codec."""
    b = np.ascontiguousarray(blocks, dtype=np.uint32)
    s = np.ascontiguousarray(starts, dtype=np.uint32)
    if b.shape != s.shape:
        raise ValueError("blocks and starts differ in shape")
    out = np.empty(b.shape, dtype=np.uint64)
    _check(lib().lazyattn_pack_entries(b.ctypes.data, s.ctypes.data, b.size, out.ctypes.data), "pack_entries")
    return out


def validate_tables(cfg: Config, tables: np.ndarray, num_entries: np.ndarray, ctx_lens: np.ndarray,
                    num_blocks: int):
    """(status, bad_req, bad_entry) for host copies of a batch's tables."""
    t = np.ascontiguousarray(tables, dtype=np.uint64)
    ne = np.ascontiguousarray(num_entries, dtype=np.int32)
    cl = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    br, be = ctypes.c_int32(0), ctypes.c_int32(0)
    st = lib().lazyattn_validate_tables(ctypes.byref(cfg), t.ctypes.data, t.shape[0], t.shape[1] if t.ndim == 2 else 0,
                                        ne.ctypes.data, cl.ctypes.data, int(num_blocks), ctypes.byref(br),
                                        ctypes.byref(be))
    return st, br.value, be.value


def prefill_splits(cfg: Config, num_reqs: int, max_q_len: int, max_entries: int) -> int:
    return lib().lazyattn_prefill_splits(ctypes.byref(cfg), num_reqs, max_q_len, max_entries)


def prefill_splits_balanced(cfg: Config, num_reqs: int, max_q_len: int, max_entries: int, total_entries: int) -> int:
    return lib().lazyattn_prefill_splits_balanced(ctypes.byref(cfg), num_reqs, max_q_len, max_entries, total_entries)


def decode_splits(cfg: Config, num_reqs: int, max_entries: int) -> int:
    return lib().lazyattn_decode_splits(ctypes.byref(cfg), num_reqs, max_entries)


def prefill_workspace_size(cfg: Config, num_reqs: int, total_q: int, max_q_len: int, max_entries: int,
                           num_splits: int = 0) -> int:
    return lib().lazyattn_prefill_workspace_size(ctypes.byref(cfg), num_reqs, total_q, max_q_len, max_entries,
                                                 num_splits)


def decode_workspace_size(cfg: Config, num_reqs: int, max_entries: int, num_splits: int = 0) -> int:
    return lib().lazyattn_decode_workspace_size(ctypes.byref(cfg), num_reqs, max_entries, num_splits)


# ---------------------------------------------------------------------------
# GPU entry points (torch tensors in, device pointers out)
# ---------------------------------------------------------------------------
def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def make_batch(tables, num_entries, ctx_lens, frame_starts=None, req_order=None) -> Batch:
    """Batch over device tensors: tables int64/uint64 [R][E] words, num_entries/ctx_lens int32 [R],
    optional frame_starts int32 [R][E] (keys stored in document-local frames) and req_order
    int32 [R] (the order in which prefill work-groups take the requests)."""
    b = Batch()
    b.num_reqs = int(num_entries.shape[0])
    b.max_entries = int(tables.shape[1]) if tables.dim() == 2 else 0
    b.block_tables = _ptr(tables)
    b.num_entries = _ptr(num_entries)
    b.ctx_lens = _ptr(ctx_lens)
    b.frame_starts = _ptr(frame_starts) if frame_starts is not None else None
    b.req_order = _ptr(req_order) if req_order is not None else None
    b._keep = (tables, num_entries, ctx_lens, frame_starts, req_order)
    return b


def prefill(cfg: Config, q, cu_q_lens, total_q: int, max_q_len: int, k_pool, v_pool, num_blocks: int,
            batch: Batch, out, workspace=None, num_splits: int = 0, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().lazyattn_prefill(ctypes.byref(cfg), _ptr(q), _ptr(cu_q_lens), int(total_q), int(max_q_len),
                                _ptr(k_pool), _ptr(v_pool), int(num_blocks), ctypes.byref(batch), int(num_splits),
                                _ptr(out), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "lazyattn_prefill")


def decode(cfg: Config, q, k_pool, v_pool, num_blocks: int, batch: Batch, out, workspace=None,
           num_splits: int = 0, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().lazyattn_decode(ctypes.byref(cfg), _ptr(q), _ptr(k_pool), _ptr(v_pool), int(num_blocks),
                               ctypes.byref(batch), int(num_splits), _ptr(out), _ptr(workspace), ws_bytes,
                               _stream(stream))
    _check(st, "lazyattn_decode")


def decode_runs_plan(cfg: Config, tables: np.ndarray, num_entries: np.ndarray, ctx_lens: np.ndarray,
                     num_blocks: int) -> dict:
    """Host plan of a shared-run decode (lazyattn_decode_runs_plan) from host copies of the batch:
    numpy arrays items [n][RUN_ITEM_INTS], words, refs [m][2], req_ref_begin [R+1], req_refs [m]."""
    t = np.ascontiguousarray(tables, dtype=np.uint64)
    ne = np.ascontiguousarray(num_entries, dtype=np.int32)
    cl = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    R, E = int(ne.shape[0]), (int(t.shape[1]) if t.ndim == 2 else 0)
    ni, nw, nr = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    L = lib()
    st = L.lazyattn_decode_runs_plan(ctypes.byref(cfg), t.ctypes.data, R, E, ne.ctypes.data, cl.ctypes.data,
                                     int(num_blocks), 0, 0, 0, None, None, None, None, None,
                                     ctypes.byref(ni), ctypes.byref(nw), ctypes.byref(nr))
    if st != EWORKSPACE and st != OK:
        _check(st, "lazyattn_decode_runs_plan")
    items = np.zeros((max(ni.value, 1), RUN_ITEM_INTS), dtype=np.int32)
    words = np.zeros(max(nw.value, 1), dtype=np.uint64)
    refs = np.zeros((max(nr.value, 1), 2), dtype=np.int32)
    begin = np.zeros(R + 1, dtype=np.int32)
    rrefs = np.zeros(max(nr.value, 1), dtype=np.int32)
    st = L.lazyattn_decode_runs_plan(ctypes.byref(cfg), t.ctypes.data, R, E, ne.ctypes.data, cl.ctypes.data,
                                     int(num_blocks), items.shape[0], words.shape[0], refs.shape[0],
                                     items.ctypes.data, words.ctypes.data, refs.ctypes.data, begin.ctypes.data,
                                     rrefs.ctypes.data, ctypes.byref(ni), ctypes.byref(nw), ctypes.byref(nr))
    _check(st, "lazyattn_decode_runs_plan")
    return dict(items=items[:ni.value], words=words[:nw.value], refs=refs[:nr.value], req_ref_begin=begin,
                req_refs=rrefs[:nr.value])


def decode_runs_workspace_size(cfg: Config, num_refs: int) -> int:
    return lib().lazyattn_decode_runs_workspace_size(ctypes.byref(cfg), int(num_refs))


def make_run_plan(items, words, refs, req_ref_begin, req_refs) -> RunPlan:
    """RunPlan over device int32/uint32 tensors (kept alive by the struct)."""
    p = RunPlan()
    p.num_items = int(items.shape[0])
    p.num_words = int(words.shape[0])
    p.num_refs = int(refs.shape[0])
    p.items, p.words, p.refs = _ptr(items), _ptr(words), _ptr(refs)
    p.req_ref_begin, p.req_refs = _ptr(req_ref_begin), _ptr(req_refs)
    p._keep = (items, words, refs, req_ref_begin, req_refs)
    return p


def decode_runs(cfg: Config, q, k_pool, v_pool, num_blocks: int, num_reqs: int, plan: RunPlan, out, workspace=None,
                stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().lazyattn_decode_runs(ctypes.byref(cfg), _ptr(q), _ptr(k_pool), _ptr(v_pool), int(num_blocks),
                                    int(num_reqs), ctypes.byref(plan), _ptr(out), _ptr(workspace), ws_bytes,
                                    _stream(stream))
    _check(st, "lazyattn_decode_runs")


def decode_noalloc(cfg: Config, q, k_pool, v_pool, num_blocks: int, batch: Batch, out, num_splits: int = 0,
                   stream=None) -> None:
    """lazyattn_decode with the split partials in the library's own device array (no workspace)."""
    st = lib().lazyattn_decode_noalloc(ctypes.byref(cfg), _ptr(q), _ptr(k_pool), _ptr(v_pool), int(num_blocks),
                                       ctypes.byref(batch), int(num_splits), _ptr(out), _stream(stream))
    _check(st, "lazyattn_decode_noalloc")


def prefill_attend(cfg: Config, q, cu_q_lens, total_q: int, max_q_len: int, k_pool, v_pool, num_blocks: int,
                   batch: Batch, out, workspace=None, num_splits: int = 0, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().lazyattn_prefill_attend(ctypes.byref(cfg), _ptr(q), _ptr(cu_q_lens), int(total_q), int(max_q_len),
                                       _ptr(k_pool), _ptr(v_pool), int(num_blocks), ctypes.byref(batch),
                                       int(num_splits), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "lazyattn_prefill_attend")


def decode_attend(cfg: Config, q, k_pool, v_pool, num_blocks: int, batch: Batch, out, workspace=None,
                  num_splits: int = 0, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().lazyattn_decode_attend(ctypes.byref(cfg), _ptr(q), _ptr(k_pool), _ptr(v_pool), int(num_blocks),
                                      ctypes.byref(batch), int(num_splits), _ptr(out), _ptr(workspace), ws_bytes,
                                      _stream(stream))
    _check(st, "lazyattn_decode_attend")


def merge_splits(cfg: Config, num_rows: int, num_splits: int, workspace, out, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().lazyattn_merge_splits(ctypes.byref(cfg), int(num_rows), int(num_splits), _ptr(workspace), ws_bytes,
                                     _ptr(out), _stream(stream))
    _check(st, "lazyattn_merge_splits")


def append_kv(cfg: Config, k_pool, v_pool, num_blocks: int, k_new, v_new, slots, stream=None) -> None:
    st = lib().lazyattn_append_kv(ctypes.byref(cfg), _ptr(k_pool), _ptr(v_pool), int(num_blocks), _ptr(k_new),
                                  _ptr(v_new), _ptr(slots), int(slots.shape[0]), _stream(stream))
    _check(st, "lazyattn_append_kv")


def materialize_kv(cfg: Config, k_pool, v_pool, num_blocks: int, batch: Batch, dst_tables, dst_k_pool, dst_v_pool,
                   dst_num_blocks: int, stream=None) -> None:
    st = lib().lazyattn_materialize_kv(ctypes.byref(cfg), _ptr(k_pool), _ptr(v_pool), int(num_blocks),
                                       ctypes.byref(batch), _ptr(dst_tables), _ptr(dst_k_pool), _ptr(dst_v_pool),
                                       int(dst_num_blocks), _stream(stream))
    _check(st, "lazyattn_materialize_kv")


def rotate_queries(cfg: Config, q, cu_q_lens, total_q: int, max_q_len: int, batch: Batch, q_out,
                   stream=None) -> None:
    st = lib().lazyattn_rotate_queries(ctypes.byref(cfg), _ptr(q), _ptr(cu_q_lens), int(total_q), int(max_q_len),
                                       ctypes.byref(batch), _ptr(q_out), _stream(stream))
    _check(st, "lazyattn_rotate_queries")


def append_kv_framed(cfg: Config, k_pool, v_pool, num_blocks: int, k_new, v_new, slots, frame_index,
                     stream=None) -> None:
    st = lib().lazyattn_append_kv_framed(ctypes.byref(cfg), _ptr(k_pool), _ptr(v_pool), int(num_blocks),
                                         _ptr(k_new), _ptr(v_new), _ptr(slots), _ptr(frame_index),
                                         int(slots.shape[0]), _stream(stream))
    _check(st, "lazyattn_append_kv_framed")


def debug_decode_tables(batch: Batch, out, stream=None) -> None:
    st = lib().lazyattn_debug_decode_tables(ctypes.byref(batch), _ptr(out), _stream(stream))
    _check(st, "lazyattn_debug_decode_tables")


# ---------------------------------------------------------------------------
# block pool manager (host only)
# ---------------------------------------------------------------------------
CACHE_POLICIES = {"agnostic": 0, "aware": 1, "prefix": 2}
DOC_MISS, DOC_HIT, DOC_BYPASS = 0, 1, 2


class Pool:
    """A lazyattn_pool handle: documents -> physical blocks under a block budget (LRU eviction)."""

    def __init__(self, num_blocks: int, policy: str = "agnostic"):
        h = ctypes.c_void_p()
        _check(lib().lazyattn_pool_create(int(num_blocks), CACHE_POLICIES[policy], ctypes.byref(h)), "pool_create")
        self._h = h

    def close(self):
        if self._h:
            lib().lazyattn_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def admit(self, doc_ids, doc_lens):
        """(status uint8 [n], blocks uint32 [E], starts uint32 [E], ticket) for one request."""
        ids = np.ascontiguousarray(doc_ids, dtype=np.int64)
        lens = np.ascontiguousarray(doc_lens, dtype=np.int32)
        cap = int(((lens.astype(np.int64) + 15) // 16).sum())
        blocks = np.empty(max(cap, 1), dtype=np.uint32)
        starts = np.empty(max(cap, 1), dtype=np.uint32)
        status = np.empty(max(ids.size, 1), dtype=np.uint8)
        ne, t = ctypes.c_int32(), ctypes.c_int64()
        _check(lib().lazyattn_pool_admit(self._h, ids.ctypes.data, lens.ctypes.data, int(ids.size), blocks.ctypes.data,
                                         starts.ctypes.data, cap, ctypes.byref(ne), status.ctypes.data,
                                         ctypes.byref(t)), "pool_admit")
        return status[:ids.size], blocks[:ne.value], starts[:ne.value], int(t.value)

    def release(self, ticket: int):
        _check(lib().lazyattn_pool_release(self._h, int(ticket)), "pool_release")

    def stats(self) -> dict:
        st = PoolStats()
        _check(lib().lazyattn_pool_get_stats(self._h, ctypes.byref(st)), "pool_get_stats")
        return st.as_dict()

    def run_trace(self, doc_ids, doc_lens, req_offsets):
        ids = np.ascontiguousarray(doc_ids, dtype=np.int64)
        lens = np.ascontiguousarray(doc_lens, dtype=np.int32)
        off = np.ascontiguousarray(req_offsets, dtype=np.int64)
        _check(lib().lazyattn_pool_run_trace(self._h, ids.ctypes.data, lens.ctypes.data, off.ctypes.data,
                                             int(off.size - 1)), "pool_run_trace")
