"""Put a workload's host arrays into device memory in the library's layouts.

Pure data movement: pools are allocated NaN-filled (so padding rows and
never-written blocks poison any result that reads them) and the written
blocks are scattered in; table words are packed with the library's own
host codec.  No attention arithmetic happens here.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import _abi


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_device(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Host values (bf16 bit patterns or float32) -> device tensor of the matching dtype."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def config_for(spec, pe: str = None, softmax_scale: float = 0.0, exact_max: bool = False,
               inv_freq: np.ndarray = None, kv_format: str = "plain", keys: str = None) -> _abi.Config:
    """keys: where the RoPE prefill turns the keys ("fused", "once", or None for the library's choice)."""
    return _abi.make_config(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.dtype,
                            pe or spec.pe, spec.rope_theta, softmax_scale, block_size=spec.block_size,
                            exact_max=exact_max, inv_freq=inv_freq, kv_format=kv_format, keys=keys)


class DevicePools:
    """K pool [nb][Hkv][B][D] and V pool [nb][Hkv][D][B] on the device."""

    def __init__(self, wl, device="cuda", block_permutation: np.ndarray = None):
        kp, vp = wl.pools()
        s = wl.spec
        dt = torch_dtype(s.dtype)
        nb = wl.num_blocks
        self.num_blocks = nb
        self.dtype = s.dtype
        self.k = torch.full((nb, s.num_kv_heads, s.block_size, s.head_dim), float("nan"), dtype=dt, device=device)
        self.v = torch.full((nb, s.num_kv_heads, s.head_dim, s.block_size), float("nan"), dtype=dt, device=device)
        ids = kp.ids if block_permutation is None else block_permutation[kp.ids]
        idx = torch.from_numpy(np.asarray(ids, dtype=np.int64)).to(device)
        self.k[idx] = to_device(kp.data, s.dtype, device)
        self.v[idx] = to_device(vp.data, s.dtype, device)


class WrittenPools:
    """K/V pools whose documents are written by the library's own append:
    lazyattn_append_kv (FP8 pools: quantised there), or with ``framed``
    lazyattn_append_kv_framed (keys in document-local frames, R(j) k with j the
    index inside the document).  Never-written slots hold NaN (FP8: code 0xFF)."""

    framed = False

    def __init__(self, wl, cfg, device="cuda"):
        s = wl.spec
        if s.dtype != "bf16":
            raise ValueError("written pools are bf16 only")
        nb = wl.num_blocks
        self.num_blocks = nb
        self.dtype = s.dtype
        self.fp8 = cfg.kv_format == _abi.KV_FORMATS["fp8"]
        if self.fp8:
            shape = (nb, s.num_kv_heads, _abi.FP8_CHUNK_BYTES)
            self.k = torch.full(shape, 0xFF, dtype=torch.uint8, device=device)
            self.v = torch.full(shape, 0xFF, dtype=torch.uint8, device=device)
        else:
            dt = torch_dtype(s.dtype)
            self.k = torch.full((nb, s.num_kv_heads, s.block_size, s.head_dim), float("nan"), dtype=dt, device=device)
            self.v = torch.full((nb, s.num_kv_heads, s.head_dim, s.block_size), float("nan"), dtype=dt, device=device)
        ks, vs, sl, fi = [], [], [], []
        for d in wl.referenced_docs:
            k, v = wl.doc_kv(int(d))
            slots, j = wl.doc_frame_tokens(int(d))
            ks.append(k)
            vs.append(v)
            sl.append(slots)
            fi.append(j)
        if ks:
            chunk = 1 << 16                       # tokens per append call
            k, v = np.concatenate(ks), np.concatenate(vs)
            sl, fi = np.concatenate(sl).astype(np.int64), np.concatenate(fi).astype(np.int32)
            for a in range(0, sl.size, chunk):
                b = min(sl.size, a + chunk)
                kd, vd = to_device(k[a:b], s.dtype, device), to_device(v[a:b], s.dtype, device)
                sd = torch.from_numpy(sl[a:b]).to(device)
                if self.framed:
                    _abi.append_kv_framed(cfg, self.k, self.v, nb, kd, vd, sd, torch.from_numpy(fi[a:b]).to(device))
                else:
                    _abi.append_kv(cfg, self.k, self.v, nb, kd, vd, sd)


class FramedPools(WrittenPools):
    """Pools in document-local frames (see WrittenPools)."""

    framed = True


class DeviceTables:
    """Packed block tables plus per-request counts (and frame starts) for one call."""

    def __init__(self, table_blocks: np.ndarray, table_starts: np.ndarray, num_entries: np.ndarray,
                 ctx_lens: np.ndarray, device="cuda", block_permutation: np.ndarray = None,
                 frame_starts: np.ndarray = None, req_order: np.ndarray = None):
        blocks = table_blocks if block_permutation is None else \
            block_permutation[table_blocks.astype(np.int64)].astype(np.uint32)
        self.words_host = _abi.pack_entries(blocks, table_starts)
        self.tables = torch.from_numpy(self.words_host.view(np.int64)).to(device)
        self.num_entries = torch.from_numpy(np.ascontiguousarray(num_entries, dtype=np.int32)).to(device)
        self.ctx_lens = torch.from_numpy(np.ascontiguousarray(ctx_lens, dtype=np.int32)).to(device)
        self.frame_starts = None if frame_starts is None else \
            torch.from_numpy(np.ascontiguousarray(frame_starts, dtype=np.int32)).to(device)
        self.req_order = None if req_order is None else \
            torch.from_numpy(np.ascontiguousarray(req_order, dtype=np.int32)).to(device)
        self.batch = _abi.make_batch(self.tables, self.num_entries, self.ctx_lens, self.frame_starts,
                                     self.req_order)

    @classmethod
    def from_inputs(cls, inputs: dict, device="cuda", block_permutation=None, framed=False, req_order=None):
        return cls(inputs["table_blocks"], inputs["table_starts"], inputs["num_entries"], inputs["ctx_lens"],
                   device, block_permutation, inputs["frame_starts"] if framed else None, req_order)


def longest_first(num_entries: np.ndarray) -> np.ndarray:
    """Request order with the longest tables first (ties in batch order): prefill work-groups
    taking the requests in this order leave the short ones to fill the end of the launch."""
    return np.argsort(-np.asarray(num_entries, dtype=np.int64), kind="stable").astype(np.int32)


def append_tokens(cfg, pools: DevicePools, inputs: dict, dtype: str, device="cuda", block_permutation=None):
    """Write a batch of new tokens' K/V (inputs k_new, v_new, slots) into the pools."""
    if inputs is None:
        return
    slots = inputs["slots"]
    if block_permutation is not None:
        slots = block_permutation[slots // 16] * 16 + slots % 16
    k = to_device(inputs["k_new"], dtype, device)
    v = to_device(inputs["v_new"], dtype, device)
    sl = torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int64)).to(device)
    if getattr(pools, "framed", False):
        fi = torch.from_numpy(np.ascontiguousarray(inputs["frame_index"], dtype=np.int32)).to(device)
        _abi.append_kv_framed(cfg, pools.k, pools.v, pools.num_blocks, k, v, sl, fi)
    else:
        _abi.append_kv(cfg, pools.k, pools.v, pools.num_blocks, k, v, sl)


class PrefillCall:
    """Device inputs and output/workspace buffers of one prefill call."""

    def __init__(self, cfg, spec, inputs: dict, device="cuda", num_splits: Optional[int] = None,
                 block_permutation=None, framed: bool = False, req_order="longest_first"):
        """req_order: the order in which the work-groups take the requests: "longest_first"
        (longest table first), None (batch order) or an int32 array; the results are the same.
        num_splits: None = the library's own heuristic when the requests are taken longest first
        (the short requests then fill the end of the launch: splitting the long ones for balance
        no longer pays), else chosen from the batch's table lengths (known on the host) with
        lazyattn_prefill_splits_balanced; 0 = the library's own heuristic; > 0 = that many."""
        self.cfg = cfg
        order = longest_first(inputs["num_entries"]) if isinstance(req_order, str) else req_order
        if isinstance(req_order, str) and req_order != "longest_first":
            raise ValueError(f"unknown request order {req_order!r}")
        self.tables = DeviceTables.from_inputs(inputs, device, block_permutation, framed, order)
        self.q = to_device(inputs["q"], spec.dtype, device)
        self.cu_q = torch.from_numpy(inputs["cu_q_lens"].astype(np.int32)).to(device)
        self.total_q = int(inputs["total_q"])
        self.max_q_len = int(inputs["max_q_len"])
        self.out = torch.empty_like(self.q)
        R = len(inputs["ctx_lens"])
        if num_splits is None and isinstance(req_order, str):
            num_splits = 0
        if num_splits is None:
            ne = np.asarray(inputs["num_entries"], dtype=np.int64)
            num_splits = _abi.prefill_splits_balanced(cfg, R, self.max_q_len, int(ne.max(initial=0)),
                                                      int(ne.sum()))
        self.num_splits = num_splits
        self.splits = num_splits if num_splits > 0 else \
            _abi.prefill_splits(cfg, R, self.max_q_len, self.tables.batch.max_entries)
        ws = _abi.prefill_workspace_size(cfg, R, self.total_q, self.max_q_len, self.tables.batch.max_entries,
                                         num_splits)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device) if ws > 0 else None

    def run(self, pools: DevicePools, stream=None):
        _abi.prefill(self.cfg, self.q, self.cu_q, self.total_q, self.max_q_len, pools.k, pools.v, pools.num_blocks,
                     self.tables.batch, self.out, self.workspace, self.num_splits, stream)
        return self.out

    def attend(self, pools: DevicePools, stream=None):
        _abi.prefill_attend(self.cfg, self.q, self.cu_q, self.total_q, self.max_q_len, pools.k, pools.v,
                            pools.num_blocks, self.tables.batch, self.out, self.workspace, self.num_splits, stream)

    def merge(self, stream=None):
        _abi.merge_splits(self.cfg, self.total_q, self.splits, self.workspace, self.out, stream)


class RunDecodeCall:
    """One decode step over shared runs (lazyattn_decode_runs): the plan is cut from the batch's
    tables on the host and copied to the device with the queries; num_blocks is the pool's."""

    def __init__(self, cfg, spec, inputs: dict, num_blocks: int, device="cuda", block_permutation=None):
        self.cfg = cfg
        blocks = inputs["table_blocks"] if block_permutation is None else \
            block_permutation[inputs["table_blocks"].astype(np.int64)].astype(np.uint32)
        words = _abi.pack_entries(blocks, inputs["table_starts"])
        self.plan_host = _abi.decode_runs_plan(cfg, words, inputs["num_entries"], inputs["ctx_lens"], num_blocks)
        h = self.plan_host
        dev = {k: torch.from_numpy(np.ascontiguousarray(v).view(np.int64) if v.dtype == np.uint64 else
                                   np.ascontiguousarray(v)).to(device) for k, v in h.items()}
        self.plan = _abi.make_run_plan(dev["items"], dev["words"], dev["refs"], dev["req_ref_begin"],
                                       dev["req_refs"])
        self.q = to_device(inputs["q"], spec.dtype, device)
        self.out = torch.empty_like(self.q)
        self.num_reqs = len(inputs["ctx_lens"])
        ws = _abi.decode_runs_workspace_size(cfg, h["refs"].shape[0])
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device) if ws > 0 else None

    def run(self, pools: DevicePools, stream=None):
        _abi.decode_runs(self.cfg, self.q, pools.k, pools.v, pools.num_blocks, self.num_reqs, self.plan, self.out,
                         self.workspace, stream)
        return self.out


class DecodeCall:
    """Device inputs and output/workspace buffers of one decode step."""

    def __init__(self, cfg, spec, inputs: dict, device="cuda", num_splits: int = 0, block_permutation=None,
                 framed: bool = False, req_order="longest_first"):
        """req_order: the order in which the work-groups take the requests, as for PrefillCall."""
        self.cfg = cfg
        order = longest_first(inputs["num_entries"]) if isinstance(req_order, str) else req_order
        if isinstance(req_order, str) and req_order != "longest_first":
            raise ValueError(f"unknown request order {req_order!r}")
        self.tables = DeviceTables.from_inputs(inputs, device, block_permutation, framed, order)
        self.q = to_device(inputs["q"], spec.dtype, device)
        self.out = torch.empty_like(self.q)
        self.num_splits = num_splits
        R = self.q.shape[0]
        self.splits = num_splits if num_splits > 0 else _abi.decode_splits(cfg, R, self.tables.batch.max_entries)
        ws = _abi.decode_workspace_size(cfg, R, self.tables.batch.max_entries, num_splits)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device) if ws > 0 else None

    def run(self, pools: DevicePools, stream=None):
        _abi.decode(self.cfg, self.q, pools.k, pools.v, pools.num_blocks, self.tables.batch, self.out,
                    self.workspace, self.num_splits, stream)
        return self.out

    def attend(self, pools: DevicePools, stream=None):
        _abi.decode_attend(self.cfg, self.q, pools.k, pools.v, pools.num_blocks, self.tables.batch, self.out,
                           self.workspace, self.num_splits, stream)

    def merge(self, stream=None):
        _abi.merge_splits(self.cfg, self.q.shape[0], self.splits, self.workspace, self.out, stream)


class MaterializedPrefill:
    """The materialise-then-attend baseline for one prefill call: private copies
    of every request's blocks (K rotated at absolute positions), queries rotated
    at theirs, and the rotation-free prefill over the copy."""

    def __init__(self, spec, inputs: dict, device="cuda", num_splits: int = 0):
        self.cfg_rope = config_for(spec)
        self.cfg_none = config_for(spec, pe="none")
        n_ent = np.asarray(inputs["num_entries"], dtype=np.int64)
        starts = inputs["table_starts"]
        R, E = inputs["table_blocks"].shape
        dst_blocks = np.zeros((R, E), dtype=np.uint32)
        off = 0
        for r in range(R):
            dst_blocks[r, :n_ent[r]] = np.arange(off, off + n_ent[r], dtype=np.uint32)
            off += int(n_ent[r])
        self.dst_num_blocks = max(off, 1)
        dt = torch_dtype(spec.dtype)
        self.k = torch.empty((self.dst_num_blocks, spec.num_kv_heads, spec.block_size, spec.head_dim), dtype=dt,
                             device=device)
        self.v = torch.empty((self.dst_num_blocks, spec.num_kv_heads, spec.head_dim, spec.block_size), dtype=dt,
                             device=device)
        self.src = DeviceTables.from_inputs(inputs, device)
        self.dst = DeviceTables(dst_blocks, starts, inputs["num_entries"], inputs["ctx_lens"], device)
        self.call = PrefillCall(self.cfg_none, spec, inputs, device, num_splits)
        self.call.tables = self.dst
        self.q_rot = torch.empty_like(self.call.q)
        self.bytes_copied = 2 * self.k.numel() * self.k.element_size()

    def materialize(self, pools: DevicePools, stream=None):
        _abi.materialize_kv(self.cfg_rope, pools.k, pools.v, pools.num_blocks, self.src.batch, self.dst.tables,
                            self.k, self.v, self.dst_num_blocks, stream)

    def rotate_queries(self, stream=None):
        c = self.call
        _abi.rotate_queries(self.cfg_rope, c.q, c.cu_q, c.total_q, c.max_q_len, self.src.batch, self.q_rot, stream)

    def attend(self, stream=None):
        c = self.call
        _abi.prefill(self.cfg_none, self.q_rot, c.cu_q, c.total_q, c.max_q_len, self.k, self.v, self.dst_num_blocks,
                     self.dst.batch, c.out, c.workspace, c.num_splits, stream)
        return c.out

    def run(self, pools: DevicePools, stream=None):
        self.materialize(pools, stream)
        self.rotate_queries(stream)
        return self.attend(stream)
