"""lazyattn_decode_noalloc (split partials in the library's own device array) against
lazyattn_decode with a caller's workspace, through the C interface (MI355X).

Two calls in a row share the array, the second with a smaller input; each must
equal lazyattn_decode's output bit for bit (same kernels, same split count).
"""
import ctypes
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import workloads as W  # noqa: E402
from position_agnostic_kv_pool_amd import _abi, staging  # noqa: E402
from _helpers import OracleState, assert_parity, gpu_f64  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    _abi.lib()


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _noalloc(cfg, call, pools, num_splits):
    out = torch.full_like(call.q, float("nan"))
    st = _abi.lib().lazyattn_decode_noalloc(ctypes.byref(cfg), call.q.data_ptr(), pools.k.data_ptr(),
                                            pools.v.data_ptr(), int(pools.num_blocks), ctypes.byref(call.tables.batch),
                                            int(num_splits), out.data_ptr(),
                                            torch.cuda.current_stream().cuda_stream)
    assert st == 0, _abi.status_string(st)
    return out


def test_noalloc_decode_equals_workspace_decode_on_two_calls():
    say("noalloc decode: 70B shape, 2 requests at the heuristic split count, then 1 request at 7 splits")
    wl = W.build_workload(W.spec(4, requests=[2], n_decode=1))
    s = wl.spec
    cfg = staging.config_for(s)
    pools = staging.DevicePools(wl, DEV)
    staging.append_tokens(cfg, pools, wl.tokens_before_step(0), s.dtype, DEV)
    d = wl.decode_step(0)
    staging.append_tokens(cfg, pools, d, s.dtype, DEV)
    orc = OracleState(wl)
    orc.append(wl.tokens_before_step(0))
    orc.append(d)
    ref = orc.decode(d)

    big = staging.DecodeCall(cfg, s, d, DEV)
    assert big.splits > 1 and big.workspace is not None
    assert big.workspace.numel() <= _abi_scratch_bytes()
    want = gpu_f64(big.run(pools))
    got = gpu_f64(_noalloc(cfg, big, pools, 0))
    assert np.array_equal(got, want)
    assert_parity(got, np.stack([ref[0], ref[1]]), "bf16", "noalloc decode 70B 2 requests")

    # second call: a smaller batch (request 0 alone), fewer splits; the array still
    # holds the first call's partials
    d1 = {k: (v[:1] if isinstance(v, np.ndarray) and v.ndim >= 1 and v.shape[0] == 2 else v) for k, v in d.items()}
    small = staging.DecodeCall(cfg, s, d1, DEV, num_splits=7)
    assert 0 < small.workspace.numel() < big.workspace.numel()
    want1 = gpu_f64(small.run(pools))
    got1 = gpu_f64(_noalloc(cfg, small, pools, 7))
    torch.cuda.synchronize()
    assert np.array_equal(got1, want1)
    assert_parity(got1, ref[0][None], "bf16", "noalloc decode 70B 1 request, 7 splits")


def test_noalloc_decode_rejects_partials_beyond_the_array():
    say("noalloc decode: a call whose partials exceed the array returns EWORKSPACE before any launch")
    wl = W.build_workload(W.spec(5, requests=[0, 96], n_decode=1))
    s = wl.spec
    cfg = staging.config_for(s)
    d = wl.decode_step(0)
    call = staging.DecodeCall(cfg, s, d, DEV)
    need = _abi.decode_workspace_size(cfg, 96, call.tables.batch.max_entries, 256)
    assert need > _abi_scratch_bytes()
    pools_k = torch.zeros(16, dtype=torch.uint8, device=DEV)
    out = torch.zeros_like(call.q)
    st = _abi.lib().lazyattn_decode_noalloc(ctypes.byref(cfg), call.q.data_ptr(), pools_k.data_ptr(),
                                            pools_k.data_ptr(), 1, ctypes.byref(call.tables.batch), 256,
                                            out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 3            # LAZYATTN_EWORKSPACE
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(out.view(torch.int16))) == 0


def _abi_scratch_bytes():
    return 16 << 20           # LAZYATTN_DECODE_SCRATCH_BYTES
