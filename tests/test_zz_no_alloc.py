"""hstu_layer_fwd_noalloc -- the entry point for callers that cannot allocate,
whose workspace is the library's static scratch array -- against
hstu_layer_fwd, the entry point it is a variant of, on the same inputs.

Two calls in a row on one GPU, the second with a smaller batch (so it runs
on scratch memory that still holds the first call's contents): each output
must equal hstu_layer_fwd's bit for bit (same kernels, same launch shapes)
and stay within the bf16 / fp32 tolerances of the fp64 oracle; the status
copied to the caller's int must be 0.  A bad page id must reach the
caller's status int and leave y untouched."""
import numpy as np
import pytest
import torch

from gpu_util import oracle_layer, stack_from_workload, to_np, tol_check
from hstu_jagged_silu_fwd_amd import _lib
from workloads import B8_KV_HIT, TINY_FP32, make_workload

pytestmark = pytest.mark.gpu


def _tensors(wl, st):
    dev = st.device
    x = torch.from_numpy(wl.x0).to(device=dev, dtype=st.tdtype)
    off = torch.from_numpy(wl.new_offsets).to(dev)
    hl = torch.from_numpy(wl.hist_len).to(dev)
    ts = tso = None
    if wl.timestamps is not None:
        ts = torch.from_numpy(wl.ts_flat()).to(dev)
        tso = torch.from_numpy(wl.ts_offsets()).to(dev)
    return x, off, hl, ts, tso


def _noalloc(wl, st, x, off, hl, ts, tso, page_table=None):
    L = st.layers[0]
    y = torch.full_like(x, -3.0)
    status = torch.full((1,), -1, dtype=torch.int32, device=st.device)
    _lib.layer_fwd_noalloc(st.desc(int(x.shape[0])), x, off, hl,
                           L["page_table"] if page_table is None else page_table, st.k_pool, st.v_pool,
                           L["w1t"], L["w2t"], L["pos_bias"], y, status, ts_bias=L["ts_bias"],
                           timestamps=ts, ts_offsets=tso)
    torch.cuda.synchronize()
    return y, int(status.cpu()[0])


def _check(wl, what):
    st = stack_from_workload(wl)
    need = _lib.workspace_size(st.desc(wl.T))
    print(f"case {what}: T={wl.T} workspace={need} scratch={_lib.NOALLOC_SCRATCH_BYTES}", flush=True)
    assert need <= _lib.NOALLOC_SCRATCH_BYTES
    x, off, hl, ts, tso = _tensors(wl, st)
    y, code = _noalloc(wl, st, x, off, hl, ts, tso)
    assert code == 0, f"device status {code}"
    y_ref = torch.full_like(x, 7.0)
    st.layer(0, x, off, hl, y_ref, timestamps=ts, ts_offsets=tso)
    assert st.read_status() == 0
    assert torch.equal(y, y_ref), f"{what}: noalloc output differs from hstu_layer_fwd"
    tol_check(to_np(y), oracle_layer(wl, 0)["y"], wl.dtype, what)


def test_noalloc_two_calls_second_smaller():
    big = make_workload(B8_KV_HIT, seed=4, B=8, hist=("uniform", 256, 1500), new=("uniform", 16, 256),
                        layers=1, pool_pages=4096)
    small = make_workload(B8_KV_HIT, seed=5, B=3, hist=("uniform", 40, 700), new=("uniform", 1, 90),
                          layers=1, pool_pages=1024)
    assert small.T < big.T
    _check(big, "noalloc call 1 (8 users)")
    _check(small, "noalloc call 2 (3 users, smaller)")


def test_noalloc_fp32_with_timestamps():
    wl = make_workload(TINY_FP32, seed=3, B=4, hist=("uniform", 5, 90), new=("uniform", 1, 150),
                       pool_pages=64, ts_buckets=64, ts_mbits=2)
    _check(wl, "noalloc fp32 with timestamps")


def test_noalloc_device_error_reaches_caller_status():
    wl = make_workload(B8_KV_HIT, seed=6, B=2, hist=("uniform", 40, 90), new=("uniform", 5, 40), layers=1,
                       pool_pages=256)
    st = stack_from_workload(wl)
    x, off, hl, ts, tso = _tensors(wl, st)
    pt = st.layers[0]["page_table"].clone()
    pt[1, 0] = wl.num_pool_pages + 5                     # a page id outside the pool
    y, code = _noalloc(wl, st, x, off, hl, ts, tso, page_table=pt)
    assert code == 4, f"expected HSTU_DEV_BAD_PAGE, got {code}"
    assert bool((y == -3.0).all()), "y was written despite the device error"
