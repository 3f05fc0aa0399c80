"""hstu_stack_fwd (all layers of a batch in one call, metadata prepared once)
against the same layers called one by one: identical outputs, bit for bit,
including a batch large enough that the attention fetches work items
dynamically (its work-fetch counter must start from zero in every layer),
candidate rows, and a bad page id in the last layer's table, which must stop
the whole stack before anything is written.  The stack is also checked
against the fp64 oracle (fp32 rel L2 <= 1e-4)."""
import numpy as np
import pytest
import torch

from gpu_util import EPS, stack_from_workload, to_np, tol_check
from oracle import layer as olayer
from workloads import B8_KV_HIT, TINY_FP32, make_workload

pytestmark = pytest.mark.gpu


def inputs(wl, st):
    dev = st.device
    x = torch.from_numpy(wl.x0).to(device=dev, dtype=st.tdtype)
    return x, torch.from_numpy(wl.new_offsets).to(dev), torch.from_numpy(wl.hist_len).to(dev)


def layer_by_layer(st, x, off, hl, L, num_candidates=None):
    outs = []
    for l in range(L):
        y = torch.empty_like(x)
        st.layer(l, x, off, hl, y, num_candidates=num_candidates)
        assert st.read_status() == 0
        outs.append(y)
        x = y
    return outs


def test_stack_equals_layers_with_dynamic_work_fetch():
    print("case stack f32 many users", flush=True)
    wl = make_workload(TINY_FP32, seed=3, B=200, layers=2, hist=("uniform", 0, 50), new=("uniform", 100, 220),
                       pool_pages=4096)
    st = stack_from_workload(wl)
    x, off, hl = inputs(wl, st)
    ys = st.forward(x, off, hl, return_all=True)
    assert st.read_status() == 0
    n_items = int(st._sws[8:12].view(torch.int32).item())
    print(f"  T={wl.T} attention items={n_items}", flush=True)
    assert n_items > torch.cuda.get_device_properties(0).multi_processor_count
    ref = layer_by_layer(st, x, off, hl, 2)
    for l in range(2):
        assert torch.equal(ys[l], ref[l]), f"layer {l} differs"
    layers = [dict(w1=wl.layer(l).w1, w2=wl.layer(l).w2, pos_bias=wl.layer(l).pos_bias,
                   hist_k=wl.layer(l).hist_k, hist_v=wl.layer(l).hist_v) for l in range(2)]
    want = olayer.stack_forward(wl.x0, wl.new_len, wl.hist_len, layers, wl.attn_scale, EPS, wl.H, wl.pos_mbits)
    tol_check(to_np(ys[-1]), want[-1], "f32", "stack f32 many users")


def test_stack_equals_layers_bf16_with_candidates():
    print("case stack bf16 candidates", flush=True)
    wl = make_workload(B8_KV_HIT, seed=4, B=4, hist=("uniform", 256, 1500), new=("uniform", 16, 256), layers=3,
                       pool_pages=4096)
    st = stack_from_workload(wl)
    x, off, hl = inputs(wl, st)
    m = torch.tensor([min(50, int(n)) for n in wl.new_len], dtype=torch.int32, device=st.device)
    ys = st.forward(x, off, hl, return_all=True, num_candidates=m)
    assert st.read_status() == 0
    ref = layer_by_layer(st, x, off, hl, 3, num_candidates=m)
    for l in range(3):
        assert torch.equal(ys[l], ref[l]), f"layer {l} differs"


def test_bad_page_in_last_layer_stops_the_stack():
    print("case stack bad page", flush=True)
    wl = make_workload(TINY_FP32, seed=5, B=3, layers=3, hist=("uniform", 5, 40), new=("uniform", 10, 60),
                       pool_pages=256)
    st = stack_from_workload(wl)
    x, off, hl = inputs(wl, st)
    st.layers[2]["page_table"][1, 0] = wl.num_pool_pages            # a page id outside the pool
    ys = [torch.full_like(x, 3.0) for _ in range(3)]
    from hstu_jagged_silu_fwd_amd import _lib
    desc = st.desc(int(x.shape[0]))
    ws = torch.empty(_lib.stack_workspace_size(desc, 3), dtype=torch.uint8, device=st.device)
    L = st.layers
    _lib.stack_fwd(desc, x, off, hl, [l["page_table"] for l in L], [st.k_pool] * 3, [st.v_pool] * 3,
                   [l["w1t"] for l in L], [l["w2t"] for l in L], [l["pos_bias"] for l in L], ys, ws)
    assert _lib.read_device_status(ws) == 4
    for y in ys:
        assert torch.all(y == 3.0)


@pytest.mark.parametrize("layer,user,which,value", [(1, 77, 2, "pool"), (3, 199, -1, -1), (0, 0, 0, "pool")])
def test_bad_page_anywhere_in_a_long_validation_stops_the_stack(layer, user, which, value):
    """200 users over 4 layers: the page check gives each thread several
    pages per layer, so its loads run across layer boundaries and rounds; a
    bad id in any layer, at any user and page, must be found."""
    print(f"case stack bad page layer {layer} user {user}", flush=True)
    wl = make_workload(TINY_FP32, seed=11, B=200, layers=4, hist=("uniform", 5, 400), new=("uniform", 1, 20),
                       pool_pages=8192)
    st = stack_from_workload(wl)
    x, off, hl = inputs(wl, st)
    npages = int((wl.hist_len[user] + wl.new_len[user] + wl.page_size - 1) // wl.page_size)
    pg = which if which >= 0 else npages - 1                 # a page in use by the user
    st.layers[layer]["page_table"][user, pg] = wl.num_pool_pages if value == "pool" else value
    ys = [torch.full_like(x, 3.0) for _ in range(4)]
    from hstu_jagged_silu_fwd_amd import _lib
    desc = st.desc(int(x.shape[0]))
    ws = torch.empty(_lib.stack_workspace_size(desc, 4), dtype=torch.uint8, device=st.device)
    L = st.layers
    _lib.stack_fwd(desc, x, off, hl, [l["page_table"] for l in L], [st.k_pool] * 4, [st.v_pool] * 4,
                   [l["w1t"] for l in L], [l["w2t"] for l in L], [l["pos_bias"] for l in L], ys, ws)
    assert _lib.read_device_status(ws) == 4
    for y in ys:
        assert torch.all(y == 3.0)


def test_stack_equals_layers_with_timestamps():
    """The serving workload's timestamp bias term through the stack call."""
    print("case stack bf16 timestamps", flush=True)
    from workloads import B64_SERVING
    wl = make_workload(B64_SERVING, seed=6, B=6, hist=("zipf", 1.2, 32, 3000), new=("uniform", 1, 512), layers=2,
                       pool_pages=4096, miss_frac=0.34)
    assert wl.timestamps is not None
    st = stack_from_workload(wl)
    x, off, hl = inputs(wl, st)
    ts = torch.from_numpy(wl.ts_flat()).to(st.device)
    tso = torch.from_numpy(wl.ts_offsets()).to(st.device)
    ys = st.forward(x, off, hl, timestamps=ts, ts_offsets=tso, return_all=True)
    assert st.read_status() == 0
    xin = x
    for l in range(2):
        y = torch.empty_like(x)
        st.layer(l, xin, off, hl, y, timestamps=ts, ts_offsets=tso)
        assert st.read_status() == 0
        assert torch.equal(ys[l], y), f"layer {l} differs"
        xin = y
