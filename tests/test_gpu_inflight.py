"""Batches in flight: two stack calls over disjoint users, each on a stream
and a workspace of its own, enqueued back to back so that their kernels
overlap, give the same outputs bit for bit as the same calls run one after
the other on the current stream (the library keeps no state outside the
caller's workspace), and each workspace reports its own status; the last
layer also meets the oracle's bf16 tolerance."""
import numpy as np
import pytest
import torch

from gpu_util import oracle_layer, stack_from_workload, to_np, tol_check
from workloads import B8_KV_HIT, make_workload

pytestmark = pytest.mark.gpu


def _batch(wl, st, users):
    off = wl.new_offsets
    x = np.concatenate([wl.x0[off[u]:off[u + 1]] for u in users], axis=0)
    new_off = np.concatenate([[0], np.cumsum(wl.new_len[users])]).astype(np.int32)
    dev = st.device
    return dict(x=torch.from_numpy(x).to(dev, st.tdtype), off=torch.from_numpy(new_off).to(dev),
                hl=torch.from_numpy(wl.hist_len[users].astype(np.int32)).to(dev),
                pts=[st.layers[l]["page_table"][users].contiguous() for l in range(len(st.layers))])


def _call(st, b, **kw):
    return st.forward(b["x"], b["off"], b["hl"], page_tables=b["pts"], return_all=True, **kw)


def test_two_batches_in_flight_equal_serial_calls():
    print("case in-flight bf16 two streams", flush=True)
    wl = make_workload(B8_KV_HIT, seed=21, B=8, hist=("uniform", 256, 1500), new=("uniform", 16, 256), layers=3,
                       pool_pages=4096)
    st = stack_from_workload(wl)
    users = (np.arange(0, 4), np.arange(4, 8))
    bs = [_batch(wl, st, u) for u in users]
    ref = []
    for b in bs:
        ref.append(_call(st, b))
        assert st.read_status() == 0
    torch.cuda.synchronize()
    from hstu_jagged_silu_fwd_amd import _lib
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = []
    for b in bs:
        desc = st.desc(int(b["x"].shape[0]), num_users=len(users[0]))
        wss.append(torch.empty(_lib.stack_workspace_size(desc, 3), dtype=torch.uint8, device=st.device))
    got = []
    for _ in range(3):                       # three rounds, the two calls of a round overlapping
        got.append([_call(st, b, stream=s, workspace=w) for b, s, w in zip(bs, streams, wss)])
    for w in wss:
        assert st.read_status(w) == 0
    torch.cuda.synchronize()
    for r, outs in enumerate(got):
        for i in range(2):
            for l in range(3):
                assert torch.equal(outs[i][l], ref[i][l]), f"round {r} batch {i} layer {l} differs"
    x = wl.x0
    for l in range(3):                       # X_{l+1} = Y_l
        x = oracle_layer(wl, l, x=x)["y"]
    for i in range(2):
        rows = np.concatenate([np.arange(wl.new_offsets[u], wl.new_offsets[u + 1]) for u in users[i]])
        tol_check(to_np(got[-1][i][2]), x[rows], "bf16", f"in-flight batch {i} layer 2")


def test_graphs_replayed_in_flight_equal_serial_calls():
    """Each batch's stack call captured once into a HIP graph on a stream of
    its own, then the two graphs replayed in flight (eager work and
    synchronisations between the rounds): every replay equals the serial
    eager calls bit for bit."""
    print("case in-flight graph replays two streams", flush=True)
    wl = make_workload(B8_KV_HIT, seed=23, B=8, hist=("uniform", 256, 1500), new=("uniform", 16, 256), layers=3,
                       pool_pages=4096)
    st = stack_from_workload(wl)
    users = (np.arange(0, 4), np.arange(4, 8))
    bs = [_batch(wl, st, u) for u in users]
    ref = [_call(st, b)[-1].clone() for b in bs]
    assert st.read_status() == 0
    from hstu_jagged_silu_fwd_amd import _lib
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    graphs, outs, wss = [], [], []
    for b, s in zip(bs, streams):
        desc = st.desc(int(b["x"].shape[0]), num_users=len(users[0]))
        w = torch.empty(_lib.stack_workspace_size(desc, 3), dtype=torch.uint8, device=st.device)
        s.wait_stream(torch.cuda.current_stream())
        _call(st, b, stream=s, workspace=w)          # warm the allocator on the capture stream
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            outs.append(_call(st, b, stream=s, workspace=w)[-1])
        graphs.append(g)
        wss.append(w)
    for rep in range(3):
        junk = torch.randn(1 << 20, device=st.device).sum()   # eager work between the rounds
        torch.cuda.synchronize()
        for o in outs:
            o.fill_(7.0)
        torch.cuda.synchronize()
        for g, s in zip(graphs, streams):
            with torch.cuda.stream(s):
                g.replay()
        torch.cuda.synchronize()
        for w in wss:
            assert _lib.read_device_status(w) == 0
        for i in range(2):
            assert torch.equal(outs[i], ref[i]), f"replay {rep} batch {i} differs"
        del junk


def test_workspace_too_small_is_refused():
    wl = make_workload(B8_KV_HIT, seed=22, B=2, hist=("uniform", 40, 90), new=("uniform", 16, 40), layers=1,
                       pool_pages=256)
    st = stack_from_workload(wl)
    b = _batch(wl, st, np.arange(2))
    with pytest.raises(ValueError):
        _call(st, b, workspace=torch.empty(64, dtype=torch.uint8, device=st.device))
