"""The layer stack captured once into a HIP graph (torch.cuda.CUDAGraph) and
replayed: the library allocates nothing, records no memset and synchronises
nothing inside a call, so a whole stack call can be captured for a serving
loop.  Every replay, with eager work and synchronisations in between, must
equal the eager result bit for bit (the replays append the same K/V to the
same pool slots)."""
import numpy as np
import pytest
import torch

from gpu_util import stack_from_workload
from workloads import B8_KV_HIT, make_workload

pytestmark = pytest.mark.gpu


def test_stack_graph_replays_equal_eager():
    print("case stack graph replay", flush=True)
    wl = make_workload(B8_KV_HIT, seed=7, B=4, hist=("uniform", 256, 1500), new=("uniform", 16, 256), layers=3,
                       pool_pages=4096)
    st = stack_from_workload(wl)
    dev = st.device
    x = torch.from_numpy(wl.x0).to(device=dev, dtype=st.tdtype)
    off = torch.from_numpy(wl.new_offsets).to(dev)
    hl = torch.from_numpy(wl.hist_len).to(dev)
    eager = st.forward(x, off, hl).clone()
    assert st.read_status() == 0
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm the allocator on the capture stream
        st.forward(x, off, hl)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = st.forward(x, off, hl)
    for rep in range(4):
        junk = torch.randn(1 << 20, device=dev).sum()          # eager work between replays
        torch.cuda.synchronize()
        out.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        assert st.read_status() == 0
        assert torch.equal(out, eager), f"replay {rep} differs"
        del junk
