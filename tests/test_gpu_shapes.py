"""Every shape the layer's C ABI accepts, against the fp64 oracle.

hstu_layer_fwd takes fp32 or bf16, head dims 32, 64 and 128 and page sizes
16 to 128 (powers of two); each (dtype, head dim, page size) selects its own
attention instance and step geometry (LDS ring depth, chunk permutation,
loads per wave, pages per 32-key step), and the hidden size and row count
select the norm instance (a wave per row, 32 or 16 threads per row, 2 to 32
column groups).  All 24 combinations run here on one batch whose users
cover the structural cases -- no history, a history shorter than a page,
histories that end mid-page, two q-blocks, a single new row, no new rows --
and hidden sizes chosen so that every norm instance runs; some cases add
the timestamp term or candidate rows.  Tolerances as everywhere: bf16
relative L2 <= 1e-2 and max abs <= 3e-2, fp32 relative L2 <= 1e-4.
"""
import numpy as np
import pytest
import torch

from gpu_util import EPS, stack_from_workload, to_np, tol_check
from oracle import layer as olayer
from workloads import B8_KV_HIT, make_workload

pytestmark = pytest.mark.gpu

# (dtype, head_dim, page_size) -> (heads, extra)
GRID = {
    ("f32", 32, 16): (2, {}),          # D = 64: 16 threads per row
    ("f32", 32, 32): (6, {}),          # D = 192
    ("f32", 32, 64): (4, {}),          # D = 128: 32 threads per row
    ("f32", 32, 128): (8, {}),         # D = 256: a wave per row, one column group
    ("f32", 64, 16): (3, {}),
    ("f32", 64, 32): (4, {}),
    ("f32", 64, 64): (5, {"cand": True}),   # D = 320: 16 threads, 5 groups
    ("f32", 64, 128): (2, {}),
    ("f32", 128, 16): (1, {}),
    ("f32", 128, 32): (3, {}),
    ("f32", 128, 64): (2, {}),
    ("f32", 128, 128): (4, {"ts": True}),   # D = 512: a wave per row
    ("bf16", 32, 16): (4, {}),
    ("bf16", 32, 32): (6, {}),
    ("bf16", 32, 64): (8, {}),
    ("bf16", 32, 128): (2, {"cand": True}),
    ("bf16", 64, 16): (5, {"ts": True}),
    ("bf16", 64, 32): (1, {}),
    ("bf16", 64, 64): (4, {}),
    ("bf16", 64, 128): (6, {}),
    ("bf16", 128, 16): (2, {}),
    ("bf16", 128, 32): (5, {}),        # D = 640: 32 threads, 5 groups
    ("bf16", 128, 64): (3, {}),
    ("bf16", 128, 128): (4, {}),
}

# users: no history; history shorter than a page; history ending mid-page
# with a ragged block of new rows; a long history (several key chunks);
# no new rows; two q-blocks after a one-token history
HIST = [0, 5, 333, 1000, 50, 1]
NEW = [300, 17, 129, 64, 0, 257]


def _workload(dtype, d, ps, H, extra, seed=0, hist=HIST, new=NEW):
    over = dict(dtype=dtype, D=H * d, H=H, d=d, page_size=ps, B=len(hist), layers=extra.get("layers", 1),
                hist=("fixed", list(hist)), new=("fixed", list(new)), pool_pages=4096)
    if extra.get("ts"):
        over.update(ts_buckets=64, ts_mbits=2)
    return make_workload(B8_KV_HIT, seed=seed, **over)


def _inputs(wl, st):
    dev = st.device
    x = torch.from_numpy(wl.x0).to(device=dev, dtype=st.tdtype)
    off = torch.from_numpy(wl.new_offsets).to(dev)
    hl = torch.from_numpy(wl.hist_len).to(dev)
    ts = tso = None
    if wl.timestamps is not None:
        ts = torch.from_numpy(wl.ts_flat()).to(dev)
        tso = torch.from_numpy(wl.ts_offsets()).to(dev)
    return x, off, hl, ts, tso


def _candidates(wl):
    # all rows, none, a run crossing the 16-row groups, one, ..., and a run
    # crossing the q-block boundary
    n = wl.new_len
    m = np.zeros(wl.B, np.int32)
    pick = [n[0], 0, min(40, n[2]), 1, 0, min(200, n[5])]
    m[:len(pick)] = pick[:wl.B]
    return m


def _check_layer(wl, extra, what):
    st = stack_from_workload(wl)
    x, off, hl, ts, tso = _inputs(wl, st)
    y = torch.full_like(x, 7.0)
    m = _candidates(wl) if extra.get("cand") else None
    st.layer(0, x, off, hl, y, timestamps=ts, ts_offsets=tso,
             num_candidates=None if m is None else torch.from_numpy(m).to(st.device))
    code = st.read_status()
    assert code == 0, f"device status {code}"
    li = wl.layer(0)
    ref = olayer.layer_forward(wl.x0, wl.new_len, wl.hist_len, li.hist_k, li.hist_v, li.w1, li.w2,
                               li.pos_bias, wl.pos_mbits, wl.attn_scale, EPS, wl.H, wl.timestamps,
                               li.ts_bias, wl.ts_mbits, num_candidates=m)["y"]
    tol_check(to_np(y), ref, wl.dtype, what)


@pytest.mark.parametrize("dtype,d,ps", list(GRID), ids=[f"{a}-d{b}-ps{c}" for a, b, c in GRID])
def test_layer_shape_grid(dtype, d, ps):
    H, extra = GRID[(dtype, d, ps)]
    print(f"case shape {dtype} d={d} ps={ps} H={H} {extra}", flush=True)
    wl = _workload(dtype, d, ps, H, extra, seed=d + ps)
    _check_layer(wl, extra, f"{dtype} d={d} ps={ps} D={H * d}")


# Norm instances the grid does not reach: 32 threads per row with 10 column
# groups, 16 threads with 15 and 31 groups, and the row counts (>= 4096) at
# which D = 256 and 512 leave the wave-per-row instance.
WIDE = {
    "bf16-D1280-d128": ("bf16", 128, 32, 10, HIST, NEW),
    "bf16-D960-d64": ("bf16", 64, 64, 15, HIST, NEW),
    "f32-D1984-d64": ("f32", 64, 16, 31, [0, 40, 200], [150, 90, 33]),
    "bf16-D512-T4200": ("bf16", 128, 32, 4, [0, 100, 2000], [1800, 1500, 900]),
    "f32-D256-T4200": ("f32", 64, 64, 4, [0, 100, 2000], [1800, 1500, 900]),
}


@pytest.mark.parametrize("case", list(WIDE))
def test_layer_norm_instances(case):
    dtype, d, ps, H, hist, new = WIDE[case]
    print(f"case norm instance {case}", flush=True)
    wl = _workload(dtype, d, ps, H, {}, seed=7, hist=hist, new=new)
    _check_layer(wl, {}, case)


@pytest.mark.parametrize("dtype,d,ps,H", [("f32", 64, 16, 3), ("bf16", 32, 128, 6)])
def test_stack_other_shapes(dtype, d, ps, H):
    # a 3-layer stack call (prep once, every layer's table) at shapes other
    # than the benchmark's, each layer against the oracle's stack
    print(f"case stack {dtype} d={d} ps={ps} H={H}", flush=True)
    wl = _workload(dtype, d, ps, H, {"layers": 3}, seed=5)
    st = stack_from_workload(wl)
    ys = st.forward(wl.x0, wl.new_offsets, wl.hist_len, return_all=True)
    assert st.read_status() == 0
    layers = [dict(w1=wl.layer(l).w1, w2=wl.layer(l).w2, pos_bias=wl.layer(l).pos_bias,
                   hist_k=wl.layer(l).hist_k, hist_v=wl.layer(l).hist_v) for l in range(wl.layers)]
    refs = olayer.stack_forward(wl.x0, wl.new_len, wl.hist_len, layers, wl.attn_scale, EPS, wl.H,
                                wl.pos_mbits)
    for l in range(wl.layers):
        tol_check(to_np(ys[l]), refs[l], dtype, f"stack {dtype} d={d} ps={ps} layer {l}")


# Timestamp deltas across every branch of the bucket rule: epoch-millisecond
# values, gaps from one to billions (pairs 2^32 and more apart) and steps
# back in time (negative deltas, bucket 0); m = 0 and m = 3 keep buckets of
# deltas past 2^32 below the last bucket, so those are checked exactly.
@pytest.mark.parametrize("mbits,nb", [(0, 64), (3, 1024)])
def test_timestamp_deltas_of_every_range(mbits, nb):
    print(f"case timestamps wide m={mbits} nb={nb}", flush=True)
    hist, new = [0, 40, 700, 3], [90, 60, 120, 200]
    over = dict(dtype="bf16", D=256, H=2, d=128, page_size=32, B=len(hist), layers=1,
                hist=("fixed", hist), new=("fixed", new), pool_pages=4096, ts_buckets=nb, ts_mbits=mbits)
    wl = make_workload(B8_KV_HIT, seed=11, **over)
    rng = np.random.default_rng(11)
    ts = []
    for u in range(wl.B):
        n = int(wl.hist_len[u] + wl.new_len[u])
        kind = rng.integers(0, 4, n)
        gap = np.where(kind == 0, rng.integers(1, 10, n),
              np.where(kind == 1, rng.integers(1_000, 1_000_000, n),
              np.where(kind == 2, rng.integers(1_000_000_000, 6_000_000_000, n),
                       -rng.integers(1, 100_000, n))))
        ts.append((1_700_000_000_000 + np.cumsum(gap)).astype(np.int64))
    wl.timestamps = ts
    d = np.concatenate([t[:, None] - t[None, :] for t in ts if len(t)], axis=None)
    assert (d < 0).any() and (d >= 2**32).any() and ((d > 0) & (d < 8)).any()
    _check_layer(wl, {"ts": True}, f"timestamps m={mbits} nb={nb}")


# Short bursts of new rows (at most 96 per user on average) take the 16-wave
# attention layout (one query group per wave) in bf16; the grid above runs
# the 8-wave layout. One user's 200 rows make a 13-group q-block (one
# phase), the others two phases.
@pytest.mark.parametrize("d,ps,H", [(32, 16, 6), (64, 64, 4), (128, 32, 4)])
def test_sixteen_wave_layout(d, ps, H):
    print(f"case 16-wave layout bf16 d={d} ps={ps} H={H}", flush=True)
    hist, new = [0, 5, 333, 1000, 50, 1], [200, 17, 90, 64, 0, 3]
    assert sum(new) <= 96 * len(new)
    wl = _workload("bf16", d, ps, H, {}, seed=d + 1, hist=hist, new=new)
    _check_layer(wl, {}, f"bf16 d={d} 16 waves")
