"""GPU layer output vs the fp64 oracle on the same seeded inputs.

Reduced sizes keep the oracle to seconds while still spanning several
q-blocks, key chunks and pages, with ragged tails; tolerances: bf16 relative
L2 <= 1e-2 and max abs <= 3e-2, fp32 relative L2 <= 1e-4.
"""
import numpy as np
import pytest
import torch

from gpu_util import oracle_layer, stack_from_workload, to_np, tol_check
from oracle import layer as olayer
from workloads import B8_KV_HIT, B8_KV_HIT_LONG, B8_RECOMPUTE, B64_SERVING, TINY_FP32, make_workload

pytestmark = pytest.mark.gpu

REDUCED = {
    B8_RECOMPUTE: dict(B=3, new=("uniform", 256, 700), layers=1),
    B8_KV_HIT: dict(B=4, hist=("uniform", 256, 1500), new=("uniform", 16, 256), layers=1, pool_pages=4096),
    B8_KV_HIT_LONG: dict(B=2, hist=("uniform", 4096, 6000), layers=1, pool_pages=1024),
    B64_SERVING: dict(B=6, hist=("zipf", 1.2, 32, 3000), new=("uniform", 1, 512), layers=1, pool_pages=4096,
            miss_frac=0.34),
}


def run_layer(wl, st, l=0):
    dev = st.device
    x = torch.from_numpy(wl.x0).to(device=dev, dtype=st.tdtype)
    off = torch.from_numpy(wl.new_offsets).to(dev)
    hl = torch.from_numpy(wl.hist_len).to(dev)
    ts = tso = None
    if wl.timestamps is not None:
        ts = torch.from_numpy(wl.ts_flat()).to(dev)
        tso = torch.from_numpy(wl.ts_offsets()).to(dev)
    y = torch.empty_like(x)
    st.layer(l, x, off, hl, y, timestamps=ts, ts_offsets=tso)
    code = st.read_status()
    assert code == 0, f"device status {code}"
    return y


def test_tiny_fp32_full():
    print("case tiny fp32 full", flush=True)
    wl = make_workload(TINY_FP32, seed=0)
    st = stack_from_workload(wl)
    y = run_layer(wl, st)
    ref = oracle_layer(wl, 0)["y"]
    tol_check(to_np(y), ref, "f32", "tiny fp32")


@pytest.mark.parametrize("seed", [0, 1])
def test_tiny_fp32_seeds_with_history(seed):
    # The tiny fp32 model with a cached history prefix and a random pool.
    print(f"case tiny fp32 with history seed={seed}", flush=True)
    wl = make_workload(TINY_FP32, seed=seed, hist=("uniform", 5, 90), new=("uniform", 1, 150), B=5,
                       pool_pages=64, pos_buckets=32)
    st = stack_from_workload(wl)
    y = run_layer(wl, st)
    tol_check(to_np(y), oracle_layer(wl, 0)["y"], "f32", f"tiny fp32 with history seed {seed}")


@pytest.mark.parametrize("name", [B8_RECOMPUTE, B8_KV_HIT, B8_KV_HIT_LONG, B64_SERVING])
def test_reduced_bf16_layer(name):
    print(f"case reduced {name}", flush=True)
    wl = make_workload(name, seed=0, **REDUCED[name])
    st = stack_from_workload(wl)
    y = run_layer(wl, st)
    tol_check(to_np(y), oracle_layer(wl, 0)["y"], "bf16", f"{name} reduced")


def test_reduced_kv_hit_stack():
    print("case reduced 3-layer paged-KV-hit stack", flush=True)
    wl = make_workload(B8_KV_HIT, seed=2, B=3, hist=("uniform", 256, 900), new=("uniform", 16, 256),
                       pool_pages=4096)
    st = stack_from_workload(wl)
    ys = st.forward(wl.x0, wl.new_offsets, wl.hist_len, return_all=True)
    assert st.read_status() == 0
    layers = [dict(w1=wl.layer(l).w1, w2=wl.layer(l).w2, pos_bias=wl.layer(l).pos_bias,
                   hist_k=wl.layer(l).hist_k, hist_v=wl.layer(l).hist_v) for l in range(wl.layers)]
    refs = olayer.stack_forward(wl.x0, wl.new_len, wl.hist_len, layers, wl.attn_scale, 1e-6, wl.H,
                                wl.pos_mbits)
    for l in range(wl.layers):
        tol_check(to_np(ys[l]), refs[l], "bf16", f"kv-hit stack layer {l}")


@pytest.mark.parametrize("name", [B8_RECOMPUTE, B8_KV_HIT])
def test_reduced_bf16_other_layers_fed_x0(name):
    # Each layer's own weights/history on the generator's X (per-layer parity).
    wl = make_workload(name, seed=3, **dict(REDUCED[name], layers=3))
    for l in (1, 2):
        print(f"case reduced {name} layer {l}", flush=True)
        st = stack_from_workload(wl, layers=[l])
        y = run_layer(wl, st)
        tol_check(to_np(y), oracle_layer(wl, l)["y"], "bf16", f"{name} layer {l}")
