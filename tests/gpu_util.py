"""Helpers shared by the GPU tests: move a seeded workload onto the device
through the library, and compare against the oracle."""
from __future__ import annotations

import numpy as np
import torch

from hstu_jagged_silu_fwd_amd.stack import HSTUStack
from oracle import layer as olayer

EPS = 1e-6
BF16_REL_L2 = 1e-2
BF16_MAX_ABS = 3e-2
F32_REL_L2 = 1e-4


def tol_check(y_gpu, y_ref, dtype: str, what: str = ""):
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite GPU output"
    den = np.linalg.norm(y_ref)
    rel = np.linalg.norm(y_gpu - y_ref) / max(den, 1e-300)
    mx = float(np.max(np.abs(y_gpu - y_ref))) if y_gpu.size else 0.0
    print(f"[parity] {what}: rel_l2={rel:.3e} max_abs={mx:.3e} |ref|={den:.3e}", flush=True)
    if dtype == "bf16":
        assert rel <= BF16_REL_L2 and mx <= BF16_MAX_ABS, (what, rel, mx)
    else:
        assert rel <= F32_REL_L2, (what, rel, mx)
    return rel, mx


def stack_from_workload(wl, num_layers=None, pool_fill=None, layers=None):
    """Device stack for workload `wl`: weights, page tables, and the cached
    history K/V appended with kv_pages_append (positions 0..hist-1)."""
    L = wl.layers if num_layers is None else num_layers
    idx = list(range(L)) if layers is None else list(layers)
    st = HSTUStack(num_users=wl.B, num_heads=wl.H, head_dim=wl.d, page_size=wl.page_size,
                   num_pool_pages=wl.num_pool_pages, max_pages_per_user=wl.max_pages,
                   pos_buckets=wl.pos_buckets, pos_mbits=wl.pos_mbits,
                   attn_scale=wl.attn_scale, norm_eps=EPS, dtype=wl.dtype,
                   ts_buckets=wl.ts_buckets, ts_mbits=wl.ts_mbits, num_layers=len(idx),
                   pool_fill=pool_fill)
    hoff = np.concatenate([[0], np.cumsum(wl.hist_len.astype(np.int64))]).astype(np.int32)
    zeros = np.zeros(wl.B, dtype=np.int32)
    for j, l in enumerate(idx):
        li = wl.layer(l)
        st.set_layer(j, w1t=li.w1t, w2t=li.w2t, pos_bias=li.pos_bias, page_table=li.page_table,
                     ts_bias=li.ts_bias)
        if int(hoff[-1]) > 0:
            k = np.concatenate(li.hist_k, axis=0)
            v = np.concatenate(li.hist_v, axis=0)
            st.append(j, k, v, hoff, zeros)
            code = int(st.status.cpu()[0])
            assert code == 0, f"history append failed with device code {code}"
    return st


def oracle_layer(wl, l, x=None, rows=None, users=None):
    """Oracle output of layer l of `wl` on input x (default: the workload's
    X).  `users` restricts the computation to a subset of users (their rows
    are returned in jagged order)."""
    li = wl.layer(l)
    x = wl.x0 if x is None else x
    if users is None:
        return olayer.layer_forward(x, wl.new_len, wl.hist_len, li.hist_k, li.hist_v, li.w1, li.w2,
                                    li.pos_bias, wl.pos_mbits, wl.attn_scale, EPS, wl.H,
                                    wl.timestamps, li.ts_bias, wl.ts_mbits, rows=rows)
    off = wl.new_offsets
    xs = np.concatenate([x[off[u]:off[u + 1]] for u in users], axis=0)
    sub = lambda a: [a[u] for u in users]
    return olayer.layer_forward(xs, wl.new_len[users], wl.hist_len[users], sub(li.hist_k), sub(li.hist_v),
                                li.w1, li.w2, li.pos_bias, wl.pos_mbits, wl.attn_scale, EPS, wl.H,
                                None if wl.timestamps is None else sub(wl.timestamps), li.ts_bias,
                                wl.ts_mbits, rows=rows)


def user_rows(wl, users):
    off = wl.new_offsets
    return np.concatenate([np.arange(off[u], off[u + 1]) for u in users]).astype(np.int64)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)
