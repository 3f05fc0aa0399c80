"""Pins of the fp64 oracle against brute force, closed forms and invariants.

A plausible slip anywhere in oracle.layer (a dropped bias term, a wrong
causal boundary, a swapped U/V/Q/K block, a transposed operand, a wrong
history/new ordering, a wrong norm) fails at least one of these.
"""
import math

import numpy as np
import pytest

from oracle import brute, layer, paging
from oracle.buckets import bucket
from workloads import B8_KV_HIT, CONFIGS, TINY_FP32, make_workload

EPS = 1e-6


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(np.linalg.norm(b), 1e-300)
    return np.linalg.norm(a - b) / den


def small_case(seed, B=3, news=(0, 1, 5), hists=(0, 3, 7), D=8, H=2, nb=16, mbits=2, ts=False):
    rng = np.random.default_rng(seed)
    news = np.array(news, dtype=np.int64)
    hists = np.array(hists, dtype=np.int64)
    T = int(news.sum())
    x = rng.normal(0, 1, size=(T, D))
    w1 = rng.normal(0, 0.3, size=(D, 4 * D))
    w2 = rng.normal(0, 0.3, size=(D, D))
    hk = [rng.normal(0, 0.5, size=(int(c), D)) for c in hists]
    hv = [rng.normal(0, 0.5, size=(int(c), D)) for c in hists]
    pb = rng.normal(0, 0.5, size=nb)
    kw = dict(x=x, new_len=news, hist_len=hists, hist_k=hk, hist_v=hv, w1=w1,
              w2=w2, pos_bias=pb, pos_mbits=mbits, attn_scale=1.0 / 16,
              eps=EPS, H=H)
    if ts:
        tss = []
        for c, n in zip(hists, news):
            g = 1 + rng.integers(0, 9, size=int(c + n))
            if len(g):
                g[0] = 0
            tss.append(np.cumsum(g))
        kw.update(timestamps=tss, ts_bias=rng.normal(0, 0.5, size=8), ts_mbits=1)
    return kw


def test_silu_identities():
    z = np.linspace(-30, 30, 121)
    s = layer.silu(z)
    assert layer.silu(np.array([0.0]))[0] == 0.0
    # silu(z) - silu(-z) = z
    assert np.max(np.abs(s - layer.silu(-z) - z)) < 1e-12
    assert abs(layer.silu(np.array([50.0]))[0] - 50.0) < 1e-18 * 50 + 1e-12
    assert abs(layer.silu(np.array([-800.0]))[0]) == 0.0


@pytest.mark.parametrize("ts", [False, True])
@pytest.mark.parametrize("seed", [0, 1])
def test_brute_matches_oracle_edge_shapes(seed, ts):
    kw = small_case(seed, ts=ts)
    y = layer.layer_forward(**kw)["y"]
    yb = np.array(brute.layer_brute(**kw))
    assert y.shape == yb.shape
    assert rel_err(y, yb) < 1e-12


def test_brute_matches_oracle_tiny_workload():
    wl = make_workload(TINY_FP32, seed=0)
    li = wl.layer(0)
    kw = dict(x=wl.x0, new_len=wl.new_len, hist_len=wl.hist_len,
              hist_k=li.hist_k, hist_v=li.hist_v, w1=li.w1, w2=li.w2,
              pos_bias=li.pos_bias, pos_mbits=wl.pos_mbits,
              attn_scale=wl.attn_scale, eps=EPS, H=wl.H)
    y = layer.layer_forward(**kw)["y"]
    yb = np.array(brute.layer_brute(**kw))
    assert rel_err(y, yb) < 1e-12


def test_zero_keys_zero_bias_gives_zero_output():
    # K = 0 and zero bias: s = 0, SiLU(0) = 0, so A = 0, O = 0, LN(0) = 0, Y = 0.
    kw = small_case(3, news=(4, 9), hists=(5, 0), B=2)
    D = kw["w1"].shape[0]
    kw["w1"][:, 3 * D:4 * D] = 0.0
    kw["hist_k"] = [np.zeros_like(h) for h in kw["hist_k"]]
    kw["pos_bias"] = np.zeros_like(kw["pos_bias"])
    r = layer.layer_forward(**kw)
    assert np.all(r["o"] == 0.0)
    assert np.all(r["y"] == 0.0)


def test_zero_queries_gives_causal_convolution():
    # Q = 0: a(p, j) = SiLU(pos_bias[b(p - j)]) / N depends on p - j only, so
    # for c = 0 each feature of O is a causal convolution of V with that kernel.
    kw = small_case(4, news=(23,), hists=(0,), B=1, D=8, H=2, nb=12, mbits=2)
    D = 8
    kw["w1"][:, 2 * D:3 * D] = 0.0
    r = layer.layer_forward(**kw)
    n = 23
    w = np.array([layer.silu(np.array([kw["pos_bias"][bucket(dl, 2, 12)]]))[0] for dl in range(n)])
    w *= kw["attn_scale"]
    V = r["v"]
    for e in range(D):
        conv = np.convolve(w, V[:, e])[:n]
        assert np.max(np.abs(conv - r["o"][:, e])) < 1e-13


def test_single_key_closed_form():
    kw = small_case(5, news=(1,), hists=(0,), B=1)
    r = layer.layer_forward(**kw)
    D, H = 8, 2
    d = D // H
    for h in range(H):
        cols = slice(h * d, (h + 1) * d)
        s = float(np.dot(r["q"][0, cols], r["k"][0, cols])) + kw["pos_bias"][0]
        a = s / (1.0 + math.exp(-s)) * kw["attn_scale"]
        assert np.max(np.abs(r["o"][0, cols] - a * r["v"][0, cols])) < 1e-15


@pytest.mark.parametrize("ts", [False, True])
def test_jagged_equals_padded(ts):
    kw = small_case(6, B=4, news=(0, 6, 11, 3), hists=(9, 0, 4, 13), D=16, H=4, nb=20, mbits=2, ts=ts)
    y = layer.layer_forward(**kw)["y"]
    yp = layer.layer_forward_padded(**kw)
    assert rel_err(y, yp) < 1e-12


def test_cached_history_equals_full_recompute_layer():
    # Full recompute over history+new tokens, then the cached path fed the
    # history K/V of that recompute must give the same new-row outputs.
    rng = np.random.default_rng(7)
    D, H = 16, 2
    c, n = 29, 11
    x_full = rng.normal(0, 1, size=(c + n, D))
    w1 = rng.normal(0, 0.3, size=(D, 4 * D))
    w2 = rng.normal(0, 0.3, size=(D, D))
    pb = rng.normal(0, 0.5, size=24)
    common = dict(w1=w1, w2=w2, pos_bias=pb, pos_mbits=2, attn_scale=1 / 64, eps=EPS, H=H)
    full = layer.layer_forward(x=x_full, new_len=[c + n], hist_len=[0],
                               hist_k=[np.zeros((0, D))], hist_v=[np.zeros((0, D))], **common)
    cached = layer.layer_forward(x=x_full[c:], new_len=[n], hist_len=[c],
                                 hist_k=[full["k"][:c]], hist_v=[full["v"][:c]], **common)
    assert rel_err(cached["y"], full["y"][c:]) < 1e-12


def test_cached_history_equals_full_recompute_stack():
    rng = np.random.default_rng(8)
    D, H, L = 16, 4, 3
    cs, ns = [17, 0, 40], [5, 9, 1]
    B = 3
    layers_p = [dict(w1=rng.normal(0, 0.3, size=(D, 4 * D)), w2=rng.normal(0, 0.3, size=(D, D)),
                     pos_bias=rng.normal(0, 0.5, size=24)) for _ in range(L)]
    xs_full = [rng.normal(0, 1, size=(c + n, D)) for c, n in zip(cs, ns)]
    # full recompute stack, user by user (history rows + new rows as new)
    full_layers = [dict(lp, hist_k=[np.zeros((0, D))] * B, hist_v=[np.zeros((0, D))] * B) for lp in layers_p]
    x_cat = np.vstack(xs_full)
    tot = [c + n for c, n in zip(cs, ns)]
    # per layer: recompute to get K/V of history rows
    hist_k = [[None] * B for _ in range(L)]
    hist_v = [[None] * B for _ in range(L)]
    xl = x_cat
    for li, lp in enumerate(full_layers):
        r = layer.layer_forward(xl, tot, [0] * B, lp["hist_k"], lp["hist_v"], lp["w1"], lp["w2"],
                                lp["pos_bias"], 2, 1 / 64, EPS, H)
        off = np.concatenate([[0], np.cumsum(tot)])
        for u in range(B):
            hist_k[li][u] = r["k"][off[u]:off[u] + cs[u]]
            hist_v[li][u] = r["v"][off[u]:off[u] + cs[u]]
        xl = r["y"]
    y_full = xl
    off = np.concatenate([[0], np.cumsum(tot)])
    new_rows = np.concatenate([np.arange(off[u] + cs[u], off[u + 1]) for u in range(B)])
    x_new = np.vstack([xs_full[u][cs[u]:] for u in range(B)])
    cached_layers = [dict(lp, hist_k=hist_k[li], hist_v=hist_v[li]) for li, lp in enumerate(layers_p)]
    ys = layer.stack_forward(x_new, ns, cs, cached_layers, 1 / 64, EPS, H, 2)
    assert rel_err(ys[-1], y_full[new_rows]) < 1e-12


def test_causality():
    kw = small_case(9, B=2, news=(10, 6), hists=(4, 0), D=8, H=2)
    y0 = layer.layer_forward(**kw)["y"]
    x = kw["x"].copy()
    x[6, :] += 1.0          # user 0, new row t = 6
    kw["x"] = x
    y1 = layer.layer_forward(**kw)["y"]
    assert np.array_equal(y0[:6], y1[:6])        # earlier rows of user 0
    assert not np.allclose(y0[6:10], y1[6:10])   # the row itself and later rows move
    assert np.array_equal(y0[10:], y1[10:])      # other user untouched


def test_layer_norm_invariants():
    kw = small_case(10, B=2, news=(7, 12), hists=(3, 8), D=16, H=4)
    r = layer.layer_forward(**kw)
    o, nrm = r["o"], r["nrm"]
    assert np.max(np.abs(nrm.mean(axis=1))) < 1e-12
    var = o.var(axis=1)
    assert np.max(np.abs((nrm ** 2).mean(axis=1) - var / (var + EPS))) < 1e-12


def test_linear_in_w2():
    kw = small_case(11)
    y1 = layer.layer_forward(**kw)["y"]
    kw["w2"] = kw["w2"] * 2.0
    y2 = layer.layer_forward(**kw)["y"]
    assert np.array_equal(y2, 2.0 * y1)


def test_row_subset_matches_full():
    kw = small_case(12, B=3, news=(9, 14, 5), hists=(6, 0, 11), D=16, H=2)
    full = layer.layer_forward(**kw)
    rows = [0, 4, 9, 20, 27]
    part = layer.layer_forward(rows=rows, **kw)
    assert np.array_equal(part["rows"], np.array(rows))
    assert rel_err(part["y"], full["y"][rows]) < 1e-13


def test_query_blocking_invariant():
    kw = small_case(13, B=2, news=(40, 7), hists=(30, 2), D=8, H=2)
    a = layer.layer_forward(q_block=512, **kw)["y"]
    b = layer.layer_forward(q_block=3, **kw)["y"]
    assert rel_err(a, b) < 1e-13


def test_paging_roundtrip_and_permutation_invariance():
    rng = np.random.default_rng(14)
    H, d, ps, P = 2, 4, 4, 40
    D = H * d
    news = np.array([5, 0, 9])
    hists = np.array([3, 2, 0])
    T = int(news.sum())
    k_new = rng.integers(0, 65535, size=(T, D)).astype(np.uint16)
    v_new = rng.integers(0, 65535, size=(T, D)).astype(np.uint16)
    npg = (hists + news + ps - 1) // ps
    for perm_seed in (0, 1):
        perm = np.random.default_rng(perm_seed).permutation(P)
        pt = np.full((3, 4), -1, dtype=np.int32)
        pos = 0
        for u in range(3):
            pt[u, :npg[u]] = perm[pos:pos + npg[u]]
            pos += npg[u]
        kp = np.zeros((P, H, ps, d), np.uint16)
        vp = np.zeros((P, H, d, ps), np.uint16)
        paging.append_scatter(kp, vp, k_new, v_new, news, hists, pt, ps, H)
        r = 0
        for u in range(3):
            K, V = paging.gather_user(kp, vp, pt, u, int(hists[u] + news[u]), ps, H)
            n = int(news[u])
            assert np.array_equal(K[hists[u]:], k_new[r:r + n])
            assert np.array_equal(V[hists[u]:], v_new[r:r + n])
            assert not K[:hists[u]].any()     # history slots untouched
            r += n
        # exactly the touched slots changed
        touched = paging.touched_slots(news, hists, pt, ps)
        nz = {(int(p), int(s)) for p, s in zip(*np.nonzero(kp.any(axis=(1, 3))))}
        assert nz <= touched and len(touched) == int(news.sum())


def test_workload_generator_structure():
    for name in CONFIGS:
        wl = make_workload(name, seed=0, B=4, layers=2) if name != TINY_FP32 else make_workload(TINY_FP32)
        T = wl.T
        assert wl.x0.shape == (T, wl.D)
        assert wl.new_offsets[0] == 0 and np.all(np.diff(wl.new_offsets) >= 0)
        li0, li1 = wl.layer(0), wl.layer(wl.layers - 1)
        used = []
        for li in (li0, li1) if wl.layers > 1 else (li0,):
            for u in range(wl.B):
                k = int(wl.pages_per_user()[u])
                assert np.all(li.page_table[u, :k] >= 0) and np.all(li.page_table[u, :k] < wl.num_pool_pages)
                assert np.all(li.page_table[u, k:] == -1)
                used.extend(li.page_table[u, :k].tolist())
        assert len(used) == len(set(used))      # no page shared across users/layers
        if wl.dtype == "bf16":
            bits = wl.x0.view(np.uint32)
            assert np.all((bits & 0xFFFF) == 0)
    a = make_workload(B8_KV_HIT, seed=5, B=3)
    b = make_workload(B8_KV_HIT, seed=5, B=3)
    assert np.array_equal(a.x0, b.x0) and np.array_equal(a.layer(1).w1, b.layer(1).w1)
