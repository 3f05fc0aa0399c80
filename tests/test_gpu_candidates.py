"""Candidate rows, input preprocessing and cache trim on the GPU, against the
oracle (NVIDIA blog "Deploying an HSTU generative recommender with NVIDIA
Dynamo-Triton", sections "Why use HSTU for generative recommendation" and
"Benchmark setup": context, item and action tokens, candidates scored
against a user's history; the candidate mask and the row layout are the
readings the oracle states).

  * the layer with candidate counts against oracle.layer (fp32 rel L2 <=
    1e-4; bf16 rel L2 <= 1e-2, max abs <= 3e-2), with candidate runs that
    cross q-blocks, all-candidate and no-candidate users;
  * preprocessing bit-exact against oracle.preprocess rounded once to the
    dtype (one fp32 add rounded to fp32 or bf16 equals the exact sum
    rounded, since fp64 and fp32 carry more than twice the target's bits);
  * a serving loop -- tokens -> preprocessing -> cached layers with
    candidates -> trim of the candidates -- against the oracle's recompute of
    each user's context, history and current candidates from scratch.
"""
import numpy as np
import pytest
import torch

from gpu_util import EPS, stack_from_workload, to_np, tol_check
from hstu_jagged_silu_fwd_amd import _lib
from hstu_jagged_silu_fwd_amd.kvcache import KVCache
from hstu_jagged_silu_fwd_amd.stack import HSTUStack
from oracle import layer as olayer
from oracle import preprocess as oprep
from workloads import B8_KV_HIT, B8_RECOMPUTE, TINY_FP32, make_workload, round_bf16

pytestmark = pytest.mark.gpu

CASES = {
    "f32-hist": (TINY_FP32, dict(hist=("uniform", 5, 90), new=("uniform", 1, 150), B=5, pool_pages=64,
                                 pos_buckets=32)),
    "bf16-recompute": (B8_RECOMPUTE, dict(B=3, new=("uniform", 256, 700), layers=1)),
    "bf16-kv-hit": (B8_KV_HIT, dict(B=4, hist=("uniform", 256, 1500), new=("uniform", 16, 256), layers=1,
                                    pool_pages=4096)),
}


def _counts(name, n, rng):
    """Candidate counts: all rows, none, one, and runs that cross q-blocks."""
    m = np.array([int(rng.integers(0, k + 1)) for k in n], np.int32)
    if name == "bf16-recompute":
        m[:] = [n[0], min(300, n[1]), 1]
    else:
        m[0] = n[0]
        if len(n) > 1:
            m[1] = 0
    return m


def _run(wl, st, m):
    dev = st.device
    x = torch.from_numpy(wl.x0).to(device=dev, dtype=st.tdtype)
    off = torch.from_numpy(wl.new_offsets).to(dev)
    hl = torch.from_numpy(wl.hist_len).to(dev)
    ts = tso = None
    if wl.timestamps is not None:
        ts = torch.from_numpy(wl.ts_flat()).to(dev)
        tso = torch.from_numpy(wl.ts_offsets()).to(dev)
    y = torch.full_like(x, 7.0)
    st.layer(0, x, off, hl, y, timestamps=ts, ts_offsets=tso, num_candidates=torch.from_numpy(m).to(dev))
    return y, st.read_status()


@pytest.mark.parametrize("case", list(CASES))
def test_layer_with_candidates_matches_oracle(case):
    name, over = CASES[case]
    print(f"case candidates {case}", flush=True)
    wl = make_workload(name, seed=2, **over)
    m = _counts(case, wl.new_len, np.random.default_rng(5))
    print(f"  new={wl.new_len.tolist()} hist={wl.hist_len.tolist()} m={m.tolist()}", flush=True)
    st = stack_from_workload(wl)
    y, code = _run(wl, st, m)
    assert code == 0, f"device status {code}"
    li = wl.layer(0)
    ref = olayer.layer_forward(wl.x0, wl.new_len, wl.hist_len, li.hist_k, li.hist_v, li.w1, li.w2, li.pos_bias,
                               wl.pos_mbits, wl.attn_scale, EPS, wl.H, wl.timestamps, li.ts_bias, wl.ts_mbits,
                               num_candidates=m)["y"]
    tol_check(to_np(y), ref, wl.dtype, f"candidates {case}")


def test_bad_candidate_count_is_rejected_on_device():
    print("case candidates bad count", flush=True)
    wl = make_workload(TINY_FP32, seed=0)
    st = stack_from_workload(wl)
    m = np.array([0, int(wl.new_len[1]) + 1], np.int32)
    y, code = _run(wl, st, m)
    assert code == 6
    assert torch.all(y == 7.0)            # nothing written after the rejection


# ---- preprocessing ----

def _tables(rng, D, dtype, n_items=300, n_actions=5, n_ctx=40, max_pos=2200):
    def t(n):
        a = rng.normal(0, 1, size=(n, D))
        return round_bf16(a) if dtype == "bf16" else a.astype(np.float32).astype(np.float64)
    return dict(item_emb=t(n_items), action_emb=t(n_actions), ctx_emb=t(n_ctx), pos_emb=t(max_pos))


def _batch(rng, B, n_items=300, n_actions=5, n_ctx=40, max_pairs=300, max_cands=100):
    ctx = [rng.integers(0, n_ctx, size=(6 if u % 2 == 0 else 0)).tolist() for u in range(B)]
    items = [rng.integers(0, n_items, size=int(rng.integers(0, max_pairs))).tolist() for u in range(B)]
    actions = [rng.integers(0, n_actions, size=len(it)).tolist() for it in items]
    cands = [rng.integers(0, n_items, size=int(rng.integers(0, max_cands + 1))).tolist() for u in range(B)]
    hist = rng.integers(0, 1400, size=B).tolist()
    return dict(hist_len=hist, ctx=ctx, items=items, actions=actions, cands=cands)


def _jag(lists):
    off = np.concatenate([[0], np.cumsum([len(v) for v in lists])]).astype(np.int32)
    flat = np.array([i for v in lists for i in v], np.int64)
    if flat.size == 0:                      # keep a real device buffer behind every id array
        flat = np.zeros(1, np.int64)
    return off, flat


def _dev_prep(b, tab, dtype, with_actions, T=None, dev="cuda"):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    B = len(b["hist_len"])
    co, ci = _jag(b["ctx"])
    ho, ii = _jag(b["items"])
    _, ai = _jag(b["actions"])
    ko, ki = _jag(b["cands"])
    rows = [len(c) + (2 if with_actions else 1) * len(i) + len(k) for c, i, k in zip(b["ctx"], b["items"], b["cands"])]
    T = sum(rows) if T is None else T
    d = lambda a, t: torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=t)
    out = dict(x=torch.full((T, tab["pos_emb"].shape[1]), 3.0, dtype=tdt, device=dev),
               new_offsets=torch.full((B + 1,), -5, dtype=torch.int32, device=dev),
               num_candidates=torch.full((B,), -5, dtype=torch.int32, device=dev),
               device_status=torch.full((1,), -1, dtype=torch.int32, device=dev))
    _lib.preprocess(hist_len=d(b["hist_len"], torch.int32), ctx_offsets=d(co, torch.int32), ctx_ids=d(ci, torch.int64),
                    hist_offsets=d(ho, torch.int32), item_ids=d(ii, torch.int64),
                    action_ids=d(ai, torch.int64) if with_actions else None, cand_offsets=d(ko, torch.int32),
                    cand_ids=d(ki, torch.int64), item_emb=d(tab["item_emb"], tdt),
                    action_emb=d(tab["action_emb"], tdt) if with_actions else None,
                    ctx_emb=d(tab["ctx_emb"], tdt), pos_emb=d(tab["pos_emb"], tdt), **out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("with_actions", [True, False])
def test_preprocess_bit_exact(dtype, with_actions):
    print(f"case preprocess {dtype} actions={with_actions}", flush=True)
    rng = np.random.default_rng(31)
    tab = _tables(rng, 512, dtype)
    b = _batch(rng, 7)
    b["items"][3] = []                      # a user without history entries
    b["actions"][3] = []
    b["cands"][4] = []                      # and one without candidates
    out = _dev_prep(b, tab, dtype, with_actions)
    assert int(out["device_status"].item()) == 0
    x, new_len, ncand = oprep.preprocess(b["hist_len"], b["ctx"], b["items"], b["actions"] if with_actions else None,
                                         b["cands"], tab["item_emb"], tab["action_emb"], tab["ctx_emb"],
                                         tab["pos_emb"])
    want = round_bf16(x) if dtype == "bf16" else x.astype(np.float32).astype(np.float64)
    got = to_np(out["x"])
    assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} elements differ"
    assert out["new_offsets"].cpu().tolist() == np.concatenate([[0], np.cumsum(new_len)]).tolist()
    assert out["num_candidates"].cpu().tolist() == ncand.tolist()


def test_preprocess_device_errors():
    print("case preprocess errors", flush=True)
    rng = np.random.default_rng(32)
    tab = _tables(rng, 64, "f32", max_pos=600)
    b = _batch(rng, 3, max_pairs=100, max_cands=20)
    b["hist_len"] = [0, 10, 20]
    ok = _dev_prep(b, tab, "f32", True)
    assert int(ok["device_status"].item()) == 0
    bad = dict(b, items=[list(v) for v in b["items"]])
    bad["actions"] = [list(v) for v in b["actions"]]
    bad["items"][0] = bad["items"][0] + [300]              # id past the item table
    bad["actions"][0] = bad["actions"][0] + [0]
    assert int(_dev_prep(bad, tab, "f32", True)["device_status"].item()) == 7
    far = dict(b, hist_len=[0, 10, 590])                    # positions past the table
    assert int(_dev_prep(far, tab, "f32", True)["device_status"].item()) == 8
    T = sum(len(c) + 2 * len(i) + len(k) for c, i, k in zip(b["ctx"], b["items"], b["cands"]))
    short = _dev_prep(b, tab, "f32", True, T=T - 1)        # rows do not add up to T
    assert int(short["device_status"].item()) == 1
    assert torch.all(short["x"] == 3.0)


# ---- serving loop: tokens -> preprocessing -> cached layers with candidates -> trim ----

def _serving_with_candidates(dtype, seed, n_steps):
    L, ps, maxP = 2, 16, 12
    hist_cap = 100                                  # history rows per user before it restarts
    if dtype == "f32":
        wl = make_workload(TINY_FP32, seed=seed, B=2, layers=L, attn_scale=1.0 / 192)
    else:
        wl = make_workload(B8_KV_HIT, seed=seed, B=2, layers=L, hist=("const", 0), new=("const", 16),
                           attn_scale=1.0 / 192)
    D, H = wl.D, wl.H
    rng = np.random.default_rng(seed + 7)
    tab = _tables(rng, D, dtype, n_items=60, n_actions=3, n_ctx=12, max_pos=maxP * ps)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kv = KVCache(num_layers=L, num_pages=64, page_size=ps, max_pages_per_user=maxP, max_users=4)
    st = HSTUStack(num_users=1, num_heads=H, head_dim=wl.d, page_size=ps, num_pool_pages=64,
                   max_pages_per_user=maxP, pos_buckets=wl.pos_buckets, pos_mbits=wl.pos_mbits,
                   attn_scale=wl.attn_scale, norm_eps=EPS, dtype=dtype, num_layers=L)
    layers = []
    for l in range(L):
        li = wl.layer(l)
        st.set_layer(l, w1t=li.w1t, w2t=li.w2t, pos_bias=li.pos_bias, page_table=np.zeros((1, maxP), np.int32))
        layers.append(dict(w1=li.w1, w2=li.w2, pos_bias=li.pos_bias, hist_k=[np.zeros((0, D))],
                           hist_v=[np.zeros((0, D))]))
    users = {}                                      # uid -> dict(ctx, items, actions) sent so far
    kinds = {"hit": 0, "miss": 0}
    for step in range(n_steps):
        B = int(rng.integers(1, 4))
        ids = (rng.choice(6, size=B, replace=False) + 1).tolist()
        cached = kv.lookup(ids).tolist()
        batch = dict(hist_len=[], ctx=[], items=[], actions=[], cands=[])
        for uid, c in zip(ids, cached):
            k = int(rng.integers(0, 10))
            new_items = rng.integers(0, 60, size=k).tolist()
            new_acts = rng.integers(0, 3, size=k).tolist()
            cands = rng.integers(0, 60, size=int(rng.integers(1, 13))).tolist()
            u = users.get(uid)
            if u is not None and 3 + 2 * (len(u["items"]) + k) > hist_cap:   # restart the user
                kv.evict(uid)
                users.pop(uid)
                u, c = None, -1
            if u is None:
                u = users[uid] = dict(ctx=rng.integers(0, 12, size=3).tolist(), items=[], actions=[])
            if c < 0:                               # miss: context and the whole history again
                kinds["miss"] += 1
                batch["ctx"].append(u["ctx"])
                batch["items"].append(u["items"] + new_items)
                batch["actions"].append(u["actions"] + new_acts)
            else:
                kinds["hit"] += 1
                assert c == 3 + 2 * len(u["items"])
                batch["ctx"].append([])
                batch["items"].append(new_items)
                batch["actions"].append(new_acts)
            batch["cands"].append(cands)
            u["items"] = u["items"] + new_items
            u["actions"] = u["actions"] + new_acts
        n_new = [len(c) + 2 * len(i) + len(k) for c, i, k in zip(batch["ctx"], batch["items"], batch["cands"])]
        plan = kv.plan(ids, n_new)
        batch["hist_len"] = plan.hist_len.tolist()
        tables = kv.build_tables(plan)
        prep = _dev_prep(batch, tab, dtype, True)
        assert int(prep["device_status"].item()) == 0
        y = st.forward(prep["x"], prep["new_offsets"], plan.hist_len, page_tables=[tables[l] for l in range(L)],
                       num_candidates=prep["num_candidates"])
        assert st.read_status() == 0
        kv.trim(ids, [len(k) for k in batch["cands"]])
        y = to_np(y)
        off = np.concatenate([[0], np.cumsum(n_new)])
        for b, uid in enumerate(ids):
            u = users[uid]
            x_full, nl, nc = oprep.preprocess([0], [u["ctx"]], [u["items"]], [u["actions"]], [batch["cands"][b]],
                                              tab["item_emb"], tab["action_emb"], tab["ctx_emb"], tab["pos_emb"])
            x_full = round_bf16(x_full) if dtype == "bf16" else x_full.astype(np.float32).astype(np.float64)
            ys = olayer.stack_forward(x_full, nl, [0], layers, wl.attn_scale, EPS, H, wl.pos_mbits,
                                      num_candidates=nc)
            tol_check(y[off[b]:off[b + 1]], ys[-1][-n_new[b]:], dtype, f"step {step} user {uid}")
    return kinds


@pytest.mark.parametrize("dtype,seed", [("f32", 3), ("bf16", 4)])
def test_serving_with_candidates_equals_recompute(dtype, seed):
    print(f"case serving with candidates {dtype}", flush=True)
    kinds = _serving_with_candidates(dtype, seed, 14)
    print(f"  {kinds}", flush=True)
    assert kinds["hit"] > 0 and kinds["miss"] > 0


def test_candidates_at_the_pages_request_size_sampled():
    """The pages' request shape (8 users, 8,198 cached tokens, 100 candidates
    each, hidden 512, bf16): one layer on the GPU, sampled candidate rows of
    every user against the oracle computed for those rows only."""
    print("case candidates full size sampled", flush=True)
    wl = make_workload(B8_KV_HIT, seed=9, B=8, hist=("const", 8198), new=("const", 100), layers=1,
                       pool_pages=4096, max_pages=260)
    st = stack_from_workload(wl)
    m = np.full(8, 100, np.int32)
    y, code = _run(wl, st, m)
    assert code == 0, f"device status {code}"
    rng = np.random.default_rng(3)
    rows = sorted(int(u * 100 + k) for u in range(8) for k in rng.choice(100, size=3, replace=False))
    li = wl.layer(0)
    ref = olayer.layer_forward(wl.x0, wl.new_len, wl.hist_len, li.hist_k, li.hist_v, li.w1, li.w2, li.pos_bias,
                               wl.pos_mbits, wl.attn_scale, EPS, wl.H, rows=rows, num_candidates=m)["y"]
    tol_check(to_np(y)[rows], ref, "bf16", "candidates full size sampled")


def test_preprocess_empty_batch_and_empty_user():
    print("case preprocess empty", flush=True)
    rng = np.random.default_rng(33)
    tab = _tables(rng, 64, "f32", max_pos=300)
    empty = dict(hist_len=[], ctx=[], items=[], actions=[], cands=[])
    out = _dev_prep(empty, tab, "f32", True)
    assert int(out["device_status"].item()) == 0 and out["new_offsets"].cpu().tolist() == [0]
    b = dict(hist_len=[3, 7, 0], ctx=[[1], [], [2, 3]], items=[[4, 5], [], [6]], actions=[[0, 1], [], [2]],
             cands=[[7], [], []])
    out = _dev_prep(b, tab, "f32", True)
    assert int(out["device_status"].item()) == 0
    x, new_len, ncand = oprep.preprocess(b["hist_len"], b["ctx"], b["items"], b["actions"], b["cands"],
                                         tab["item_emb"], tab["action_emb"], tab["ctx_emb"], tab["pos_emb"])
    assert np.array_equal(to_np(out["x"]), x.astype(np.float32).astype(np.float64))
    assert out["new_offsets"].cpu().tolist() == [0, 6, 6, 10] and out["num_candidates"].cpu().tolist() == [1, 0, 0]
