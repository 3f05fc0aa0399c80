"""Paged KV cache manager on the GPU: the device page-table builder against
the host plan (bit-exact), and a serving loop -- recurring users, hits that
append to cached pages, misses after LRU eviction that resend the whole
sequence -- whose outputs must equal the oracle's full recompute of each
user's whole sequence (NVIDIA blog "Deploying an HSTU generative recommender
with NVIDIA Dynamo-Triton", section "Why serving large sequential
recommenders is hard": lookup / allocate / append / evict over a paged KV
table, cached history reused instead of recomputed)."""
import numpy as np
import pytest
import torch

from gpu_util import EPS, tol_check
from hstu_jagged_silu_fwd_amd.kvcache import KVCache
from hstu_jagged_silu_fwd_amd.stack import HSTUStack
from oracle import layer as olayer
from oracle.kvcache import RefKVCache
from workloads import B8_KV_HIT, TINY_FP32, make_workload

pytestmark = pytest.mark.gpu


def test_table_builder_matches_host_directory():
    print("case kv table builder", flush=True)
    rng = np.random.default_rng(11)
    cfg = dict(num_layers=3, num_pages=500, page_size=16, max_pages_per_user=24, max_users=12)
    kv, ref = KVCache(**cfg), RefKVCache(**cfg)
    directory = np.full((cfg["max_users"], cfg["num_layers"], cfg["max_pages_per_user"]), -1, np.int32)
    for step in range(40):
        B = int(rng.integers(1, 7))
        ids = (rng.choice(30, size=B, replace=False) + 100).tolist()
        n = rng.integers(0, 80, size=B).tolist()
        try:
            ref.plan(ids, n)
        except Exception:
            continue
        p = kv.plan(ids, n)
        for s, l, i, pid in p.updates.tolist():
            directory[s, l, i] = pid
        tables = kv.build_tables(p).cpu().numpy()
        assert tables.shape == (cfg["num_layers"], B, cfg["max_pages_per_user"])
        for b, uid in enumerate(ids):
            for l in range(cfg["num_layers"]):
                want = ref.page_table(uid, l)
                assert tables[l, b, :len(want)].tolist() == want, (step, uid, l)
                assert np.array_equal(tables[l, b], directory[p.slots[b], l]), (step, uid, l)


def serving_loop(dtype, seed, n_steps, host_pages=0):
    """Runs n_steps batches of recurring users through a stack whose pages
    come from a KVCache small enough to evict (with host_pages > 0, evicted
    users go to a host tier and come back by onboard copies), and checks
    every batch's outputs against the oracle recompute of each user's whole
    sequence."""
    # a user's sequence is capped at 8 pages of 16 tokens (restarted past
    # that), so a batch of up to 3 users needs at most 48 of the 56 pages and
    # always fits; 6 recurring users over 4 slots and 56 pages force evictions.
    # 1/N is the longest sequence, as in the workloads.
    L = 2
    ps, maxP, cap = 16, 12, 8 * 16
    if dtype == "f32":
        wl = make_workload(TINY_FP32, seed=seed, B=2, layers=L, attn_scale=1.0 / cap)
    else:
        wl = make_workload(B8_KV_HIT, seed=seed, B=2, layers=L, hist=("const", 0), new=("const", 16),
                           attn_scale=1.0 / cap)
    D, H = wl.D, wl.H
    cfg = dict(num_layers=L, num_pages=56, page_size=ps, max_pages_per_user=maxP, max_users=4,
               host_pages=host_pages)
    kv = KVCache(**cfg)
    st = HSTUStack(num_users=1, num_heads=H, head_dim=wl.d, page_size=ps, num_pool_pages=cfg["num_pages"],
                   max_pages_per_user=maxP, pos_buckets=wl.pos_buckets, pos_mbits=wl.pos_mbits,
                   attn_scale=wl.attn_scale, norm_eps=EPS, dtype=dtype, num_layers=L)
    layers = []
    for l in range(L):
        li = wl.layer(l)
        st.set_layer(l, w1t=li.w1t, w2t=li.w2t, pos_bias=li.pos_bias,
                     page_table=np.zeros((1, maxP), np.int32))
        layers.append(dict(w1=li.w1, w2=li.w2, pos_bias=li.pos_bias, hist_k=None, hist_v=None))
    rng = np.random.default_rng(seed + 100)
    seqs = {}                       # user -> all input rows sent so far (the stack's x)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kinds = {"hit": 0, "host_hit": 0, "miss_again": 0, "new": 0}
    for step in range(n_steps):
        B = int(rng.integers(1, 4))
        ids = (rng.choice(6, size=B, replace=False) + 1).tolist()
        fresh = [int(k) for k in rng.integers(1, 40, size=B)]
        cached, tiers = kv.lookup(ids, with_tier=True)
        rows, n_new = [], []
        for uid, c, k, tr in zip(ids, cached.tolist(), fresh, tiers.tolist()):
            xnew = rng.standard_normal((k, D))
            if dtype == "bf16":
                xnew = torch.from_numpy(xnew).to(torch.bfloat16).double().numpy()
            prev = seqs.get(uid, np.zeros((0, D)))
            if c < 0 and prev.shape[0] > 0:          # evicted: resend the whole sequence
                kinds["miss_again"] += 1
                send = np.vstack([prev, xnew])
            elif c < 0:
                kinds["new"] += 1
                send = xnew
            else:
                kinds["host_hit" if tr == 2 else "hit"] += 1
                assert c == prev.shape[0]
                send = xnew
            if prev.shape[0] + k > cap:              # restart the user's sequence
                send, xnew = send[:0], xnew[:0]
                kv.evict(uid)
                seqs.pop(uid, None)
                prev = np.zeros((0, D))
            seqs[uid] = np.vstack([prev, xnew])
            rows.append(send)
            n_new.append(send.shape[0])
        plan = kv.plan(ids, n_new)
        for uid, h in zip(ids, plan.hist_len.tolist()):
            assert h == seqs[uid].shape[0] - n_new[ids.index(uid)]
        kv.copy_pages(plan, st.k_pool, st.v_pool)     # offloads, then onboards, before the layers
        tables = kv.build_tables(plan)
        x = np.vstack(rows) if sum(n_new) else np.zeros((0, D))
        off = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
        if x.shape[0] == 0:
            continue
        y = st.forward(torch.from_numpy(x).to(tdt), off, plan.hist_len,
                       page_tables=[tables[l] for l in range(L)])
        assert st.read_status() == 0
        y = y.float().cpu().numpy().astype(np.float64)
        # oracle: each user's whole sequence recomputed from scratch; its last
        # n_new rows are the batch's rows
        for b, uid in enumerate(ids):
            if n_new[b] == 0:
                continue
            full = seqs[uid]
            ys = olayer.stack_forward(full, [full.shape[0]], [0],
                                      [dict(l0, hist_k=[np.zeros((0, D))], hist_v=[np.zeros((0, D))])
                                       for l0 in layers],
                                      wl.attn_scale, EPS, H, wl.pos_mbits)
            tol_check(y[off[b]:off[b + 1]], ys[-1][-n_new[b]:], dtype, f"step {step} user {uid}")
    return kinds


@pytest.mark.parametrize("dtype,seed", [("f32", 3), ("bf16", 4)])
def test_serving_loop_with_eviction_equals_recompute(dtype, seed):
    print(f"case kv serving loop {dtype} seed {seed}", flush=True)
    kinds = serving_loop(dtype, seed, 14)
    print(f"[kvcache] {kinds}", flush=True)
    assert kinds["hit"] > 0 and kinds["new"] > 0


@pytest.mark.parametrize("dtype,seed", [("f32", 5), ("bf16", 6)])
def test_serving_loop_with_host_tier_equals_recompute(dtype, seed):
    """Evicted users are offloaded and come back as host hits: their K/V
    reach the layers only through the offload and onboard copies."""
    print(f"case kv serving loop with host tier {dtype} seed {seed}", flush=True)
    kinds = serving_loop(dtype, seed, 16, host_pages=64)
    print(f"[kvcache] {kinds}", flush=True)
    assert kinds["host_hit"] > 0 and kinds["hit"] > 0


def test_page_copies_round_trip_bit_exact():
    """Offload pages to the host tier, onboard them into other pages: every
    byte arrives unchanged (bf16 bit patterns, both pools)."""
    print("case kv page copies", flush=True)
    from hstu_jagged_silu_fwd_amd.kvcache import Plan
    kv = KVCache(num_layers=1, num_pages=64, page_size=32, max_pages_per_user=8, max_users=4, host_pages=40)
    g = torch.Generator().manual_seed(0)
    kp = torch.randint(-32768, 32767, (64, 4, 32, 128), dtype=torch.int16, generator=g).view(torch.bfloat16).cuda()
    vp = torch.randint(-32768, 32767, (64, 4, 128, 32), dtype=torch.int16, generator=g).view(torch.bfloat16).cuda()
    k0, v0 = kp.clone(), vp.clone()
    src = list(range(0, 60, 2))                    # 30 pages out to host pages 39, 38, ...
    hostp = [39 - i for i in range(len(src))]
    off = np.array([[0, s_, h, 0] for s_, h in zip(src, hostp)], np.int32)
    kv.copy_pages(Plan(np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros((0, 4), np.int32), [], off), kp, vp)
    torch.cuda.synchronize()
    hk, hv = kv.host_k, kv.host_v
    for s_, h in zip(src, hostp):
        assert torch.equal(hk[h].view(torch.int16), k0[s_].cpu().view(torch.int16))
        assert torch.equal(hv[h].view(torch.int16), v0[s_].cpu().view(torch.int16))
    dst = [p + 1 for p in src]                     # back into the odd pages
    on = np.array([[1, d, h, 0] for d, h in zip(dst, hostp)], np.int32)
    kv.copy_pages(Plan(np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros((0, 4), np.int32), [], on), kp, vp)
    torch.cuda.synchronize()
    for s_, d in zip(src, dst):
        assert torch.equal(kp[d].view(torch.int16), k0[s_].view(torch.int16))
        assert torch.equal(vp[d].view(torch.int16), v0[s_].view(torch.int16))
    untouched = [p for p in range(64) if p not in set(dst)]
    assert torch.equal(kp[untouched].view(torch.int16), k0[untouched].view(torch.int16))
