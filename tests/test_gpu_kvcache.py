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


def serving_loop(dtype, seed, n_steps, host_pages=0, stream=None):
    """Runs n_steps batches of recurring users through a stack whose pages
    come from a KVCache small enough to evict (with host_pages > 0, evicted
    users go to a host tier and come back by onboard copies), and checks
    every batch's outputs against the oracle recompute of each user's whole
    sequence.  stream: where every call of the loop runs (default: the
    current stream).  Returns the kinds of users seen and each batch's
    outputs."""
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
    outs = []
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
        kv.copy_pages(plan, st.k_pool, st.v_pool, stream=stream)   # offloads, then onboards, first
        tables = kv.build_tables(plan, stream=stream)
        x = np.vstack(rows) if sum(n_new) else np.zeros((0, D))
        off = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
        if x.shape[0] == 0:
            continue
        y = st.forward(torch.from_numpy(x).to(tdt), off, plan.hist_len,
                       page_tables=[tables[l] for l in range(L)], stream=stream)
        assert st.read_status() == 0
        y = y.float().cpu().numpy().astype(np.float64)
        outs.append(y)
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
    return kinds, outs


@pytest.mark.parametrize("dtype,seed", [("bf16", 9), ("f32", 10)])
def test_serving_loop_with_batches_in_flight_equals_recompute(dtype, seed):
    """Two batches in flight: batch i runs on stream i mod 2 with a
    workspace of its own, and the next batch is planned while earlier ones
    still run.  A batch's users are pinned (hstu_kvcache_pin) from its plan
    until its stream has finished it, so no plan evicts them or hands out
    their pages meanwhile; a batch takes only users not in flight, and a
    plan that cannot fit beside the pinned users waits for the oldest batch
    in flight, unpins it and plans again.  The pool (56 pages, 4 slots, 6
    recurring users) forces evictions.  Every batch must equal the oracle's
    recompute of each user's whole sequence."""
    from hstu_jagged_silu_fwd_amd import _lib
    from hstu_jagged_silu_fwd_amd.kvcache import KVCacheError
    print(f"case kv serving loop with batches in flight {dtype} seed {seed}", flush=True)
    L, ps, maxP, cap, n_steps = 2, 16, 12, 8 * 16, 16
    if dtype == "f32":
        wl = make_workload(TINY_FP32, seed=seed, B=2, layers=L, attn_scale=1.0 / cap)
    else:
        wl = make_workload(B8_KV_HIT, seed=seed, B=2, layers=L, hist=("const", 0), new=("const", 16),
                           attn_scale=1.0 / cap)
    D, H = wl.D, wl.H
    kv = KVCache(num_layers=L, num_pages=56, page_size=ps, max_pages_per_user=maxP, max_users=4)
    st = HSTUStack(num_users=1, num_heads=H, head_dim=wl.d, page_size=ps, num_pool_pages=56,
                   max_pages_per_user=maxP, pos_buckets=wl.pos_buckets, pos_mbits=wl.pos_mbits,
                   attn_scale=wl.attn_scale, norm_eps=EPS, dtype=dtype, num_layers=L)
    layers = []
    for l in range(L):
        li = wl.layer(l)
        st.set_layer(l, w1t=li.w1t, w2t=li.w2t, pos_bias=li.pos_bias, page_table=np.zeros((1, maxP), np.int32))
        layers.append(dict(w1=li.w1, w2=li.w2, pos_bias=li.pos_bias, hist_k=None, hist_v=None))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s_ in streams:
        s_.wait_stream(torch.cuda.current_stream())
    ws = [torch.empty(_lib.stack_workspace_size(st.desc(3 * cap, num_users=3), L), dtype=torch.uint8,
                      device="cuda") for _ in range(2)]
    rng = np.random.default_rng(seed + 200)
    seqs, flight, results = {}, [], []
    kinds = {"hit": 0, "miss_again": 0, "new": 0, "waits": 0, "evicted": 0}

    def retire_oldest():
        ids_, ev_ = flight.pop(0)
        ev_.synchronize()
        kv.unpin(ids_)

    for step in range(n_steps):
        busy = {u for ids_, _ in flight for u in ids_}
        free = [u for u in range(1, 7) if u not in busy]
        if not free:
            retire_oldest()
            free = [u for u in range(1, 7) if u not in {u for ids_, _ in flight for u in ids_}]
        B = int(rng.integers(1, min(3, len(free)) + 1))
        ids = [int(u) for u in rng.choice(free, size=B, replace=False)]
        fresh = [int(k) for k in rng.integers(1, 40, size=B)]
        cached = kv.lookup(ids).tolist()
        rows, n_new, new_seqs = [], [], {}
        for uid, c, k in zip(ids, cached, fresh):
            xnew = rng.standard_normal((k, D))
            if dtype == "bf16":
                xnew = torch.from_numpy(xnew).to(torch.bfloat16).double().numpy()
            prev = seqs.get(uid, np.zeros((0, D)))
            if c < 0 and prev.shape[0] > 0:
                kinds["miss_again"] += 1
                send = np.vstack([prev, xnew])
            elif c < 0:
                kinds["new"] += 1
                send = xnew
            else:
                kinds["hit"] += 1
                assert c == prev.shape[0]
                send = xnew
            if prev.shape[0] + k > cap:                  # restart the user's sequence
                send, xnew = send[:0], xnew[:0]
                kv.evict(uid)
                seqs.pop(uid, None)
                prev = np.zeros((0, D))
            new_seqs[uid] = np.vstack([prev, xnew])
            rows.append(send)
            n_new.append(send.shape[0])
        while True:
            try:
                plan = kv.plan(ids, n_new)
                break
            except KVCacheError as e:                    # full beside the pinned users: wait for one
                assert e.code == -10 and flight, e
                kinds["waits"] += 1
                retire_oldest()
        kinds["evicted"] += len(plan.evicted)
        seqs.update(new_seqs)
        if sum(n_new) == 0:
            continue
        kv.pin(ids)
        s_ = streams[step % 2]
        tables = kv.build_tables(plan, stream=s_)
        x = torch.from_numpy(np.vstack(rows)).to(tdt)
        off = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
        y = st.forward(x, off, plan.hist_len, page_tables=[tables[l] for l in range(L)], stream=s_,
                       workspace=ws[step % 2])
        ev = torch.cuda.Event()
        ev.record(s_)
        flight.append((ids, ev))
        want = []
        for b, uid in enumerate(ids):
            if n_new[b] == 0:
                continue
            full = seqs[uid]
            ys = olayer.stack_forward(full, [full.shape[0]], [0],
                                      [dict(l0, hist_k=[np.zeros((0, D))], hist_v=[np.zeros((0, D))])
                                       for l0 in layers], wl.attn_scale, EPS, H, wl.pos_mbits)
            want.append((b, uid, ys[-1][-n_new[b]:]))
        results.append((step, y, off, want, ws[step % 2], s_))
    while flight:
        retire_oldest()
    torch.cuda.synchronize()
    print(f"[kvcache] in flight {kinds}", flush=True)
    for step, y, off, want, w, s_ in results:
        assert st.read_status(w) == 0
        yn = y.float().cpu().numpy().astype(np.float64)
        # the batch's rows together (a one-row user's output can be tiny)
        got_rows = np.vstack([yn[off[b]:off[b + 1]] for b, _, _ in want])
        tol_check(got_rows, np.vstack([ref for _, _, ref in want]), dtype, f"in flight step {step}")
    assert kinds["hit"] > 0 and kinds["evicted"] > 0


@pytest.mark.parametrize("dtype,seed", [("f32", 3), ("bf16", 4)])
def test_serving_loop_with_eviction_equals_recompute(dtype, seed):
    print(f"case kv serving loop {dtype} seed {seed}", flush=True)
    kinds, _ = serving_loop(dtype, seed, 14)
    print(f"[kvcache] {kinds}", flush=True)
    assert kinds["hit"] > 0 and kinds["new"] > 0


@pytest.mark.parametrize("dtype,seed", [("f32", 5), ("bf16", 6)])
def test_serving_loop_with_host_tier_equals_recompute(dtype, seed):
    """Evicted users are offloaded and come back as host hits: their K/V
    reach the layers only through the offload and onboard copies."""
    print(f"case kv serving loop with host tier {dtype} seed {seed}", flush=True)
    kinds, _ = serving_loop(dtype, seed, 16, host_pages=64)
    print(f"[kvcache] {kinds}", flush=True)
    assert kinds["host_hit"] > 0 and kinds["hit"] > 0


@pytest.mark.parametrize("dtype,seed", [("bf16", 7)])
def test_serving_loop_on_a_side_stream_equals_default_stream(dtype, seed):
    """The same serving loop (host tier included) with every call -- page
    copies, table builds, the stack -- on a side stream gives the default
    stream's outputs bit for bit: the bindings stage their inputs and
    allocate their outputs on the stream the call runs on."""
    print(f"case kv serving loop on a side stream {dtype} seed {seed}", flush=True)
    _, ref = serving_loop(dtype, seed, 10, host_pages=64)
    side = torch.cuda.Stream()
    kinds, got = serving_loop(dtype, seed, 10, host_pages=64, stream=side)
    print(f"[kvcache] side stream {kinds}", flush=True)
    assert len(got) == len(ref)
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)


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


def test_serving_loop_with_copies_overlapping_layers_equals_recompute():
    """Host-tier copies on a copy stream overlapped with the previous batch's
    layers on the compute stream, ordered by events (NVIDIA blog, same
    section: a host storage tier with onboard and offload).  Batch i's plan
    also names batch i-1's users (with no new tokens), so no in-flight user
    is evicted or has its pages handed out; batch i's copies wait for the
    layers of batch i-2 (whose pages an offload may read) and batch i's
    layers wait for its copies.  Every batch must still equal the oracle's
    recompute of each user's whole sequence."""
    print("case kv serving loop with overlapped copies", flush=True)
    dtype, seed, n_steps = "bf16", 8, 16
    L, ps, maxP, cap = 2, 16, 12, 8 * 16
    wl = make_workload(B8_KV_HIT, seed=seed, B=2, layers=L, hist=("const", 0), new=("const", 16),
                       attn_scale=1.0 / cap)
    D, H = wl.D, wl.H
    kv = KVCache(num_layers=L, num_pages=80, page_size=ps, max_pages_per_user=maxP, max_users=6, host_pages=96)
    st = HSTUStack(num_users=1, num_heads=H, head_dim=wl.d, page_size=ps, num_pool_pages=80,
                   max_pages_per_user=maxP, pos_buckets=wl.pos_buckets, pos_mbits=wl.pos_mbits,
                   attn_scale=wl.attn_scale, norm_eps=EPS, dtype=dtype, num_layers=L)
    layers = []
    for l in range(L):
        li = wl.layer(l)
        st.set_layer(l, w1t=li.w1t, w2t=li.w2t, pos_bias=li.pos_bias, page_table=np.zeros((1, maxP), np.int32))
        layers.append(dict(w1=li.w1, w2=li.w2, pos_bias=li.pos_bias, hist_k=None, hist_v=None))
    rng = np.random.default_rng(seed + 100)
    compute, copier = torch.cuda.current_stream(), torch.cuda.Stream()
    seqs, pending, kinds = {}, None, {"hit": 0, "host_hit": 0, "miss_again": 0, "new": 0}
    prev_ids, fwd_done = [], []          # users of the batch in flight; events after each batch's layers

    def check(p):
        ids_, n_, off_, y_, want_ = p
        assert st.read_status() == 0
        y_ = y_.float().cpu().numpy().astype(np.float64)
        for b, uid in enumerate(ids_):
            if n_[b] == 0:
                continue
            full = want_[uid]
            ys = olayer.stack_forward(full, [full.shape[0]], [0],
                                      [dict(l0, hist_k=[np.zeros((0, D))], hist_v=[np.zeros((0, D))])
                                       for l0 in layers], wl.attn_scale, EPS, H, wl.pos_mbits)
            tol_check(y_[off_[b]:off_[b + 1]], ys[-1][-n_[b]:], dtype, f"overlap user {uid}")

    for step in range(n_steps):
        B = int(rng.integers(1, 4))
        ids = (rng.choice(9, size=B, replace=False) + 1).tolist()
        fresh = [int(k) for k in rng.integers(1, 40, size=B)]
        # a user of the batch in flight is not restarted (its pages are being
        # read): it sits this batch out
        keep = [j for j, u in enumerate(ids)
                if not (u in prev_ids and seqs.get(u, np.zeros((0, D))).shape[0] + fresh[j] > cap)]
        ids, fresh = [ids[j] for j in keep], [fresh[j] for j in keep]
        if not ids:
            continue
        B = len(ids)
        cached, tiers = kv.lookup(ids, with_tier=True)
        rows, n_new = [], []
        for uid, c, k, tr in zip(ids, cached.tolist(), fresh, tiers.tolist()):
            xnew = torch.from_numpy(rng.standard_normal((k, D))).to(torch.bfloat16).double().numpy()
            prev = seqs.get(uid, np.zeros((0, D)))
            if prev.shape[0] + k > cap:                # restart the user's sequence
                kv.evict(uid)
                prev, c = np.zeros((0, D)), -1
            if c < 0:
                kinds["miss_again" if prev.shape[0] else "new"] += 1
                send = np.vstack([prev, xnew])
            else:
                kinds["host_hit" if tr == 2 else "hit"] += 1
                send = xnew
            seqs[uid] = np.vstack([prev, xnew])
            rows.append(send)
            n_new.append(send.shape[0])
        guard = [u for u in prev_ids if u not in ids]
        plan = kv.plan(ids + guard, n_new + [0] * len(guard))
        # copies on the copy stream, after the layers of batch i-2
        if len(fwd_done) >= 2:
            copier.wait_event(fwd_done[-2])
        kv.copy_pages(plan, st.k_pool, st.v_pool, stream=copier)
        copied = torch.cuda.Event()
        copied.record(copier)
        if pending is not None:                        # batch i-1's results (its layers overlapped the copies)
            check(pending)
        compute.wait_event(copied)
        tables = kv.build_tables(plan)
        x = torch.from_numpy(np.vstack(rows)).to(torch.bfloat16)
        off = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
        y = st.forward(x, off, plan.hist_len[:B], page_tables=[tables[l, :B] for l in range(L)])
        done = torch.cuda.Event()
        done.record(compute)
        fwd_done.append(done)
        pending = (ids, n_new, off, y, {u: seqs[u].copy() for u in ids})
        prev_ids = ids
    check(pending)
    print(f"[kvcache] overlapped {kinds}", flush=True)
    assert kinds["host_hit"] > 0 and kinds["hit"] > 0
