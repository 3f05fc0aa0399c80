"""Paged KV cache manager (host side, no GPU): the reference model and the
library against a hand-worked trace, the library against the model on
seeded random traces, and the policy's invariants.

Policy: lookup / allocation / LRU eviction of whole users over the paged
pool, NVIDIA blog "Deploying an HSTU generative recommender with NVIDIA
Dynamo-Triton", section "Why serving large sequential recommenders is hard"
(rule stated in include/hstu_kvcache.h)."""
import json
import os

import numpy as np
import pytest

from oracle.kvcache import CacheFull, Pinned, RefKVCache, TooLong
from hstu_jagged_silu_fwd_amd.kvcache import KVCache, KVCacheError

HERE = os.path.dirname(os.path.abspath(__file__))
TRACE = json.load(open(os.path.join(HERE, "golden", "kvcache_trace.json")))
HOST_TRACE = json.load(open(os.path.join(HERE, "golden", "kvcache_host_trace.json")))
ERR = {"full": -10, "too_long": -11, "invalid": -1, "pinned": -14}


def test_reference_model_follows_the_hand_worked_trace():
    ref = RefKVCache(**TRACE["config"])
    for st in TRACE["steps"]:
        if "error" in st:
            exc = {"full": CacheFull, "too_long": TooLong, "invalid": ValueError}[st["error"]]
            before = (dict((k, (v.length, v.slot)) for k, v in ref.users.items()), list(ref.free_pages))
            with pytest.raises(exc):
                ref.plan(st["ids"], st["n_new"])
            assert before == (dict((k, (v.length, v.slot)) for k, v in ref.users.items()), list(ref.free_pages))
            continue
        hist, slots, updates, evicted = ref.plan(st["ids"], st["n_new"])
        assert hist == st["hist"] and slots == st["slots"], st["why"]
        assert [list(u) for u in updates] == st["updates"], st["why"]
        assert evicted == st["evicted"], st["why"]
    fin = TRACE["final"]
    assert ref.lookup([int(k) for k in fin["lookup"]]) == list(fin["lookup"].values())
    assert len(ref.free_pages) == fin["free_pages"] and len(ref.users) == fin["cached_users"]
    for uid, per_layer in fin["tables"].items():
        assert [ref.page_table(int(uid), l) for l in range(len(per_layer))] == per_layer


def test_library_follows_the_hand_worked_trace():
    kv = KVCache(**TRACE["config"])
    for st in TRACE["steps"]:
        if "error" in st:
            before = (kv.stats(), kv.lookup([10, 20, 30]).tolist())
            with pytest.raises(KVCacheError) as ei:
                kv.plan(st["ids"], st["n_new"])
            assert ei.value.code == ERR[st["error"]], st["why"]
            assert (kv.stats(), kv.lookup([10, 20, 30]).tolist()) == before
            continue
        p = kv.plan(st["ids"], st["n_new"])
        assert p.hist_len.tolist() == st["hist"] and p.slots.tolist() == st["slots"], st["why"]
        assert p.updates.tolist() == st["updates"], st["why"]
        assert p.evicted == st["evicted"], st["why"]
    fin = TRACE["final"]
    assert kv.lookup([int(k) for k in fin["lookup"]]).tolist() == list(fin["lookup"].values())
    assert kv.stats() == (fin["free_pages"], fin["cached_users"])


def test_host_tier_reference_model_follows_the_hand_worked_trace():
    ref = RefKVCache(**HOST_TRACE["config"])
    for st in HOST_TRACE["steps"]:
        hist, slots, updates, evicted = ref.plan(st["ids"], st["n_new"])
        assert hist == st["hist"] and slots == st["slots"], st["why"]
        assert [list(u) for u in updates] == st["updates"], st["why"]
        assert [list(c) for c in ref.last_copies] == st["copies"], st["why"]
        assert evicted == st["evicted"], st["why"]
    fin = HOST_TRACE["final"]
    ids = [int(k) for k in fin["lookup"]]
    assert ref.lookup(ids) == list(fin["lookup"].values())
    assert ref.tier(ids) == list(fin["tier"].values())
    assert (len(ref.free_pages), len(ref.users), len(ref.host_free), len(ref.host)) == \
        (fin["free_pages"], fin["cached_users"], fin["free_host_pages"], fin["host_users"])


def test_host_tier_library_follows_the_hand_worked_trace():
    kv = KVCache(**HOST_TRACE["config"])
    for st in HOST_TRACE["steps"]:
        p = kv.plan(st["ids"], st["n_new"])
        assert p.hist_len.tolist() == st["hist"] and p.slots.tolist() == st["slots"], st["why"]
        assert p.updates.tolist() == st["updates"], st["why"]
        assert p.copies[:, :3].tolist() == st["copies"], st["why"]
        assert p.evicted == st["evicted"], st["why"]
    fin = HOST_TRACE["final"]
    ids = [int(k) for k in fin["lookup"]]
    lens, tiers = kv.lookup(ids, with_tier=True)
    assert lens.tolist() == list(fin["lookup"].values()) and tiers.tolist() == list(fin["tier"].values())
    assert kv.stats(host=True) == (fin["free_pages"], fin["cached_users"], fin["free_host_pages"],
                                   fin["host_users"])


def random_trace(rng, n_batches, max_b, n_ids, max_new):
    for _ in range(n_batches):
        B = int(rng.integers(0, max_b + 1))
        ids = rng.choice(n_ids, size=min(B, n_ids), replace=False).astype(np.int64) * 7919 + 3
        n = rng.integers(0, max_new + 1, size=ids.shape[0])
        yield ids.tolist(), n.tolist()


@pytest.mark.parametrize("seed,host", [(0, False), (1, False), (2, False), (3, False),
                                       (10, True), (11, True), (12, True), (13, True)])
def test_library_matches_reference_model_on_random_traces(seed, host):
    rng = np.random.default_rng(seed)
    cfg = dict(num_layers=int(rng.integers(1, 4)), num_pages=int(rng.integers(20, 200)),
               page_size=int(2 ** rng.integers(2, 6)), max_pages_per_user=int(rng.integers(2, 12)),
               max_users=int(rng.integers(2, 16)))
    if host:
        cfg["host_pages"] = int(rng.integers(4, 300))
    ref, kv = RefKVCache(**cfg), KVCache(**cfg)
    outcomes = {"ok": 0, "full": 0, "too_long": 0}
    for ids, n in random_trace(rng, 300, 6, 24, 3 * cfg["page_size"]):
        try:
            want = ref.plan(ids, n)
        except (CacheFull, TooLong) as e:
            kind = "full" if isinstance(e, CacheFull) else "too_long"
            outcomes[kind] += 1
            with pytest.raises(KVCacheError) as ei:
                kv.plan(ids, n)
            assert ei.value.code == ERR[kind]
            continue
        outcomes["ok"] += 1
        got = kv.plan(ids, n)
        assert got.hist_len.tolist() == want[0]
        assert got.slots.tolist() == want[1]
        assert [tuple(u) for u in got.updates.tolist()] == [tuple(u) for u in want[2]]
        assert got.evicted == want[3]
        assert [tuple(c) for c in got.copies[:, :3].tolist()] == [tuple(c) for c in ref.last_copies]
        assert kv.stats(host=True) == (len(ref.free_pages), len(ref.users), len(ref.host_free), len(ref.host))
        probe = list(range(3, 24 * 7919, 7919 * 3))
        lens, tiers = kv.lookup(probe, with_tier=True)
        assert lens.tolist() == ref.lookup(probe) and tiers.tolist() == ref.tier(probe)
    assert outcomes["ok"] > 50


@pytest.mark.parametrize("seed", [5, 6])
def test_invariants_on_random_traces(seed):
    """Pages are owned by at most one (user, layer) and never lost; a user
    holds exactly ceil(len / page_size) pages per layer; an eviction only
    happens when the batch would not fit otherwise and takes the least
    recently planned user outside the batch."""
    rng = np.random.default_rng(seed)
    cfg = dict(num_layers=2, num_pages=64, page_size=8, max_pages_per_user=6, max_users=6)
    ref = RefKVCache(**cfg)
    L, ps = cfg["num_layers"], cfg["page_size"]
    for ids, n in random_trace(rng, 400, 5, 16, 20):
        free_before = len(ref.free_pages)
        slots_before = len(ref.free_slots)
        cached_before = {uid: L * len(u.pages[0]) for uid, u in ref.users.items()}
        order = sorted((u.last_use, uid) for uid, u in ref.users.items() if uid not in set(ids))
        try:
            hist, slots, updates, evicted = ref.plan(ids, n)
        except (CacheFull, TooLong):
            continue
        owned = ref.owned_pages()
        pages = [p for p, _, _ in owned]
        assert len(pages) == len(set(pages))
        assert sorted(pages + ref.free_pages) == list(range(cfg["num_pages"]))
        for uid, u in ref.users.items():
            for lp in u.pages:
                assert len(lp) == -(-u.length // ps)
        # evictions take the least recently planned users outside the batch ...
        assert evicted == [uid for _, uid in order[:len(evicted)]]
        # ... and only as many as needed: one fewer would not have fitted
        need = L * sum(-(-(h + k) // ps) for h, k in zip(hist, n)) - sum(cached_before.get(i, 0) for i in ids)
        misses = sum(1 for i in ids if i not in cached_before)
        assert len(updates) == need
        if evicted:
            freed = sum(cached_before[uid] for uid in evicted[:-1])
            assert free_before + freed < need or slots_before + len(evicted) - 1 < misses
        else:
            assert free_before >= need and slots_before >= misses


@pytest.mark.parametrize("seed", [7, 8])
def test_host_tier_invariants_on_random_traces(seed):
    """Host pages are held by at most one (user, layer) and never lost; no
    user is in both tiers; an offloaded user's host pages receive exactly its
    GPU pages; an onboarded user's first pages come from exactly its host
    pages, in position order; a host hit keeps its history."""
    rng = np.random.default_rng(seed)
    cfg = dict(num_layers=2, num_pages=48, page_size=8, max_pages_per_user=5, max_users=5, host_pages=30)
    ref = RefKVCache(**cfg)
    for ids, n in random_trace(rng, 400, 4, 14, 20):
        gpu_before = {uid: [list(p) for p in u.pages] for uid, u in ref.users.items()}
        host_before = {uid: ([list(p) for p in e.pages], e.length) for uid, e in ref.host.items()}
        try:
            hist, slots, updates, evicted = ref.plan(ids, n)
        except (CacheFull, TooLong):
            continue
        assert not (set(ref.users) & set(ref.host))
        hp = [p for e in ref.host.values() for lp in e.pages for p in lp]
        assert len(hp) == len(set(hp)) and sorted(hp + ref.host_free) == list(range(cfg["host_pages"]))
        offl = [c for c in ref.last_copies if c[0] == 0]
        onb = [c for c in ref.last_copies if c[0] == 1]
        assert ref.last_copies == offl + onb
        for uid in evicted:
            if uid in ref.host and uid not in host_before:
                got = {(g, h) for _, g, h in offl if h in {p for lp in ref.host[uid].pages for p in lp}}
                want = {(g, h) for gl, hl in zip(gpu_before[uid], ref.host[uid].pages) for g, h in zip(gl, hl)}
                assert got == want
        for b, uid in enumerate(ids):
            if uid in host_before and uid not in gpu_before:
                assert hist[b] == host_before[uid][1]
                u = ref.users[uid]
                want = [(1, u.pages[l][i], host_before[uid][0][l][i])
                        for l in range(cfg["num_layers"]) for i in range(len(host_before[uid][0][l]))]
                assert sorted(c for c in onb if c in set(want)) == sorted(want)


def test_lookup_does_not_touch_recency():
    kv = KVCache(num_layers=1, num_pages=4, page_size=4, max_pages_per_user=2, max_users=2)
    kv.plan([1], [4])
    kv.plan([2], [4])
    kv.lookup([1, 2, 1])             # would make 1 the most recent if it counted
    p = kv.plan([3], [4])
    assert p.evicted == [1]


def test_explicit_evict_and_reuse():
    kv = KVCache(num_layers=2, num_pages=8, page_size=4, max_pages_per_user=2, max_users=3)
    kv.plan([7, 8], [8, 4])
    assert kv.stats() == (8 - 2 * 2 - 2 * 1, 2)
    assert kv.evict(7) is True
    assert kv.evict(7) is False
    assert kv.stats() == (8 - 2, 1)
    assert kv.lookup([7, 8]).tolist() == [-1, 4]
    p = kv.plan([9], [8])
    assert p.hist_len.tolist() == [0] and p.evicted == []


def test_bad_arguments_rejected():
    with pytest.raises(KVCacheError):
        KVCache(num_layers=0, num_pages=4, page_size=4, max_pages_per_user=2, max_users=2)
    with pytest.raises(KVCacheError):
        KVCache(num_layers=1, num_pages=4, page_size=3, max_pages_per_user=2, max_users=2)
    kv = KVCache(num_layers=1, num_pages=4, page_size=4, max_pages_per_user=2, max_users=2)
    with pytest.raises(KVCacheError) as ei:
        kv.plan([1], [-1])
    assert ei.value.code == -1
    assert kv.stats() == (4, 0)


# ---- trim: candidates scored once are dropped from the cached history ----

TRIM_CFG = dict(num_layers=2, num_pages=8, page_size=2, max_pages_per_user=4, max_users=2)


def _trim_trace(cache):
    """Worked by hand from the rule (free pages start as a stack that pops
    0, 1, 2, ...):
      plan A(+5): 3 pages per layer: layer 0 takes 0, 1, 2, layer 1 takes
        3, 4, 5; slot 0;
      trim A by 2: length 3 keeps ceil(3/2) = 2 pages per layer; page index 2
        of layer 0 (page 2), then of layer 1 (page 5) are pushed, so 5 is on
        top, then 2;
      plan A(+2): history 3, length 5 needs one more page per layer: layer 0
        pops 5, layer 1 pops 2; pages 7 and 6 stay free."""
    p1 = cache.plan([11], [5])
    cache.trim([11], [2])
    mid = cache.lookup([11])
    p2 = cache.plan([11], [2])
    return p1, mid, p2


def _updates(p):
    return [tuple(int(v) for v in u) for u in (p.updates.tolist() if hasattr(p, "updates") else p[2])]


def test_trim_hand_worked_trace_model_and_library():
    want1 = [(0, 0, 0, 0), (0, 0, 1, 1), (0, 0, 2, 2), (0, 1, 0, 3), (0, 1, 1, 4), (0, 1, 2, 5)]
    want2 = [(0, 0, 2, 5), (0, 1, 2, 2)]
    ref = RefKVCache(**TRIM_CFG)
    h1 = ref.plan([11], [5])
    ref.trim([11], [2])
    assert ref.lookup([11]) == [3]
    h2 = ref.plan([11], [2])
    assert [tuple(u) for u in h1[2]] == want1 and [tuple(u) for u in h2[2]] == want2
    assert h2[0] == [3] and sorted(ref.free_pages) == [6, 7]
    kv = KVCache(**TRIM_CFG)
    p1, mid, p2 = _trim_trace(kv)
    assert _updates(p1) == want1 and mid.tolist() == [3]
    assert _updates(p2) == want2 and p2.hist_len.tolist() == [3]
    assert kv.stats() == (2, 1)


def test_trim_rejects_bad_arguments_and_changes_nothing():
    kv = KVCache(**TRIM_CFG)
    kv.plan([11, 12], [3, 2])
    before = (kv.stats(), kv.lookup([11, 12]).tolist())
    for ids, k in [([13], [0]), ([11, 11], [1, 1]), ([11], [4]), ([11], [-1]), ([11, 13], [1, 0])]:
        with pytest.raises(KVCacheError) as ei:
            kv.trim(ids, k)
        assert ei.value.code == -1
        assert (kv.stats(), kv.lookup([11, 12]).tolist()) == before
    kv.trim([11, 12], [3, 0])                  # to zero length: the user stays, pageless
    assert kv.lookup([11, 12]).tolist() == [0, 2] and kv.stats() == (8 - 2, 2)


@pytest.mark.parametrize("seed,host", [(20, False), (21, False), (22, True), (23, True)])
def test_library_matches_reference_model_with_trims(seed, host):
    """Random plans, each followed by a trim of a random part of what it
    added (as a serving step drops its candidates), library against model."""
    rng = np.random.default_rng(seed)
    cfg = dict(num_layers=int(rng.integers(1, 4)), num_pages=int(rng.integers(20, 120)),
               page_size=int(2 ** rng.integers(2, 5)), max_pages_per_user=int(rng.integers(2, 10)),
               max_users=int(rng.integers(2, 10)))
    if host:
        cfg["host_pages"] = int(rng.integers(4, 200))
    ref, kv = RefKVCache(**cfg), KVCache(**cfg)
    ok = 0
    for ids, n in random_trace(rng, 250, 5, 20, 3 * cfg["page_size"]):
        try:
            want = ref.plan(ids, n)
        except (CacheFull, TooLong):
            with pytest.raises(KVCacheError):
                kv.plan(ids, n)
            continue
        got = kv.plan(ids, n)
        assert _updates(got) == [tuple(u) for u in want[2]] and got.evicted == want[3]
        drop = [int(rng.integers(0, k + 1)) for k in n]
        ref.trim(ids, drop)
        kv.trim(ids, drop)
        ok += 1
        assert kv.stats(host=True) == (len(ref.free_pages), len(ref.users), len(ref.host_free), len(ref.host))
        assert kv.lookup(ids).tolist() == ref.lookup(ids)
        owned = ref.owned_pages()
        assert sorted([p for p, _, _ in owned] + ref.free_pages) == list(range(cfg["num_pages"]))
        for u in ref.users.values():
            assert all(len(lp) == -(-u.length // cfg["page_size"]) for lp in u.pages)
    assert ok > 50


# ---- pins: users of batches still in flight are kept ----

PIN_CFG = dict(num_layers=1, num_pages=4, page_size=4, max_pages_per_user=4, max_users=4)


def test_pins_hand_worked_model_and_library():
    """Pool of 4 pages.  User 1 takes 2 pages and is pinned (its batch in
    flight): a batch of user 2 needing 3 pages cannot evict it and fails;
    plan, evict and trim naming user 1 fail; after one of two pins is undone
    it still holds; after the second, user 2's batch evicts it."""
    ref, kv = RefKVCache(**PIN_CFG), KVCache(**PIN_CFG)
    for c in (ref, kv):
        c.plan([1], [8])
        c.pin([1])
        c.pin([1])
    with pytest.raises(CacheFull):
        ref.plan([2], [12])
    with pytest.raises(KVCacheError) as ei:
        kv.plan([2], [12])
    assert ei.value.code == ERR["full"]
    assert kv.stats() == (2, 1) and len(ref.free_pages) == 2
    with pytest.raises(Pinned):
        ref.plan([1, 3], [1, 1])
    with pytest.raises(Pinned):
        ref.evict(1)
    with pytest.raises(Pinned):
        ref.trim([1], [1])
    for call in (lambda: kv.plan([3, 1], [1, 1]), lambda: kv.evict(1), lambda: kv.trim([1], [1])):
        with pytest.raises(KVCacheError) as ei:
            call()
        assert ei.value.code == ERR["pinned"]
    assert kv.stats() == (2, 1) and kv.lookup([1, 3]).tolist() == [8, -1]
    # a batch that fits beside the pinned user goes through
    assert kv.plan([3], [8]).evicted == [] and ref.plan([3], [8])[3] == []
    for c in (ref, kv):
        c.unpin([1])                              # one pin left
    with pytest.raises(CacheFull):
        ref.plan([2], [12])
    with pytest.raises(KVCacheError):
        kv.plan([2], [12])
    for c in (ref, kv):
        c.unpin([1])
    want = ref.plan([2], [12])
    got = kv.plan([2], [12])
    assert want[3] == got.evicted == [1, 3]       # least recently planned first
    assert [tuple(u) for u in got.updates.tolist()] == [tuple(u) for u in want[2]]


def test_pin_rejects_bad_arguments_and_changes_nothing():
    kv = KVCache(**PIN_CFG)
    kv.plan([1, 2], [4, 4])
    for ids, pin in (([5], True), ([1, 1], True), ([1], False), ([1, 5], True)):
        with pytest.raises(KVCacheError) as ei:
            (kv.pin if pin else kv.unpin)(ids)
        assert ei.value.code == ERR["invalid"]
    assert kv.evict(1) is True                    # nothing was pinned


@pytest.mark.parametrize("seed,host", [(20, False), (21, False), (22, True), (23, True)])
def test_library_matches_reference_model_with_batches_in_flight(seed, host):
    """Random plans with up to two earlier batches kept in flight (pinned,
    then unpinned oldest first); batches avoid the users in flight, as a
    server must.  Plans, evictions and failures agree exactly."""
    rng = np.random.default_rng(seed)
    cfg = dict(num_layers=int(rng.integers(1, 3)), num_pages=int(rng.integers(24, 60)),
               page_size=int(2 ** rng.integers(2, 4)), max_pages_per_user=int(rng.integers(4, 12)),
               max_users=int(rng.integers(8, 14)))
    if host:
        cfg["host_pages"] = int(rng.integers(4, 100))
    ref, kv = RefKVCache(**cfg), KVCache(**cfg)
    flight = []
    evicted_beside_pins = 0
    outcomes = {"ok": 0, "full": 0, "too_long": 0}
    for ids, n in random_trace(rng, 300, 5, 24, 3 * cfg["page_size"]):
        busy = {u for b in flight for u in b}
        keep = [k for k, u in enumerate(ids) if u not in busy]
        ids, n = [ids[k] for k in keep], [n[k] for k in keep]
        if len(flight) == 2:
            done = flight.pop(0)
            ref.pin(done, pin=False)
            kv.unpin(done)
        try:
            want = ref.plan(ids, n)
        except (CacheFull, TooLong) as e:
            kind = "full" if isinstance(e, CacheFull) else "too_long"
            outcomes[kind] += 1
            with pytest.raises(KVCacheError) as ei:
                kv.plan(ids, n)
            assert ei.value.code == ERR[kind]
            continue
        outcomes["ok"] += 1
        got = kv.plan(ids, n)
        assert got.hist_len.tolist() == want[0] and got.slots.tolist() == want[1]
        assert [tuple(u) for u in got.updates.tolist()] == [tuple(u) for u in want[2]]
        assert got.evicted == want[3]
        assert not set(got.evicted) & {u for b in flight for u in b}
        evicted_beside_pins += bool(got.evicted and flight)
        assert [tuple(c) for c in got.copies[:, :3].tolist()] == [tuple(c) for c in ref.last_copies]
        assert kv.stats(host=True) == (len(ref.free_pages), len(ref.users), len(ref.host_free), len(ref.host))
        if ids and rng.random() < 0.7:
            ref.pin(ids)
            kv.pin(ids)
            flight.append(ids)
    assert outcomes["ok"] > 50 and evicted_beside_pins > 10
