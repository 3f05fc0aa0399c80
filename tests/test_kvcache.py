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

from oracle.kvcache import CacheFull, RefKVCache, TooLong
from hstu_jagged_silu_fwd_amd.kvcache import KVCache, KVCacheError

HERE = os.path.dirname(os.path.abspath(__file__))
TRACE = json.load(open(os.path.join(HERE, "golden", "kvcache_trace.json")))
ERR = {"full": -10, "too_long": -11, "invalid": -1}


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


def random_trace(rng, n_batches, max_b, n_ids, max_new):
    for _ in range(n_batches):
        B = int(rng.integers(0, max_b + 1))
        ids = rng.choice(n_ids, size=min(B, n_ids), replace=False).astype(np.int64) * 7919 + 3
        n = rng.integers(0, max_new + 1, size=ids.shape[0])
        yield ids.tolist(), n.tolist()


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_library_matches_reference_model_on_random_traces(seed):
    rng = np.random.default_rng(seed)
    cfg = dict(num_layers=int(rng.integers(1, 4)), num_pages=int(rng.integers(20, 200)),
               page_size=int(2 ** rng.integers(2, 6)), max_pages_per_user=int(rng.integers(2, 12)),
               max_users=int(rng.integers(2, 16)))
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
        assert kv.stats() == (len(ref.free_pages), len(ref.users))
        probe = list(range(3, 24 * 7919, 7919 * 3))
        assert kv.lookup(probe).tolist() == ref.lookup(probe)
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
