"""Reference model of the paged KV cache manager.  TEST INFRASTRUCTURE.

The NVIDIA blog "Deploying an HSTU generative recommender with NVIDIA
Dynamo-Triton" (section "Why serving large sequential recommenders is hard")
says the GPU KV cache is a paged data table supporting lookup, allocation,
append and eviction, and that when GPU cache space runs short old users are
evicted under an LRU-like policy.  The pages give no further rule; the rule
modelled here is the one the library header states:

  * a plan takes a batch of distinct users with n_new tokens each; a cached
    user is a hit (history length = its cached tokens), any other a miss
    (history 0);
  * a user holds ceil(tokens / page_size) pages in every layer;
  * if the batch cannot fit even after freeing everything held by users
    outside it, the plan fails and changes nothing;
  * otherwise, while pages or slots are short, the cached user outside the
    batch whose last plan is oldest is evicted: its pages go onto the
    free-page stack layer by layer and index by index, its slot onto the
    free-slot stack;
  * users are served in batch order: a miss takes the top free slot; missing
    pages are taken off the top of the free-page stack, layer 0 first, and
    each assignment is reported as (slot, layer, page index, page id);
  * every batch user's last-use time becomes the clock value of its place in
    the batch (the last one most recent), and its cached length history +
    n_new.

With a host tier of host_pages pages (the blog's host storage tier, same
section, with onboard and offload):

  * a user cached on the host is a hit too; it needs all its GPU pages and a
    slot again, and the first ceil(len / page_size) pages of each layer are
    onboard copies (host page -> GPU page) of its host pages, which go back
    onto the host free stack once the whole batch has its pages;
  * an evicted user is offloaded when its pages fit the tier: host users that
    are neither in the batch nor offloaded by this plan are dropped, oldest
    host entry first, until the free host pages suffice (a user with more
    pages than the whole tier is dropped instead); it takes host pages off the
    host free stack, layer 0 first, and each page is an offload copy (GPU
    page -> host page); it becomes the newest host entry;
  * every offload is listed before every onboard.

Trim (candidate tokens scored once are not history): a GPU-cached user's
cached length shrinks by a given count; the pages past ceil(new length /
page_size) go onto the free-page stack layer by layer and index by index
(as in an eviction); recency is unchanged.

Pins (a reading for batches in flight, i.e. layer calls of earlier plans still
running while the next batch is planned; the pages give no rule for it): a
pinned GPU-cached user is never evicted and counts as neither free nor
evictable when a plan checks whether its batch fits; a plan, an explicit
evict or a trim that names a pinned user fails and changes nothing; pins
count, and unpinning an unpinned user is an error.

This model keeps last-use / entry times and picks victims by minimum time;
the library keeps linked recency lists.  The two agree exactly on every
output, which the tests check on random traces.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Sequence, Tuple


class CacheFull(Exception):
    pass


class TooLong(Exception):
    pass


class Pinned(Exception):
    pass


@dataclass
class _User:
    slot: int
    length: int
    pages: List[List[int]]      # per layer, page ids in position order
    last_use: int


@dataclass
class _HostUser:
    length: int
    pages: List[List[int]]      # per layer, host page ids in position order
    entered: int


@dataclass
class RefKVCache:
    num_layers: int
    num_pages: int
    page_size: int
    max_pages_per_user: int
    max_users: int
    host_pages: int = 0
    users: Dict[int, _User] = field(default_factory=dict)
    free_pages: List[int] = field(default_factory=list)    # top = end of the list
    free_slots: List[int] = field(default_factory=list)
    clock: int = 0
    host: Dict[int, _HostUser] = field(default_factory=dict)
    host_free: List[int] = field(default_factory=list)
    host_clock: int = 0
    pins: Dict[int, int] = field(default_factory=dict)     # user id -> pin count (> 0)

    def __post_init__(self):
        self.free_pages = list(range(self.num_pages - 1, -1, -1))
        self.free_slots = list(range(self.max_users - 1, -1, -1))
        self.host_free = list(range(self.host_pages - 1, -1, -1))

    def _pages_for(self, tokens: int) -> int:
        return -(-tokens // self.page_size)

    def lookup(self, ids: Sequence[int]) -> List[int]:
        return [self.users[i].length if i in self.users else
                (self.host[i].length if i in self.host else -1) for i in ids]

    def tier(self, ids: Sequence[int]) -> List[int]:
        return [1 if i in self.users else (2 if i in self.host else 0) for i in ids]

    def _evict(self, uid: int) -> None:
        u = self.users.pop(uid)
        for layer_pages in u.pages:
            for p in layer_pages:
                self.free_pages.append(p)
        self.free_slots.append(u.slot)

    def _drop_host(self, uid: int) -> None:
        for layer_pages in self.host.pop(uid).pages:
            for p in layer_pages:
                self.host_free.append(p)

    def pin(self, ids: Sequence[int], pin: bool = True) -> None:
        """Pins (or unpins) distinct GPU-cached users; all or nothing
        (ValueError)."""
        ids = list(ids)
        if len(set(ids)) != len(ids) or any(i not in self.users for i in ids) or \
                (not pin and any(self.pins.get(i, 0) == 0 for i in ids)):
            raise ValueError("bad pin")
        for i in ids:
            n = self.pins.get(i, 0) + (1 if pin else -1)
            if n:
                self.pins[i] = n
            else:
                del self.pins[i]

    def unpin(self, ids: Sequence[int]) -> None:
        self.pin(ids, pin=False)

    def evict(self, uid: int) -> bool:
        if uid in self.pins:
            raise Pinned(uid)
        if uid in self.users:
            self._evict(uid)
            return True
        if uid in self.host:
            self._drop_host(uid)
            return True
        return False

    def plan(self, ids: Sequence[int], n_new: Sequence[int]):
        """Returns (hist_len, slots, updates, evicted) or raises ValueError,
        CacheFull or TooLong (state unchanged)."""
        ids, n_new = list(ids), list(n_new)
        if len(set(ids)) != len(ids) or any(n < 0 for n in n_new):
            raise ValueError("duplicate user or negative count")
        hist = [self.users[i].length if i in self.users else
                (self.host[i].length if i in self.host else 0) for i in ids]
        need = []
        for i, h, n in zip(ids, hist, n_new):
            if i in self.pins:
                raise Pinned(i)
            if h + n > self.max_pages_per_user * self.page_size:
                raise TooLong(i)
            held = len(self.users[i].pages[0]) if i in self.users else 0
            need.append(self._pages_for(h + n) - held)
        need_pages = self.num_layers * sum(need)
        misses = sum(1 for i in ids if i not in self.users)
        outside = [i for i in self.users if i not in set(ids) and i not in self.pins]
        can_free = sum(self.num_layers * len(self.users[i].pages[0]) for i in outside)
        if len(self.free_pages) + can_free < need_pages or len(self.free_slots) + len(outside) < misses:
            raise CacheFull()
        evicted, offloads, onboards, offloaded_now = [], [], [], set()
        while len(self.free_pages) < need_pages or len(self.free_slots) < misses:
            victim = min(outside, key=lambda i: self.users[i].last_use)
            outside.remove(victim)
            evicted.append(victim)
            v = self.users[victim]
            vp = self.num_layers * len(v.pages[0])
            if 0 < self.host_pages and vp <= self.host_pages:
                droppable = sorted((e.entered, uid) for uid, e in self.host.items()
                                   if uid not in set(ids) and uid not in offloaded_now)
                while len(self.host_free) < vp and droppable:
                    self._drop_host(droppable.pop(0)[1])
                if len(self.host_free) >= vp:
                    hp = [[self.host_free.pop() for _ in lp] for lp in v.pages]
                    for gl, hl in zip(v.pages, hp):
                        offloads += [(0, g, h) for g, h in zip(gl, hl)]
                    self.host_clock += 1
                    self.host[victim] = _HostUser(v.length, hp, self.host_clock)
                    offloaded_now.add(victim)
            self._evict(victim)
        slots, updates, onboarded = [], [], []
        for i, h, n, k in zip(ids, hist, n_new, need):
            back = None
            if i not in self.users:
                back = self.host.get(i)
                self.users[i] = _User(self.free_slots.pop(), 0,
                                      [[] for _ in range(self.num_layers)], 0)
            u = self.users[i]
            for layer in range(self.num_layers):
                for _ in range(k):
                    p = self.free_pages.pop()
                    idx = len(u.pages[layer])
                    updates.append((u.slot, layer, idx, p))
                    u.pages[layer].append(p)
                    if back is not None and idx < len(back.pages[layer]):
                        onboards.append((1, p, back.pages[layer][idx]))
            if back is not None:
                onboarded.append(i)
            u.length = h + n
            slots.append(u.slot)
        for i in onboarded:
            self._drop_host(i)
        for i in ids:
            self.clock += 1
            self.users[i].last_use = self.clock
        self.last_copies = offloads + onboards
        return hist, slots, updates, evicted

    def trim(self, ids: Sequence[int], drop: Sequence[int]) -> None:
        """Shortens each user's cached length by drop tokens (all users must
        be GPU-cached, distinct, with drop in [0, length]; else ValueError and
        no change)."""
        ids, drop = list(ids), list(drop)
        if len(set(ids)) != len(ids) or any(i not in self.users for i in ids) or \
                any(k < 0 or k > self.users[i].length for i, k in zip(ids, drop)):
            raise ValueError("bad trim")
        if any(i in self.pins for i in ids):
            raise Pinned(ids)
        for i, k in zip(ids, drop):
            u = self.users[i]
            u.length -= k
            keep = self._pages_for(u.length)
            for layer_pages in u.pages:
                for p in layer_pages[keep:]:
                    self.free_pages.append(p)
                del layer_pages[keep:]

    def page_table(self, uid: int, layer: int) -> List[int]:
        return list(self.users[uid].pages[layer])

    def owned_pages(self) -> List[Tuple[int, int, int]]:
        """(page, user, layer) for every held page."""
        return [(p, uid, l) for uid, u in self.users.items() for l, ps in enumerate(u.pages) for p in ps]
