"""Binding of the paged KV cache manager (include/hstu_kvcache.h): lookup,
page allocation and LRU eviction on the host (with an optional pinned host
tier that evicted users are offloaded to and onboarded back from), page-table
building and page copies on the device.  Argument marshalling only: every
decision is made by libhstu.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

from . import _lib

I32, I64 = ctypes.c_int32, ctypes.c_int64
P = ctypes.c_void_p

KV_STATUS = {0: "ok", -1: "invalid argument", -10: "cache full", -11: "sequence too long",
             -12: "output capacity", -13: "HIP launch failed"}


class KVCacheError(RuntimeError):
    def __init__(self, where: str, code: int):
        super().__init__(f"{where}: {KV_STATUS.get(code, 'unknown')} ({code})")
        self.code = code


class KVUpdate(ctypes.Structure):
    _fields_ = [("slot", I32), ("layer", I32), ("page_index", I32), ("page_id", I32)]


_bound = None


def _lib_kv() -> ctypes.CDLL:
    global _bound
    lib = _lib.load()
    if _bound is lib:
        return lib
    lib.hstu_kvcache_create.restype = P
    lib.hstu_kvcache_create.argtypes = [I32, I64, I32, I32, I32, I64]
    lib.hstu_kvcache_destroy.restype = None
    lib.hstu_kvcache_destroy.argtypes = [P]
    lib.hstu_kvcache_directory_elems.restype = I64
    lib.hstu_kvcache_directory_elems.argtypes = [P]
    lib.hstu_kvcache_plan.restype = I32
    lib.hstu_kvcache_plan.argtypes = [P, I32, P, P, P, P, P, I32, ctypes.POINTER(I32), P, I32,
                                      ctypes.POINTER(I32), P, I32, ctypes.POINTER(I32)]
    lib.hstu_kvcache_lookup.restype = I32
    lib.hstu_kvcache_lookup.argtypes = [P, I32, P, P, P]
    lib.hstu_kvcache_evict.restype = I32
    lib.hstu_kvcache_evict.argtypes = [P, I64, ctypes.POINTER(I32)]
    lib.hstu_kvcache_trim.restype = I32
    lib.hstu_kvcache_trim.argtypes = [P, I32, P, P]
    lib.hstu_kvcache_pin.restype = I32
    lib.hstu_kvcache_pin.argtypes = [P, I32, P, I32]
    lib.hstu_kvcache_stats.restype = I32
    lib.hstu_kvcache_stats.argtypes = [P, ctypes.POINTER(I64), ctypes.POINTER(I32), ctypes.POINTER(I64),
                                       ctypes.POINTER(I32)]
    lib.hstu_kv_tables_build.restype = I32
    lib.hstu_kv_tables_build.argtypes = [P, I32, I32, I32, P, I32, P, I32, P, P]
    lib.hstu_kv_copy_pages.restype = I32
    lib.hstu_kv_copy_pages.argtypes = [P, P, P, P, I64, I64, I64, I64, P, I32, I32, P]
    _bound = lib
    return lib


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(P) if a.size else None


@dataclass
class Plan:
    hist_len: np.ndarray      # [B] int32: cached tokens reused (0 = miss)
    slots: np.ndarray         # [B] int32: directory slots
    updates: np.ndarray       # [n, 4] int32: (slot, layer, page index, page id)
    evicted: List[int]        # user ids evicted from the GPU by this plan
    copies: np.ndarray        # [m, 4] int32: (onboard, gpu page, host page, 0), offloads first

    @property
    def n_offload(self) -> int:
        return int(np.count_nonzero(self.copies[:, 0] == 0)) if self.copies.size else 0


class KVCache:
    """Host cache manager over a pool of num_pages pages of page_size tokens
    shared by num_layers layers (and, with host_pages > 0, a host tier of that
    many pages), plus the device page directory."""

    def __init__(self, *, num_layers: int, num_pages: int, page_size: int, max_pages_per_user: int,
                 max_users: int, host_pages: int = 0):
        self.lib = _lib_kv()
        self.L, self.P, self.ps = num_layers, num_pages, page_size
        self.maxP, self.max_users, self.PH = max_pages_per_user, max_users, host_pages
        h = self.lib.hstu_kvcache_create(num_layers, num_pages, page_size, max_pages_per_user, max_users,
                                         host_pages)
        if not h:
            raise KVCacheError("hstu_kvcache_create", -1)
        self.h = P(h)
        self._dir = None
        self._bufs = {}           # reusable plan output buffers (see _scratch)
        self._counts = (I32(0), I32(0), I32(0))
        self._pinned = None       # reused pinned host staging buffer for updates and slots
        self._staged = None       # event after the last copy out of it
        self._dstage = None       # device side of those copies
        self._cpinned = None      # the same for page copies
        self._cstaged = None
        self.host_k = self.host_v = None

    def close(self) -> None:
        if self.h:
            self.lib.hstu_kvcache_destroy(self.h)
            self.h = P(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def lookup(self, user_ids: Sequence[int], with_tier: bool = False):
        """Cached tokens per user (-1: not cached); with_tier also returns the
        tier per user (0 none, 1 GPU, 2 host)."""
        ids = np.ascontiguousarray(user_ids, dtype=np.int64)
        out = np.empty(ids.shape[0], dtype=np.int32)
        tier = np.empty(ids.shape[0], dtype=np.int32)
        rc = self.lib.hstu_kvcache_lookup(self.h, ids.shape[0], _np_ptr(ids), _np_ptr(out), _np_ptr(tier))
        if rc != 0:
            raise KVCacheError("hstu_kvcache_lookup", rc)
        return (out, tier) if with_tier else out

    def _scratch(self, name: str, rows: int, cols: int, dtype):
        """A reusable host array of at least `rows` rows and its address
        (numpy's .ctypes accessor costs tens of microseconds per call, so
        the plan's output buffers are made once and their addresses kept)."""
        a = self._bufs.get(name)
        if a is None or a[0].shape[0] < rows:
            arr = np.empty((max(rows, 1), cols) if cols else max(rows, 1), dtype=dtype)
            a = self._bufs[name] = (arr, arr.__array_interface__["data"][0])
        return a

    def plan(self, user_ids: Sequence[int], n_new: Sequence[int]) -> Plan:
        ids = np.ascontiguousarray(user_ids, dtype=np.int64)
        n = np.ascontiguousarray(n_new, dtype=np.int32)
        if ids.shape != n.shape or ids.ndim != 1:
            raise KVCacheError("plan", -1)
        B = ids.shape[0]
        # every user holds at most max_pages pages per layer: a buffer of
        # L * B * max_pages records always suffices (only the records written
        # are ever touched), so no lookup is needed to size it
        cap = self.L * B * self.maxP
        upd, upd_p = self._scratch("upd", cap, 4, np.int32)
        ev, ev_p = self._scratch("ev", self.max_users, 0, np.int64)
        ccap = 2 * self.P if self.PH > 0 else 0
        cps, cps_p = self._scratch("cps", ccap, 4, np.int32)
        hist = np.empty(B, dtype=np.int32)
        slots = np.empty(B, dtype=np.int32)
        addr = lambda a: a.__array_interface__["data"][0] if a.size else None
        nu, ne, nc = self._counts
        rc = self.lib.hstu_kvcache_plan(self.h, B, addr(ids), addr(n), addr(hist), addr(slots),
                                        upd_p, cap, ctypes.byref(nu), ev_p, self.max_users, ctypes.byref(ne),
                                        cps_p, ccap, ctypes.byref(nc))
        if rc != 0:
            raise KVCacheError("hstu_kvcache_plan", rc)
        return Plan(hist, slots, upd[:nu.value].copy(), ev[:ne.value].tolist(), cps[:nc.value].copy())

    def evict(self, user_id: int) -> bool:
        found = I32(0)
        rc = self.lib.hstu_kvcache_evict(self.h, int(user_id), ctypes.byref(found))
        if rc != 0:
            raise KVCacheError("hstu_kvcache_evict", rc)
        return bool(found.value)

    def trim(self, user_ids: Sequence[int], n_drop: Sequence[int]) -> None:
        """Shortens each user's cached length by n_drop tokens (candidates
        scored once are not kept as history); all or nothing."""
        ids = np.ascontiguousarray(user_ids, dtype=np.int64)
        k = np.ascontiguousarray(n_drop, dtype=np.int32)
        if ids.shape != k.shape or ids.ndim != 1:
            raise KVCacheError("trim", -1)
        rc = self.lib.hstu_kvcache_trim(self.h, ids.shape[0], _np_ptr(ids), _np_ptr(k))
        if rc != 0:
            raise KVCacheError("hstu_kvcache_trim", rc)

    def pin(self, user_ids: Sequence[int]) -> None:
        """Pins GPU-cached users while a planned batch of theirs is in flight
        (its layer calls still running on some stream): no plan evicts them
        or hands out their pages, and a plan, evict or trim that names one
        fails (HSTU_KV_PINNED).  All or nothing; pins count."""
        self._pin(user_ids, 1)

    def unpin(self, user_ids: Sequence[int]) -> None:
        """Undoes one pin of each user (once its batch's calls have finished)."""
        self._pin(user_ids, 0)

    def _pin(self, user_ids, pin: int) -> None:
        ids = np.ascontiguousarray(user_ids, dtype=np.int64)
        if ids.ndim != 1:
            raise KVCacheError("pin", -1)
        rc = self.lib.hstu_kvcache_pin(self.h, ids.shape[0], _np_ptr(ids), pin)
        if rc != 0:
            raise KVCacheError("hstu_kvcache_pin", rc)

    def stats(self, host: bool = False):
        """(free GPU pages, GPU-cached users), plus (free host pages, host users)
        when host is set."""
        fp, cu, fh, hu = I64(0), I32(0), I64(0), I32(0)
        rc = self.lib.hstu_kvcache_stats(self.h, ctypes.byref(fp), ctypes.byref(cu), ctypes.byref(fh),
                                         ctypes.byref(hu))
        if rc != 0:
            raise KVCacheError("hstu_kvcache_stats", rc)
        return (fp.value, cu.value, fh.value, hu.value) if host else (fp.value, cu.value)

    def host_tier(self, page_shape_k, page_shape_v, dtype):
        """The pinned host tier arrays [host_pages, *page_shape] (allocated on
        first use)."""
        import torch
        if self.host_k is None:
            self.host_k = torch.empty((self.PH, *page_shape_k), dtype=dtype, pin_memory=True)
            self.host_v = torch.empty((self.PH, *page_shape_v), dtype=dtype, pin_memory=True)
        return self.host_k, self.host_v

    def copy_pages(self, plan: Plan, k_pool, v_pool, stream=None) -> None:
        """Runs the plan's offloads, then its onboards, between the device pools
        and the pinned host tier (call before the batch's layers), on `stream`
        (default: the current stream)."""
        with _lib.stream_scope(stream):
            self._copy_pages(plan, k_pool, v_pool)

    def _copy_pages(self, plan: Plan, k_pool, v_pool) -> None:
        import torch
        m = plan.copies.shape[0]
        if m == 0:
            return
        hk, hv = self.host_tier(tuple(k_pool.shape[1:]), tuple(v_pool.shape[1:]), k_pool.dtype)
        need = 4 * m
        if self._cpinned is None or self._cpinned.numel() < need:
            # a plan reports at most 2 * num_pages copies: sized once
            self._cpinned = torch.empty(max(need, 8 * self.P, 1024), dtype=torch.int32, pin_memory=True)
        if self._cstaged is None:
            self._cstaged = torch.cuda.Event()
        self._cstaged.synchronize()
        host = self._cpinned[:need]
        host.numpy()[:] = plan.copies.reshape(-1)
        dev = host.to(device=k_pool.device, non_blocking=True)
        self._cstaged.record()
        pbk = k_pool[0].numel() * k_pool.element_size()
        pbv = v_pool[0].numel() * v_pool.element_size()
        rc = self.lib.hstu_kv_copy_pages(P(k_pool.data_ptr()), P(v_pool.data_ptr()), P(hk.data_ptr()),
                                         P(hv.data_ptr()), pbk, pbv, int(k_pool.shape[0]), self.PH,
                                         P(dev.data_ptr()), plan.n_offload, m, _lib._stream(None))
        if rc != 0:
            raise KVCacheError("hstu_kv_copy_pages", rc)

    def directory(self, device="cuda"):
        """The device page directory [max_users, L, max_pages] (allocated on
        first use; the caller keeps it with the cache)."""
        import torch
        if self._dir is None:
            n = int(self.lib.hstu_kvcache_directory_elems(self.h))
            self._dir = torch.full((n,), -1, dtype=torch.int32, device=device)
        return self._dir

    def build_tables(self, plan: Plan, device="cuda", stream=None):
        """Applies the plan's updates to the device directory and returns the
        batch's page tables [L, B, max_pages] int32 on the device, all on
        `stream` (default: the current stream)."""
        with _lib.stream_scope(stream):
            return self._build_tables(plan, device)

    def _build_tables(self, plan: Plan, device="cuda"):
        import torch
        d = self.directory(device)
        B = plan.slots.shape[0]
        nu = plan.updates.shape[0]
        # updates and slots travel in one copy from a pinned staging buffer,
        # sized once for the most records a batch of B users can produce
        # (pinned allocations are slow: growing it batch by batch cost more
        # than the whole build)
        need = 4 * nu + B
        if self._pinned is None or self._pinned.numel() < need:
            worst = 4 * self.L * B * self.maxP + B
            self._pinned = torch.empty(max(need, worst, 1024), dtype=torch.int32, pin_memory=True)
        if self._staged is None:
            self._staged = torch.cuda.Event()       # one event, re-recorded (creating one per call
                                                    # now and then costs tens of microseconds)
        self._staged.synchronize()                  # the previous build is done with both staging
                                                    # buffers (on whichever stream it ran)
        host = self._pinned[:need]
        host[:4 * nu].numpy()[:] = plan.updates.reshape(-1)
        host[4 * nu:].numpy()[:] = plan.slots
        # ... into a device buffer of the same size, kept (a fresh one of the
        # batch's size each time sends the caching allocator to the driver
        # now and then for a new segment)
        if self._dstage is None or self._dstage.numel() < self._pinned.numel():
            self._dstage = torch.empty(self._pinned.numel(), dtype=torch.int32, device=d.device)
        dev = self._dstage[:need]
        dev.copy_(host, non_blocking=True)
        upd = dev[:4 * nu]
        slots = dev[4 * nu:]
        tables = torch.empty((self.L, B, self.maxP), dtype=torch.int32, device=d.device)
        st = _lib._stream(None)
        rc = self.lib.hstu_kv_tables_build(P(d.data_ptr()), self.L, self.max_users, self.maxP,
                                           P(upd.data_ptr()) if nu else None, int(nu),
                                           P(slots.data_ptr()) if B else None, B,
                                           P(tables.data_ptr()) if B else None, st)
        if rc != 0:
            raise KVCacheError("hstu_kv_tables_build", rc)
        self._staged.record()
        return tables
