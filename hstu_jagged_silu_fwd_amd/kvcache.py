"""Binding of the paged KV cache manager (include/hstu_kvcache.h): lookup,
page allocation and LRU eviction on the host, page-table building on the
device.  Argument marshalling only: every decision is made by libhstu.
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
    lib.hstu_kvcache_create.argtypes = [I32, I64, I32, I32, I32]
    lib.hstu_kvcache_destroy.restype = None
    lib.hstu_kvcache_destroy.argtypes = [P]
    lib.hstu_kvcache_directory_elems.restype = I64
    lib.hstu_kvcache_directory_elems.argtypes = [P]
    lib.hstu_kvcache_plan.restype = I32
    lib.hstu_kvcache_plan.argtypes = [P, I32, P, P, P, P, P, I32, ctypes.POINTER(I32), P, I32,
                                      ctypes.POINTER(I32)]
    lib.hstu_kvcache_lookup.restype = I32
    lib.hstu_kvcache_lookup.argtypes = [P, I32, P, P]
    lib.hstu_kvcache_evict.restype = I32
    lib.hstu_kvcache_evict.argtypes = [P, I64, ctypes.POINTER(I32)]
    lib.hstu_kvcache_stats.restype = I32
    lib.hstu_kvcache_stats.argtypes = [P, ctypes.POINTER(I64), ctypes.POINTER(I32)]
    lib.hstu_kv_tables_build.restype = I32
    lib.hstu_kv_tables_build.argtypes = [P, I32, I32, I32, P, I32, P, I32, P, P]
    _bound = lib
    return lib


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(P) if a.size else None


@dataclass
class Plan:
    hist_len: np.ndarray      # [B] int32: cached tokens reused (0 = miss)
    slots: np.ndarray         # [B] int32: directory slots
    updates: np.ndarray       # [n, 4] int32: (slot, layer, page index, page id)
    evicted: List[int]        # user ids evicted by this plan


class KVCache:
    """Host cache manager over a pool of num_pages pages of page_size tokens
    shared by num_layers layers, plus the device page directory."""

    def __init__(self, *, num_layers: int, num_pages: int, page_size: int, max_pages_per_user: int,
                 max_users: int):
        self.lib = _lib_kv()
        self.L, self.P, self.ps = num_layers, num_pages, page_size
        self.maxP, self.max_users = max_pages_per_user, max_users
        h = self.lib.hstu_kvcache_create(num_layers, num_pages, page_size, max_pages_per_user, max_users)
        if not h:
            raise KVCacheError("hstu_kvcache_create", -1)
        self.h = P(h)
        self._dir = None
        self._pinned = None       # reused pinned host staging buffer for updates and slots

    def close(self) -> None:
        if self.h:
            self.lib.hstu_kvcache_destroy(self.h)
            self.h = P(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def lookup(self, user_ids: Sequence[int]) -> np.ndarray:
        ids = np.ascontiguousarray(user_ids, dtype=np.int64)
        out = np.empty(ids.shape[0], dtype=np.int32)
        rc = self.lib.hstu_kvcache_lookup(self.h, ids.shape[0], _np_ptr(ids), _np_ptr(out))
        if rc != 0:
            raise KVCacheError("hstu_kvcache_lookup", rc)
        return out

    def plan(self, user_ids: Sequence[int], n_new: Sequence[int]) -> Plan:
        ids = np.ascontiguousarray(user_ids, dtype=np.int64)
        n = np.ascontiguousarray(n_new, dtype=np.int32)
        if ids.shape != n.shape or ids.ndim != 1:
            raise KVCacheError("plan", -1)
        B = ids.shape[0]
        cached = np.maximum(self.lookup(ids), 0).astype(np.int64)
        cap = int(self.L * np.sum((cached + np.maximum(n, 0) + self.ps - 1) // self.ps))
        upd = np.empty((max(cap, 1), 4), dtype=np.int32)
        ev = np.empty(max(self.max_users, 1), dtype=np.int64)
        hist = np.empty(B, dtype=np.int32)
        slots = np.empty(B, dtype=np.int32)
        nu, ne = I32(0), I32(0)
        rc = self.lib.hstu_kvcache_plan(self.h, B, _np_ptr(ids), _np_ptr(n), _np_ptr(hist), _np_ptr(slots),
                                        upd.ctypes.data_as(P), cap, ctypes.byref(nu), ev.ctypes.data_as(P),
                                        ev.shape[0], ctypes.byref(ne))
        if rc != 0:
            raise KVCacheError("hstu_kvcache_plan", rc)
        return Plan(hist, slots, upd[:nu.value].copy(), ev[:ne.value].tolist())

    def evict(self, user_id: int) -> bool:
        found = I32(0)
        rc = self.lib.hstu_kvcache_evict(self.h, int(user_id), ctypes.byref(found))
        if rc != 0:
            raise KVCacheError("hstu_kvcache_evict", rc)
        return bool(found.value)

    def stats(self):
        fp, cu = I64(0), I32(0)
        rc = self.lib.hstu_kvcache_stats(self.h, ctypes.byref(fp), ctypes.byref(cu))
        if rc != 0:
            raise KVCacheError("hstu_kvcache_stats", rc)
        return fp.value, cu.value

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
        batch's page tables [L, B, max_pages] int32 on the device."""
        import torch
        d = self.directory(device)
        B = plan.slots.shape[0]
        nu = plan.updates.shape[0]
        # updates and slots travel in one copy from a pinned staging buffer
        need = 4 * nu + B
        if self._pinned is None or self._pinned.numel() < need:
            self._pinned = torch.empty(max(need, 1024) * 2, dtype=torch.int32, pin_memory=True)
            self._staged = None
        if getattr(self, "_staged", None) is not None:
            self._staged.synchronize()              # the previous copy out of the buffer is done
        host = self._pinned[:need]
        host[:4 * nu].numpy()[:] = plan.updates.reshape(-1)
        host[4 * nu:].numpy()[:] = plan.slots
        dev = host.to(device=d.device, non_blocking=True)
        self._staged = torch.cuda.Event()
        self._staged.record()
        upd = dev[:4 * nu]
        slots = dev[4 * nu:]
        tables = torch.empty((self.L, B, self.maxP), dtype=torch.int32, device=d.device)
        st = _lib._stream(stream)
        rc = self.lib.hstu_kv_tables_build(P(d.data_ptr()), self.L, self.max_users, self.maxP,
                                           P(upd.data_ptr()) if nu else None, int(nu),
                                           P(slots.data_ptr()) if B else None, B,
                                           P(tables.data_ptr()) if B else None, st)
        if rc != 0:
            raise KVCacheError("hstu_kv_tables_build", rc)
        return tables
