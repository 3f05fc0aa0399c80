"""Paged KV pool indexing: append (scatter) and gather.  TEST INFRASTRUCTURE.

The NVIDIA blog "Deploying an HSTU generative recommender with NVIDIA
Dynamo-Triton" (section "Why serving large sequential recommenders is hard")
describes the GPU KV cache as a paged KV data table supporting lookup,
allocate, append and evict, read directly by the HSTU attention kernel.  The
pages give no layout; the layout used here (and stated in the library header)
is:

  * user u's token at absolute position p lives in page
    page_table[u, p // page_size] at slot p % page_size;
  * K pool  [P, H, page_size, d]: element (page, h, slot, e);
  * V pool  [P, H, d, page_size]: element (page, h, e, slot).

The functions work on arrays of any dtype (e.g. uint16 bit patterns of bf16)
so that comparisons against the GPU pools are bit-exact.
"""
from __future__ import annotations

import numpy as np


def slot_of(page_table: np.ndarray, u: int, p: int, page_size: int):
    return int(page_table[u, p // page_size]), p % page_size


def append_scatter(k_pool, v_pool, k_new, v_new, new_len, hist_len,
                   page_table, page_size, H):
    """Write new rows' K/V into the pools in place.  k_new / v_new [T, D]
    hold the new rows of all users back to back; user u's row t goes to
    absolute position hist_len[u] + t."""
    D = k_new.shape[1]
    d = D // H
    r = 0
    for u in range(len(new_len)):
        c = int(hist_len[u])
        for t in range(int(new_len[u])):
            page, slot = slot_of(page_table, u, c + t, page_size)
            for h in range(H):
                k_pool[page, h, slot, :] = k_new[r, h * d:(h + 1) * d]
                v_pool[page, h, :, slot] = v_new[r, h * d:(h + 1) * d]
            r += 1


def gather_user(k_pool, v_pool, page_table, u, length, page_size, H):
    """Read positions 0..length-1 of user u back as [length, D] arrays."""
    d = k_pool.shape[3]
    D = H * d
    K = np.zeros((length, D), dtype=k_pool.dtype)
    V = np.zeros((length, D), dtype=v_pool.dtype)
    for p in range(length):
        page, slot = slot_of(page_table, u, p, page_size)
        for h in range(H):
            K[p, h * d:(h + 1) * d] = k_pool[page, h, slot, :]
            V[p, h * d:(h + 1) * d] = v_pool[page, h, :, slot]
    return K, V


def touched_slots(new_len, hist_len, page_table, page_size):
    """Set of (page, slot) pairs written by an append (for canary checks)."""
    out = set()
    for u in range(len(new_len)):
        c = int(hist_len[u])
        for t in range(int(new_len[u])):
            out.add(slot_of(page_table, u, c + t, page_size))
    return out
