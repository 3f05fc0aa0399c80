#!/usr/bin/env python3
"""Benchmark: new-token throughput of a 3-layer bf16 HSTU stack over a 100%-hit
paged KV cache at batch 8, on one MI355X.

Workload (synthetic, seeded): 8 users per step, cached history U{256..4096}
tokens and U{16..256} new tokens per user, hidden 512, 4 heads, head dim 128,
32-token pages scattered over a 2^16-page pool, 128 log-buckets of relative
position, scale 1/4096.  A step runs the three layers over one batch; the new
K/V of every layer is appended into the pool by the projection kernel.  To keep
the KV stream honest against the 256 MB Infinity Cache, steps rotate over
`--instances` independent batches (different users and pages) whose KV
working set together exceeds that cache.

Prints one JSON line with the throughput (wall clock over K steps, each one
hstu_stack_fwd call that prepares the batch metadata once and runs the three
layers' kernels, synchronised on both sides), the attention kernel's roofline
position (HBM-bound: algorithmic bytes / its mean duration, from start/stop
events that the runtime stamps on each attention kernel's execution in a
second pass over the same steps) and a CPU baseline (the fp64 oracle on a
bounded sample of the same workload).  The same line carries records of the
other configurations through the same path: the 8-layer long-history hit
(`long_history`, HBM roofline), the batch-8 full recompute and the 64-user
serving mix (`full_recompute`, `serving_mix`, MFMA roofline), with the
cached-against-recomputed ratios and the batch-invariant mode's cost.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HSTU layer new-tokens/sec at batch 8 (paged KV hit); % bf16 MFMA peak, HBM GB/s"
WORKLOAD = "3layer-bf16-b8-paged-kv-hit"    # workloads.B8_KV_HIT
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
EPS = 1e-6


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--instances", type=int, default=6)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=WORKLOAD,
                    help="time another configuration of the workload table through the same path (one instance; "
                         "the JSON line then carries no CPU baseline)")
    ap.add_argument("--no-events", action="store_true", help="skip the per-kernel event pass (no roofline or stage split)")
    ap.add_argument("--no-extras", action="store_true",
                    help="headline workload only: no 8-layer long-history record and no cached-vs-recompute ratios")
    ap.add_argument("--kvcache", action="store_true",
                    help="measure the KV cache manager (plan on the host, page tables on the device) "
                         "on a serving stream instead of the layer")
    ap.add_argument("--kvhost", action="store_true",
                    help="measure the host tier: page-copy bandwidth and a user's onboard time "
                         "against recomputing its history")
    ap.add_argument("--rank", action="store_true",
                    help="ranking requests shaped like the pages' workload (8,198 cached context+history "
                         "tokens, 100 candidates, batch 8, 3 and 8 layers): tokens -> preprocessing -> "
                         "layers with candidates, cached vs full recompute")
    ap.add_argument("--beam", action="store_true",
                    help="Semantic-ID beam-decode attention over a shared context KV (4 requests, beam 256, "
                         "16 query / 8 KV heads of 128, bf16; contexts 1,000 and 5,000; steps 0-2)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="the projection products of the batch-8 workloads (cached hit, full recompute) through "
                         "the vendor GEMM library (torch.matmul -> hipBLASLt, plain products without the fused "
                         "epilogues) beside this library's projection stages on the same batches")
    ap.add_argument("--in-flight", type=int, default=0, metavar="S",
                    help="only the headline steps with S batches in flight (graph replays; S divides --instances), "
                         "after the same steps serialised on one stream, as one JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (for calibrating rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="turn four rocprofv3 --pmc output folders into the attention traffic record")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# HBM traffic of the attention kernel from rocprofv3 counters.  FETCH_SIZE and
# WRITE_SIZE (KiB per dispatch) are each scaled by what the same counter reads
# for a plain copy of COPY_BYTES, and kept in TRAFFIC_FILE together with a
# hash of the sources that shape the kernel's memory traffic; the record is
# only used while that hash still matches.
# ---------------------------------------------------------------------------
COPY_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "paged_silu_attn_3layer_b8_kv_hit_traffic.json")
TRAFFIC_SOURCES = ("attn.hip", "prep.hip", "common.h")


def traffic_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "hstu_jagged_silu_fwd_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def copy_calibration():
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 5}), flush=True)


def _pmc_mean(folder, counter, kernel_substr):
    import csv
    import glob
    vals = []
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel_substr} under {folder}")
    return sum(vals) / len(vals), len(vals)


def summarize_pmc(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    fetch, nf = _pmc_mean(fetch_dir, "FETCH_SIZE", "attn_kernel")
    write, nw = _pmc_mean(write_dir, "WRITE_SIZE", "attn_kernel")
    cfetch, _ = _pmc_mean(copy_fetch_dir, "FETCH_SIZE", "opy")      # the copy kernel
    cwrite, _ = _pmc_mean(copy_write_dir, "WRITE_SIZE", "opy")
    ff = COPY_BYTES / (cfetch * 1024.0)
    wf = COPY_BYTES / (cwrite * 1024.0)
    rec = dict(kernel="paged_silu_attn", sources_sha256=traffic_source_hash(),
               fetch_kib_per_launch=fetch, write_kib_per_launch=write, launches=nf,
               copy_fetch_factor=ff, copy_write_factor=wf,
               traffic_bytes_per_launch=(fetch * ff + write * wf) * 1024.0)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec), flush=True)


def load_traffic():
    """Calibrated HBM bytes per attention launch, or None when the record is
    missing or was taken on other kernel sources."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != traffic_source_hash():
        return None
    return rec["traffic_bytes_per_launch"]


class Bench:
    def __init__(self, args, wl=None):
        """The stack of workload args.workload (the headline workload with
        args.instances independent batches, others with one), or of the
        given workload `wl` (one batch of all its users)."""
        import torch
        import hstu_jagged_silu_fwd_amd as hs
        from hstu_jagged_silu_fwd_amd import _lib
        from workloads import CONFIGS, make_workload

        self.torch, self.hs, self._lib = torch, hs, _lib
        self.lib = hs.load()
        self.hip = _lib.hip_runtime()
        if wl is None:
            name = args.workload
            self.R = args.instances if name == WORKLOAD or getattr(args, "any_instances", False) else 1
            B = CONFIGS[name]["B"]
            wl = make_workload(name, seed=args.seed, B=B * self.R)
        else:
            self.R = 1
            B = wl.B
        self.B = B
        self.wl = wl
        self.L, self.D, self.H, self.d = wl.layers, wl.D, wl.H, wl.d
        dev = torch.device("cuda")
        bf = torch.bfloat16 if wl.dtype == "bf16" else torch.float32      # the workload's element type
        has_ts = wl.ts_buckets > 0
        assert not has_ts or self.R == 1, "timestamps: one instance"
        self.k_pool = torch.empty((wl.num_pool_pages, wl.H, wl.page_size, wl.d), dtype=bf, device=dev)
        self.v_pool = torch.empty((wl.num_pool_pages, wl.H, wl.d, wl.page_size), dtype=bf, device=dev)
        common = dict(num_heads=wl.H, head_dim=wl.d, page_size=wl.page_size,
                      max_pages_per_user=wl.max_pages, num_pool_pages=wl.num_pool_pages,
                      pos_buckets=wl.pos_buckets, pos_mbits=wl.pos_mbits,
                      attn_scale=wl.attn_scale, norm_eps=EPS, dtype=wl.dtype,
                      ts_buckets=wl.ts_buckets, ts_mbits=wl.ts_mbits)
        self.common = common
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.layers = []
        hoff = np.concatenate([[0], np.cumsum(wl.hist_len.astype(np.int64))]).astype(np.int32)
        for l in range(self.L):
            li = wl.layer(l)
            lay = dict(w1t=torch.from_numpy(li.w1t).to(dev, bf), w2t=torch.from_numpy(li.w2t).to(dev, bf),
                       pos_bias=torch.from_numpy(li.pos_bias).to(dev),
                       ts_bias=torch.from_numpy(li.ts_bias).to(dev) if has_ts else None,
                       pt_all=torch.from_numpy(li.page_table).to(dev))
            # history of all users of all instances, positions 0..hist-1
            k = torch.from_numpy(np.concatenate(li.hist_k)).to(dev, bf)
            v = torch.from_numpy(np.concatenate(li.hist_v)).to(dev, bf)
            d_app = hs.make_desc(num_users=wl.B, total_new=int(hoff[-1]), **common)
            hs.kv_pages_append(d_app, k, v, torch.from_numpy(hoff).to(dev),
                               torch.zeros(wl.B, dtype=torch.int32, device=dev), lay["pt_all"],
                               self.k_pool, self.v_pool, status)
            assert hs.read_device_status(status) == 0
            del k, v
            self.layers.append(lay)
        # per-instance buffers and prebuilt argument lists
        self.inst = []
        ws_bytes = 0
        for i in range(self.R):
            us = list(range(B * i, B * (i + 1)))
            off = wl.new_offsets
            rows = slice(int(off[us[0]]), int(off[us[-1] + 1]))
            T = rows.stop - rows.start
            newl = wl.new_len[us]
            hist = wl.hist_len[us]
            io = dict(T=T, users=us, new_len=newl, hist=hist,
                      off=torch.from_numpy(np.concatenate([[0], np.cumsum(newl)]).astype(np.int32)).to(dev),
                      hist_t=torch.from_numpy(hist.astype(np.int32)).to(dev),
                      x=torch.from_numpy(wl.x0[rows]).to(dev, bf),
                      ys=[torch.empty((T, self.D), dtype=bf, device=dev) for _ in range(self.L)],
                      pts=[lay["pt_all"][B * i:B * (i + 1)].contiguous() for lay in self.layers],
                      ts=torch.from_numpy(wl.ts_flat()).to(dev) if has_ts else None,
                      tso=torch.from_numpy(wl.ts_offsets()).to(dev) if has_ts else None,
                      desc=hs.make_desc(num_users=B, total_new=T, **common))
            inv = hs.make_desc(num_users=B, total_new=T, batch_invariant=True, **common)
            ws_bytes = max(ws_bytes, hs.workspace_size(io["desc"]), _lib.stack_workspace_size(io["desc"], self.L),
                           _lib.stack_workspace_size(inv, self.L))   # room for the batch-invariant mode too
            self.inst.append(io)
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream().cuda_stream
        P = ctypes.c_void_p
        for io in self.inst:
            args = []
            for l in range(self.L):
                lay = self.layers[l]
                x = io["x"] if l == 0 else io["ys"][l - 1]
                args.append((ctypes.byref(io["desc"]), P(x.data_ptr()), P(io["off"].data_ptr()),
                             P(io["hist_t"].data_ptr()), P(io["pts"][l].data_ptr()),
                             P(self.k_pool.data_ptr()), P(self.v_pool.data_ptr()),
                             P(lay["w1t"].data_ptr()), P(lay["w2t"].data_ptr()),
                             P(lay["pos_bias"].data_ptr()),
                             P(lay["ts_bias"].data_ptr()) if has_ts else None,
                             P(io["ts"].data_ptr()) if has_ts else None,
                             P(io["tso"].data_ptr()) if has_ts else None,
                             P(io["ys"][l].data_ptr()), P(self.ws.data_ptr()),
                             ctypes.c_size_t(ws_bytes), P(self.stream)))
            io["args"] = args
            # the whole step as one hstu_stack_fwd call (metadata prepared once)
            arr = lambda ts: (P * self.L)(*[P(t.data_ptr()) for t in ts])
            io["keep"] = [arr(io["pts"]), arr([self.k_pool] * self.L), arr([self.v_pool] * self.L),
                          arr([lay["w1t"] for lay in self.layers]), arr([lay["w2t"] for lay in self.layers]),
                          arr([lay["pos_bias"] for lay in self.layers]), arr(io["ys"]),
                          arr([lay["ts_bias"] for lay in self.layers]) if has_ts else None]
            k = io["keep"]
            io["stack_args"] = (ctypes.byref(io["desc"]), self.L, P(io["x"].data_ptr()), P(io["off"].data_ptr()),
                                P(io["hist_t"].data_ptr()), None, k[0], k[1], k[2], k[3], k[4], k[5], k[7],
                                P(io["ts"].data_ptr()) if has_ts else None,
                                P(io["tso"].data_ptr()) if has_ts else None,
                                k[6], P(self.ws.data_ptr()), ctypes.c_size_t(ws_bytes), P(self.stream))
        torch.cuda.synchronize()

    def step(self, s, events=None):
        io = self.inst[s % self.R]
        if events is None:                 # the timed pass: one call for the whole stack
            rc = self.lib.hstu_stack_fwd(*io["stack_args"])
            if rc != 0:
                raise RuntimeError(f"hstu_stack_fwd failed: {rc}")
            return
        for l in range(self.L):            # the event pass: layer by layer, each stage bracketed
            rc = self.lib.hstu_layer_fwd_timed(*io["args"][l], events[l])
            if rc != 0:
                raise RuntimeError(f"hstu_layer_fwd_timed failed: {rc}")

    def make_events(self, steps):
        hip = self.hip
        hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        n = 2 * self._lib.NUM_STAGES
        evs = []
        for _ in range(steps):
            per_layer = []
            for _ in range(self.L):
                arr = (ctypes.c_void_p * n)()
                for j in range(n):
                    e = ctypes.c_void_p()
                    assert hip.hipEventCreate(ctypes.byref(e)) == 0
                    arr[j] = e
                per_layer.append(arr)
            evs.append(per_layer)
        return evs

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float(0)
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        assert rc == 0, rc
        return ms.value

    def attn_work(self, io):
        """Work of one attention launch on instance io: the algorithmic bytes
        (every cached history key's K and V row read once, 2 * D elements per
        key: 4 * D bytes in bf16), the broader count that also takes the new
        rows' K/V, the queries and one fp32 output, and the FLOPs (4 * D per
        query-key pair)."""
        D = self.D
        es = 2 if self.wl.dtype == "bf16" else 4
        hist_kv = kv = 0
        flops = 0
        for c, n in zip(io["hist"].tolist(), io["new_len"].tolist()):
            hist_kv += c * 2 * D * es
            kv += (c + n) * 2 * D * es            # K and V rows read once
            flops += 4 * D * (n * c + n * (n + 1) // 2)
        T = io["T"]
        return hist_kv, kv + T * D * es + T * D * 4, flops


def host_info():
    """The CPU model and the logical CPUs the host reports."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count()}


def cpu_baseline(wl, B, R, min_seconds=10.0):
    """The fp64 oracle (as it stands) on whole batches of the same workload,
    batch after batch, until at least `min_seconds` of CPU work are done."""
    import threadpoolctl
    from oracle import layer as olayer
    off = wl.new_offsets
    t0 = time.perf_counter()
    rows = batches = 0
    while True:
        i = batches % R
        us = list(range(B * i, B * (i + 1)))
        x = wl.x0[int(off[us[0]]):int(off[us[-1] + 1])]
        for l in range(wl.layers):
            li = wl.layer(l)
            r = olayer.layer_forward(x, wl.new_len[us], wl.hist_len[us], [li.hist_k[u] for u in us],
                                     [li.hist_v[u] for u in us], li.w1, li.w2, li.pos_bias, wl.pos_mbits,
                                     wl.attn_scale, EPS, wl.H)
            x = r["y"]
        rows += x.shape[0]
        batches += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    return dict(value=rows / dt, unit="new tokens/s", cores=int(threads), kind="oracle", host=host_info(),
                sample=f"{batches} batches of the same workload ({B} users each, {rows} new rows in total, "
                       f"all {wl.layers} layers, every key), fp64 numpy, {dt:.1f} s")


# ---------------------------------------------------------------------------
# KV cache manager measurement: a stream of batches of 64 users drawn with
# Zipf(1.2) popularity from 4096 users, U{1..512} new tokens each, over the
# 8-layer serving pool (2^17 pages of 32 tokens, 1040 pages per user row,
# 1024 cached users at most).  Misses resend the whole sequence, as in the
# serving workload; a sequence restarts once it would pass 4096 tokens, so
# that any batch fits the pool.  Timed: the host plan (lookup, eviction,
# allocation) and the device page-table build of every batch.
# ---------------------------------------------------------------------------
def kvcache_bench(args):
    import numpy as np
    import torch
    from hstu_jagged_silu_fwd_amd.kvcache import KVCache
    L, P, ps, maxP, users, pop, B, cap = 8, 1 << 17, 32, 1040, 1024, 4096, 64, 4096
    rng = np.random.default_rng(args.seed)
    kv = KVCache(num_layers=L, num_pages=P, page_size=ps, max_pages_per_user=maxP, max_users=users)
    length = {}
    def batch():
        ids = []
        while len(ids) < B:
            u = int(min(rng.zipf(1.2), pop))
            if u not in ids:
                ids.append(u)
        cached = kv.lookup(ids)
        n = []
        for u, c in zip(ids, cached.tolist()):
            k = int(rng.integers(1, 513))
            full = length.get(u, 0) + k
            if full > cap:                            # restart an over-long user
                kv.evict(u)
                full, c = k, -1
            length[u] = full
            n.append(k if c >= 0 else full)
        return ids, n
    for _ in range(args.warmup * 20):
        ids, n = batch()
        kv.build_tables(kv.plan(ids, n))
    torch.cuda.synchronize()
    nb = args.steps * 5
    # long-lived objects out of the collector's way, as a serving loop would
    # do (a full collection otherwise lands on one timed batch now and then)
    import gc
    gc.collect()
    gc.freeze()
    host, dev, enq, hits, upd, ev = [], [], [], 0, 0, 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(nb):
        ids, n = batch()
        t0 = time.perf_counter()
        p = kv.plan(ids, n)
        host.append(time.perf_counter() - t0)
        e0.record()
        t1 = time.perf_counter()
        kv.build_tables(p)
        enq.append(time.perf_counter() - t1)
        e1.record()
        torch.cuda.synchronize()
        dev.append(e0.elapsed_time(e1) * 1e-3)
        hits += int((p.hist_len > 0).sum())
        upd += p.updates.shape[0]
        ev += len(p.evicted)
    print(json.dumps({
        "metric": "KV cache plan + page-table build per batch", "value": (sum(host) + sum(dev)) / nb * 1e6,
        "unit": "us per batch of 64 users", "higher_is_better": False, "n_gpus": 1, "batches": nb,
        "host_plan_us": sum(host) / nb * 1e6, "device_tables_us": sum(dev) / nb * 1e6,
        "tables_host_enqueue_us": sum(enq) / nb * 1e6,
        "p50_us": {"host_plan": 1e6 * float(np.median(host)), "device_tables": 1e6 * float(np.median(dev)),
                   "tables_host_enqueue": 1e6 * float(np.median(enq))},
        "p99_max_us": {k: [1e6 * float(np.percentile(v, 99)), 1e6 * float(np.max(v))]
                       for k, v in (("host_plan", host), ("device_tables", dev), ("tables_host_enqueue", enq))},
        "note": "device_tables is the event window around the table build, which includes the host's "
                "staging of the update records",
        "hit_rate": hits / (nb * B), "page_updates_per_batch": upd / nb, "evictions_per_batch": ev / nb,
        "config": {"workload": "kvcache-serving-stream", "layers": L, "pool_pages": P, "page_size": ps,
                   "max_pages_per_user": maxP, "max_users": users, "population": pop, "batch": B,
                   "popularity": "zipf(1.2)", "new": "U{1..512}", "max_tokens": cap}}), flush=True)


# ---------------------------------------------------------------------------
# Host tier measurement on the 3-layer bf16 batch-8 shapes (hidden 512, 4
# heads of 128, 32-token pages; a page of one layer is 32 KiB of K and 32
# KiB of V): bandwidth of the page-copy kernel offloading and onboarding
# 4096 pages, and, for one user with a 4096-token history, the onboard of
# its 3 x 128 pages against recomputing the history through the 3 layers
# (the layer call with no cache on 4096 new rows).
# ---------------------------------------------------------------------------
def kvhost_bench(args):
    import numpy as np
    import torch
    from hstu_jagged_silu_fwd_amd.kvcache import KVCache, Plan
    from hstu_jagged_silu_fwd_amd.stack import HSTUStack
    from workloads import B8_KV_HIT, make_workload
    H, d, ps, L, npg = 4, 128, 32, 3, 4096
    P = 2 * npg
    kv = KVCache(num_layers=L, num_pages=P, page_size=ps, max_pages_per_user=160, max_users=4, host_pages=npg)
    kp = torch.zeros((P, H, ps, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros((P, H, d, ps), dtype=torch.bfloat16, device="cuda")
    page_bytes = 2 * H * ps * d * 2
    empty = (np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros((0, 4), np.int32), [])
    def run(copies, stream=None):
        kv.copy_pages(Plan(*empty, copies), kp, vp, stream=stream)
    off = np.array([[0, i, i, 0] for i in range(npg)], np.int32)
    on = np.array([[1, npg + i, i, 0] for i in range(npg)], np.int32)
    for _ in range(3):
        run(off); run(on)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    t_off = t_on = 0.0
    reps = 10
    for _ in range(reps):
        e[0].record(); run(off); e[1].record(); run(on); e[2].record()
        torch.cuda.synchronize()
        t_off += e[0].elapsed_time(e[1]); t_on += e[1].elapsed_time(e[2])
    t_off, t_on = t_off / reps * 1e-3, t_on / reps * 1e-3
    # one user: onboard 3 x 128 pages vs recompute 4096 tokens through 3 layers
    upages = (4096 // ps) * L
    on_user = on[:upages]
    for _ in range(3):
        run(on_user)
    torch.cuda.synchronize()
    e[0].record()
    for _ in range(reps):
        run(on_user)
    e[1].record()
    torch.cuda.synchronize()
    t_user = e[0].elapsed_time(e[1]) / reps * 1e-3
    wl = make_workload(B8_KV_HIT, seed=0, B=1, hist=("const", 0), new=("const", 4096))
    st = HSTUStack(num_users=1, num_heads=H, head_dim=d, page_size=ps, num_pool_pages=P, max_pages_per_user=160,
                   pos_buckets=wl.pos_buckets, pos_mbits=wl.pos_mbits, attn_scale=wl.attn_scale, num_layers=L)
    for l in range(L):
        li = wl.layer(l)
        table = np.concatenate([np.arange(128 * l, 128 * (l + 1)), np.zeros(32)]).astype(np.int32)[None, :]
        st.set_layer(l, w1t=li.w1t, w2t=li.w2t, pos_bias=li.pos_bias, page_table=table)
    x = torch.from_numpy(wl.x0).to("cuda", torch.bfloat16)
    off_u = np.array([0, 4096], np.int32)
    for _ in range(3):
        st.forward(x, off_u, np.zeros(1, np.int32))
    torch.cuda.synchronize()
    e[0].record()
    for _ in range(reps):
        st.forward(x, off_u, np.zeros(1, np.int32))
    e[1].record()
    torch.cuda.synchronize()
    t_rec = e[0].elapsed_time(e[1]) / reps * 1e-3
    # overlap: one user's onboard on a copy stream while another request's
    # layers run on the compute stream (different pages: nothing to order
    # between them), against the two back to back on one stream
    copier = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    def pair(overlap):
        if overlap:
            copier.wait_stream(compute)
            run(on_user, stream=copier)
        else:
            run(on_user)
        st.forward(x, off_u, np.zeros(1, np.int32))
        if overlap:
            compute.wait_stream(copier)
    for ov in (False, True):
        for _ in range(3):
            pair(ov)
    torch.cuda.synchronize()
    t_pair = {}
    for ov in (False, True):
        e[0].record()
        for _ in range(reps):
            pair(ov)
        e[1].record()
        torch.cuda.synchronize()
        t_pair[ov] = e[0].elapsed_time(e[1]) / reps * 1e-3
    hidden = (t_pair[False] - t_pair[True]) / min(t_user, t_rec)
    gb = npg * page_bytes / 1e9
    print(json.dumps({
        "metric": "host-tier page copies: offload / onboard bandwidth; onboard vs recompute of one user",
        "value": gb / t_on, "unit": "GB/s onboard (host -> HBM)", "higher_is_better": True, "n_gpus": 1,
        "offload_GBs": gb / t_off, "onboard_GBs": gb / t_on, "pages": npg, "page_bytes": page_bytes,
        "user_onboard_us": t_user * 1e6, "user_recompute_us": t_rec * 1e6,
        "recompute_over_onboard": t_rec / t_user,
        "onboard_then_layers_us": t_pair[False] * 1e6, "onboard_overlapped_with_layers_us": t_pair[True] * 1e6,
        "overlap_hidden_fraction": hidden,
        "overlap_note": "one user's onboard (copy stream) against another request's 3 layers (compute stream), "
                        "hidden fraction = (serial - overlapped) / the shorter of the two",
        "config": {"workload": "kvhost-3layer-bf16-hist4096", "layers": L, "hidden": H * d, "heads": H,
                   "head_dim": d, "page_size": ps, "user_tokens": 4096, "user_pages": upages}}), flush=True)


# ---------------------------------------------------------------------------
# Ranking requests on the pages' workload shape (hidden 512, 4 heads, bf16;
# per user 6 context tokens and 4,096 item/action pairs = 8,198 history
# tokens, plus 100 candidates: 8,298 tokens, position table of the aligned
# 8,320): batch 8, 3 and 8 layers.  Synthetic stand-in for the pages'
# KuaiRand-1K inputs: item ids uniform over a 100,000-row table, 8 action
# types, context ids over a 1,000-row table.  Two request kinds:
#   hit:       the history is cached; a request sends the 100 candidates of
#              each user (800 rows): preprocessing, then the layers with
#              every new row a candidate;
#   recompute: nothing cached; a request sends all 8,298 tokens of each user
#              (66,384 rows) with the last 100 as candidates.
# Latency per logical request = time of one batch / 8.
# ---------------------------------------------------------------------------
def rank_cpu_baseline(hist, m, D, H, L, min_seconds=10.0):
    """The fp64 oracle on cached ranking requests of one user each (its
    history K/V given, its m candidates computed through L layers), request
    after request until min_seconds of CPU work are done."""
    import threadpoolctl
    from oracle import layer as olayer
    rng = np.random.default_rng(1)
    layers = [dict(w1=rng.normal(0, 0.02, (D, 4 * D)), w2=rng.normal(0, 0.02, (D, D)),
                   pos_bias=rng.normal(0, 0.1, 128), hist_k=[rng.normal(0.05, 0.24, (hist, D))],
                   hist_v=[rng.normal(0.05, 0.24, (hist, D))]) for _ in range(L)]
    t0 = time.perf_counter()
    n = 0
    while True:
        olayer.stack_forward(rng.normal(0, 1, (m, D)), [m], [hist], layers, 1.0 / 8320, EPS, H, 3,
                             num_candidates=[m])
        n += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    return dict(value=1e3 * dt / n, unit="ms per logical request", cores=int(threads), kind="oracle",
                sample=f"{n} cached ranking requests of one user ({m} candidates over {hist} cached tokens, "
                       f"{L} layers), fp64 numpy, {dt:.1f} s")


def rank_bench(args):
    import torch
    from hstu_jagged_silu_fwd_amd import _lib
    from hstu_jagged_silu_fwd_amd.stack import HSTUStack
    from workloads.gen import BIAS_STD, W_STD, round_bf16
    B, D, H, d, ps = 8, 512, 4, 128, 32
    n_ctx, pairs, m, max_pos = 6, 4096, 100, 8320
    hist = n_ctx + 2 * pairs
    maxP = max_pos // ps
    n_items, n_actions, n_ctxv = 100_000, 8, 1000
    rng = np.random.default_rng(args.seed)
    dev = "cuda"
    bf = torch.bfloat16
    tab = lambda n, sd: torch.from_numpy(round_bf16(rng.normal(0, sd, size=(n, D)).astype(np.float32))).to(dev, bf)
    item_emb, action_emb, ctx_emb, pos_emb = tab(n_items, 0.8), tab(n_actions, 0.8), tab(n_ctxv, 0.8), tab(max_pos, 0.6)
    i32 = lambda a: torch.tensor(np.asarray(a), dtype=torch.int32, device=dev)
    i64 = lambda a: torch.tensor(np.asarray(a), dtype=torch.int64, device=dev)

    def request(hit):
        ctx = np.zeros(1, np.int64) if hit else rng.integers(0, n_ctxv, B * n_ctx)   # (one unused id when none)
        k = 0 if hit else pairs
        r = dict(hist_len=i32([hist if hit else 0] * B),
                 ctx_offsets=i32(np.arange(B + 1) * (0 if hit else n_ctx)), ctx_ids=i64(ctx),
                 hist_offsets=i32(np.arange(B + 1) * k),
                 item_ids=i64(rng.integers(0, n_items, max(B * k, 1))),
                 action_ids=i64(rng.integers(0, n_actions, max(B * k, 1))),
                 cand_offsets=i32(np.arange(B + 1) * m), cand_ids=i64(rng.integers(0, n_items, B * m)))
        T = B * (m if hit else hist + m)
        r.update(item_emb=item_emb, action_emb=action_emb, ctx_emb=ctx_emb, pos_emb=pos_emb,
                 x=torch.empty((T, D), dtype=bf, device=dev),
                 new_offsets=torch.empty(B + 1, dtype=torch.int32, device=dev),
                 num_candidates=torch.empty(B, dtype=torch.int32, device=dev),
                 device_status=torch.zeros(1, dtype=torch.int32, device=dev))
        return r, T

    out_all = {}
    for L in (3, 8):
        P = L * B * maxP
        st = HSTUStack(num_users=B, num_heads=H, head_dim=d, page_size=ps, num_pool_pages=P, max_pages_per_user=maxP,
                       pos_buckets=128, pos_mbits=3, attn_scale=1.0 / max_pos, norm_eps=EPS, dtype="bf16",
                       num_layers=L)
        perm = rng.permutation(P).astype(np.int32)
        for l in range(L):
            st.set_layer(l, w1t=round_bf16(rng.normal(0, W_STD, size=(4 * D, D)).astype(np.float32)),
                         w2t=round_bf16(rng.normal(0, W_STD, size=(D, D)).astype(np.float32)),
                         pos_bias=rng.normal(0, BIAS_STD, size=128).astype(np.float32),
                         page_table=perm[l * B * maxP:(l + 1) * B * maxP].reshape(B, maxP))
        res = {}
        # recompute first: it also fills the pool with every user's history
        lib = _lib.load()
        for kind, steps in (("recompute", max(3, args.steps // 6)), ("hit", args.steps)):
            req, T = request(kind == "hit")
            # argument lists built once (the timed loop only calls the library)
            pdesc = _lib.PrepDesc(num_users=B, hidden=D, dtype=_lib.HSTU_BF16, total_new=T, item_rows=n_items,
                                  action_rows=n_actions, ctx_rows=n_ctxv, max_positions=max_pos)
            ptr = lambda k: ctypes.c_void_p(req[k].data_ptr())
            stream = torch.cuda.current_stream().cuda_stream
            pargs = [ctypes.byref(pdesc)] + [ptr(k) for k in (
                "hist_len", "ctx_offsets", "ctx_ids", "hist_offsets", "item_ids", "action_ids", "cand_offsets",
                "cand_ids", "item_emb", "action_emb", "ctx_emb", "pos_emb", "x", "new_offsets", "num_candidates",
                "device_status")] + [ctypes.c_void_p(stream)]
            ldesc = st.desc(T)
            ws = st.workspace(T)
            ys = [torch.empty((T, D), dtype=bf, device=dev) for _ in range(2)]
            largs = []
            for l in range(L):
                Ll = st.layers[l]
                xin = req["x"] if l == 0 else ys[(l - 1) % 2]
                largs.append([ctypes.byref(ldesc), ctypes.c_void_p(xin.data_ptr()), ptr("new_offsets"),
                              ptr("hist_len"), ptr("num_candidates"), ctypes.c_void_p(Ll["page_table"].data_ptr()),
                              ctypes.c_void_p(st.k_pool.data_ptr()), ctypes.c_void_p(st.v_pool.data_ptr()),
                              ctypes.c_void_p(Ll["w1t"].data_ptr()), ctypes.c_void_p(Ll["w2t"].data_ptr()),
                              ctypes.c_void_p(Ll["pos_bias"].data_ptr()), None, None, None,
                              ctypes.c_void_p(ys[l % 2].data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                              ctypes.c_size_t(ws.numel()), ctypes.c_void_p(stream), None])

            # the timed request: preprocessing, then the whole stack in one call
            sws = torch.empty(max(_lib.stack_workspace_size(ldesc, L), ws.numel()), dtype=torch.uint8, device=dev)
            P = ctypes.c_void_p
            parr = lambda vals: (P * L)(*[P(v) for v in vals])
            keep = [parr([st.layers[l]["page_table"].data_ptr() for l in range(L)]),
                    parr([st.k_pool.data_ptr()] * L), parr([st.v_pool.data_ptr()] * L),
                    parr([st.layers[l]["w1t"].data_ptr() for l in range(L)]),
                    parr([st.layers[l]["w2t"].data_ptr() for l in range(L)]),
                    parr([st.layers[l]["pos_bias"].data_ptr() for l in range(L)]),
                    parr([ys[l % 2].data_ptr() for l in range(L)])]
            sargs = [ctypes.byref(ldesc), L, ptr("x"), ptr("new_offsets"), ptr("hist_len"), ptr("num_candidates"),
                     *keep[:6], None, None, None, keep[6], P(sws.data_ptr()), ctypes.c_size_t(sws.numel()),
                     P(stream)]

            def run():
                rc = lib.hstu_preprocess(*pargs)
                rc |= lib.hstu_stack_fwd(*sargs)
                if rc != 0:
                    raise RuntimeError(f"ranking request failed: {rc}")
            for _ in range(args.warmup):
                run()
            torch.cuda.synchronize()
            assert int(req["device_status"].item()) == 0 and st.read_status(sws) == 0
            t0 = time.perf_counter()
            for _ in range(steps):
                run()
            torch.cuda.synchronize()
            wall = (time.perf_counter() - t0) / steps
            # the preprocessing alone (two kernels), event-bracketed
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                lib.hstu_preprocess(*pargs)
            e1.record()
            torch.cuda.synchronize()
            prep_us = 1e3 * e0.elapsed_time(e1) / steps
            prep_bytes = T * 3 * D * 2 + T * 8           # two table rows read, one row written; the id
            res[kind] = dict(rows=T, ms_per_batch=1e3 * wall, ms_per_request=1e3 * wall / B,
                             tokens_per_s=T / wall, preprocess_us=prep_us,
                             preprocess_gbs=prep_bytes / (prep_us * 1e-6) / 1e9)
            if kind == "hit" and L == 3:
                # event pass over the same calls: each layer's stage kernels
                # bracketed by runtime-stamped events; the attention's roofline
                hip = _lib.hip_runtime()
                hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
                hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
                nev = 2 * _lib.NUM_STAGES
                evs = []
                for _ in range(steps * L):
                    arr = (ctypes.c_void_p * nev)()
                    for j in range(nev):
                        e = ctypes.c_void_p()
                        assert hip.hipEventCreate(ctypes.byref(e)) == 0
                        arr[j] = e
                    evs.append(arr)
                for st_i in range(steps):
                    lib.hstu_preprocess(*pargs)
                    for l, a_l in enumerate(largs):
                        assert lib.hstu_layer_fwd_cand(*a_l[:-1], evs[st_i * L + l]) == 0
                torch.cuda.synchronize()
                ms = ctypes.c_float(0)
                stage = np.zeros(_lib.NUM_STAGES)
                for arr in evs:
                    for k in range(_lib.NUM_STAGES):
                        assert hip.hipEventElapsedTime(ctypes.byref(ms), arr[2 * k], arr[2 * k + 1]) == 0
                        stage[k] += ms.value
                stage_us = 1e3 * stage / len(evs)
                attn_bytes = B * (hist + m) * 4 * D + T * D * 2 + T * D * 4   # K/V rows once, Q, fp32 partial out
                attn_flops = 4 * D * B * m * (hist + 1)
                ach = attn_bytes / (stage_us[2] * 1e-6) / 1e9
                res["hit"]["stages_us"] = {n: float(v) for n, v in zip(_lib.STAGES, stage_us)}
                res["hit"]["roofline"] = dict(kernel="paged_silu_attn (candidates)", bound="hbm", achieved=ach,
                                              peak=HBM_PEAK_GBS, unit="GB/s", frac=ach / HBM_PEAK_GBS,
                                              traffic=None, mean_us=float(stage_us[2]),
                                              bytes_per_launch=attn_bytes,
                                              mfma_frac=attn_flops / (stage_us[2] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS)
        res["recompute_over_hit"] = res["recompute"]["ms_per_batch"] / res["hit"]["ms_per_batch"]
        out_all[f"{L}layer"] = res
        del st
        torch.cuda.empty_cache()
    out_all["cpu_baseline"] = None if args.no_cpu_baseline else rank_cpu_baseline(hist, m, D, H, 3)
    print(json.dumps({
        "metric": "ranking request latency, pages-shaped workload (cached history vs full recompute)",
        "unit": "ms per logical request", "higher_is_better": False, "n_gpus": 1, "dtype": "bf16",
        "data": "synthetic", "steps_hit": args.steps, "results": out_all,
        "config": {"workload": "rank-bf16-b8-ctx6-hist8192-cand100", "batch": B, "hidden": D, "heads": H,
                   "history_tokens": hist, "candidates": m, "context_tokens": n_ctx, "item_action_pairs": pairs,
                   "position_table": max_pos, "page_size": ps, "item_table_rows": n_items}}), flush=True)


# ---------------------------------------------------------------------------
# Beam-decode attention of Semantic-ID GR on the pages' request shapes
# (offline: 4 requests, context 1,000, beam 256, 3 decoded tokens; online:
# context 5,000, concurrency 4).  The decoder's attention shape (16 query
# heads, 8 KV heads, head dim 128, bf16) is that of a Qwen3-1.7B-class model,
# which the pages name without giving its shape.  One call = one decode step
# of one layer for every beam of every request.
# ---------------------------------------------------------------------------
def beam_cpu_baseline(ctx, R, W, Hq, Hkv, d, min_seconds=10.0):
    """The fp64 oracle on decode step 2 for one request of 16 beams at a
    time (a bounded sample), scaled to a whole call of R requests x W beams."""
    import threadpoolctl
    from oracle.beam import beam_decode_attention
    rng = np.random.default_rng(2)
    w = 16
    q = rng.normal(0, 1, (1, w, Hq, d))
    ck, cv = [rng.normal(0, 1, (ctx, Hkv, d))], [rng.normal(0, 1, (ctx, Hkv, d))]
    bk, bv = rng.normal(0, 1, (1, 3, w, Hkv, d)), rng.normal(0, 1, (1, 3, w, Hkv, d))
    path = rng.integers(0, w, (1, w, 2))
    t0 = time.perf_counter()
    n = 0
    while True:
        beam_decode_attention(q, ck, cv, bk, bv, path, 2, d ** -0.5)
        n += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    return dict(value=1e6 * dt / n * (R * W) / w, unit="us per decode step (all beams), scaled", cores=int(threads),
                kind="oracle", sample=f"{n} calls of 1 request x {w} beams at context {ctx}, step 2, fp64 numpy, "
                                      f"{dt:.1f} s, scaled by {R * W // w}")


def beam_bench(args):
    import torch
    from hstu_jagged_silu_fwd_amd import _lib
    from hstu_jagged_silu_fwd_amd import beam as hb
    R, W, Hq, Hkv, d, S = 4, 256, 16, 8, 128, 3
    rng = torch.Generator(device="cuda").manual_seed(args.seed)
    bf = torch.bfloat16
    lib = hb._lib_beam()
    res = {}
    for ctx in (1000, 5000):
        Cmax = (ctx + 31) // 32 * 32
        rnd = lambda *shape: torch.randn(*shape, generator=rng, device="cuda", dtype=torch.float32).to(bf)
        q = rnd(R, W, Hq, d)
        ck, cvt = rnd(R, Hkv, Cmax, d), rnd(R, Hkv, d, Cmax)
        bk, bv = rnd(R, S, W, Hkv, d), rnd(R, S, W, Hkv, d)
        ctx_len = torch.full((R,), ctx, dtype=torch.int32, device="cuda")
        path = torch.randint(0, W, (R, W, S), generator=rng, device="cuda", dtype=torch.int32)
        out = torch.empty_like(q)
        per = {}
        for t in range(S):
            desc = hb.make_desc(q, ck, bk, t, d ** -0.5)
            ws = torch.empty(hb.workspace_size(desc), dtype=torch.uint8, device="cuda")
            pth = path[:, :, :t].contiguous() if t else None
            argv = [ctypes.byref(desc)] + [ctypes.c_void_p(x.data_ptr()) if x is not None else None
                                           for x in (q, ck, cvt, ctx_len, bk, bv, pth, out, ws)] + \
                   [ctypes.c_size_t(ws.numel()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)]
            for _ in range(args.warmup):
                lib.hstu_beam_decode_attn(*argv)
            torch.cuda.synchronize()
            assert int(ws[:4].view(torch.int32).item()) == 0
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                rc = lib.hstu_beam_decode_attn(*argv)
            e1.record()
            torch.cuda.synchronize()
            assert rc == 0
            us = 1e3 * e0.elapsed_time(e1) / args.steps
            keys = ctx + t + 1
            flops = 4.0 * R * W * Hq * keys * d
            byts = 2.0 * (2 * R * Hkv * ctx * d + 2 * R * W * Hq * d + 2 * R * (t + 1) * W * Hkv * d)
            per[f"step{t}"] = dict(us=us, tflops=flops / us / 1e6, mfma_frac=flops / us / 1e6 / BF16_PEAK_TFLOPS,
                                   gbs=byts / us / 1e3, hbm_frac=byts / us / 1e3 / HBM_PEAK_GBS,
                                   algorithmic_bytes=byts, flops=flops)
        if not args.no_cpu_baseline and ctx == 1000:
            res["cpu_baseline"] = beam_cpu_baseline(ctx, R, W, Hq, Hkv, d)
        res[f"ctx{ctx}"] = per
        del q, ck, cvt, bk, bv, out
        torch.cuda.empty_cache()
    print(json.dumps({
        "metric": "Semantic-ID beam-decode attention per decode step and layer", "unit": "us",
        "higher_is_better": False, "n_gpus": 1, "dtype": "bf16", "data": "synthetic", "steps": args.steps,
        "results": res,
        "config": {"workload": "sid-beam-decode-r4-w256-hq16-hkv8-d128", "requests": R, "beam_width": W,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "contexts": [1000, 5000], "decode_steps": S,
                   "timing": "event-bracketed back-to-back calls (split kernel + combine kernel)"}}), flush=True)


def vendor_gemm(args):
    """X*W1 ([T, D] x [D, 4D]) and G*W2 ([T, D] x [D, D]) of every batch of
    the batch-8 workloads through torch.matmul (hipBLASLt), against this
    library's projection stages (X*W1 with its SiLU, split and K/V append
    epilogue; G*W2) from the event pass over the same batches.  The vendor
    products are replayed from a captured graph of 10 calls per batch, so the
    host's launch cost is not timed; each replay's result is checked against
    the eager product."""
    import torch
    from workloads import B8_RECOMPUTE
    res = {}
    for name in (WORKLOAD, B8_RECOMPUTE):
        b = Bench(argparse.Namespace(workload=name, instances=args.instances, seed=args.seed))
        m = time_stack(b, max(6, b.R * 2), 2, events=True)
        st = {k: 1e3 * m["stage_ms"][j] / m["n_launch"] for j, k in enumerate(b._lib.STAGES)}
        D = b.D
        g = torch.Generator(device="cuda").manual_seed(args.seed)
        w1 = torch.randn(4 * D, D, generator=g, device="cuda").to(torch.bfloat16)
        w2 = torch.randn(D, D, generator=g, device="cuda").to(torch.bfloat16)
        per = {"w1": [], "w2": []}
        for io in b.inst:
            a = torch.randn(io["T"], D, generator=g, device="cuda").to(torch.bfloat16)
            for key, w in (("w1", w1), ("w2", w2)):
                wt = w.t()
                out = torch.empty(io["T"], w.shape[0], dtype=torch.bfloat16, device="cuda")
                for _ in range(3):
                    torch.matmul(a, wt, out=out)
                torch.cuda.synchronize()
                want = out.clone()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    for _ in range(10):
                        torch.matmul(a, wt, out=out)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                reps = 20
                graph.replay()
                torch.cuda.synchronize()
                e0.record()
                for _ in range(reps):
                    graph.replay()
                e1.record()
                torch.cuda.synchronize()
                for _ in range(2):                       # replays with eager work between, each checked
                    out.zero_()
                    graph.replay()
                    torch.cuda.synchronize()
                    assert torch.equal(out, want), "graph replay differs from the eager product"
                per[key].append(1e3 * e0.elapsed_time(e1) / (10 * reps))
                del graph
        rows = [io["T"] for io in b.inst]
        fl1 = sum(2.0 * t * D * 4 * D for t in rows) / len(rows)
        fl2 = sum(2.0 * t * D * D for t in rows) / len(rows)
        v1, v2 = float(np.mean(per["w1"])), float(np.mean(per["w2"]))
        res[name] = dict(rows_per_batch=rows, hidden=D,
                         x_w1=dict(vendor_us=v1, ours_us=st["proj"], vendor_tflops=fl1 / v1 / 1e6,
                                   ours_tflops=fl1 / st["proj"] / 1e6,
                                   ours_note="includes SiLU, the U|V|Q|K split and the K/V page append"),
                         g_w2=dict(vendor_us=v2, ours_us=st["out"], vendor_tflops=fl2 / v2 / 1e6,
                                   ours_tflops=fl2 / st["out"] / 1e6))
        del b
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "projection GEMM time per layer, this library against the vendor library",
                      "unit": "us", "higher_is_better": False, "n_gpus": 1, "dtype": "bf16",
                      "data": "synthetic", "results": res,
                      "timing": "ours: hipExtLaunchKernel events per launch (event pass); vendor: graph replay "
                                "of 10 torch.matmul calls per batch, mean per call"}), flush=True)


def main():
    args = parse()
    if args.vendor_gemm:
        vendor_gemm(args)
        return
    if args.beam:
        beam_bench(args)
        return
    if args.rank:
        rank_bench(args)
        return
    if args.kvhost:
        kvhost_bench(args)
        return
    if args.kvcache:
        kvcache_bench(args)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}), flush=True)
        sys.exit(2)
    import torch
    from workloads import B8_KV_HIT_LONG, B8_RECOMPUTE, B64_SERVING
    if args.in_flight > 0:
        b = Bench(args)
        m = time_stack(b, args.steps, args.warmup, events=False)
        serial = m["tokens"] / m["wall"]
        rec = in_flight(b, args.steps, args.warmup, args.in_flight, serial, graphs=True)
        rec.update(workload=b.wl.name, serial_value=serial, serial_ms_per_step=1e3 * m["wall"] / args.steps)
        print(json.dumps(rec), flush=True)
        return
    b = Bench(args)
    m = time_stack(b, args.steps, args.warmup, events=not args.no_events)
    value = m["tokens"] / m["wall"]
    from workloads import CONFIGS
    spec = CONFIGS[b.wl.name]
    out = dict(metric=METRIC if b.wl.name == WORKLOAD else f"HSTU stack new-tokens/sec ({b.wl.name})",
               value=value, unit="new tokens/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=1e3 * m["wall"] / args.steps, higher_is_better=True,
               scaling="weak", vs_baseline=None, dtype=b.wl.dtype, data="synthetic",
               config=dict(workload=b.wl.name, layers=b.L, batch=b.B, hidden=b.D, heads=b.H,
                           head_dim=b.d, page_size=b.wl.page_size, pool_pages=b.wl.num_pool_pages,
                           hist=str(spec["hist"]), new=str(spec["new"]), instances=b.R,
                           timestamps=b.wl.ts_buckets > 0,
                           new_tokens_per_step=m["tokens"] / args.steps,
                           per_layer_new_tokens_per_s=value * b.L))
    if m.get("stage_ms") is not None:
        out["roofline"] = roofline_of(m, load_traffic() if b.wl.name == WORKLOAD else None)
        add_stages(out, m, b, args.steps)
    headline = b.wl.name == WORKLOAD and not args.no_events and not args.no_extras
    if headline:
        # the same users recomputed from scratch (nothing cached), against
        # the cached step of the same batch
        out["cache_speedup"] = {b.wl.name: cache_speedup(args, b)}
        out["batch_invariant"] = invariant_cost(b, args.steps, args.warmup, m)
        # the same steps with two and three batches in flight (serving)
        out["in_flight"] = [guarded(in_flight, b, args.steps, args.warmup, 2, value)] + \
            [guarded(in_flight, b, args.steps, args.warmup, k, value, graphs=True) for k in (1, 2, 3)]
    if not args.no_cpu_baseline and b.wl.name == WORKLOAD:
        out["cpu_baseline"] = cpu_baseline(b.wl, b.B, b.R)
    if headline:
        # the 8-layer long-history hit (where the pages' KV streaming lives)
        del b
        torch.cuda.empty_cache()
        bl, rec = workload_record(args, B8_KV_HIT_LONG, max(4, args.steps // 6), 2)
        out["cache_speedup"][bl.wl.name] = cache_speedup(args, bl)
        out["long_history"] = rec
        del bl
        torch.cuda.empty_cache()
        out["long_history"]["in_flight"] = guarded(
            lambda: workload_in_flight(args, B8_KV_HIT_LONG, max(6, args.steps // 6), 2, 3)[1])
        torch.cuda.empty_cache()
        # the compute-bound configurations: the batch-8 full recompute and the
        # 64-user serving mix (its long miss users' causal recomputes)
        for name, key, st in ((B8_RECOMPUTE, "full_recompute", max(4, args.steps // 6)),
                              (B64_SERVING, "serving_mix", 3)):
            bx, out[key] = workload_record(args, name, st, 1, bound="mfma")
            del bx
            torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def guarded(fn, *a, **kw):
    """An extra record of the JSON line: its failure is reported in the
    record instead of ending the run before the headline line is printed."""
    import torch
    try:
        return fn(*a, **kw)
    except Exception as e:                      # noqa: BLE001 -- reported, not hidden
        torch.cuda.synchronize()
        return {"error": f"{type(e).__name__}: {e}"}


def in_flight(b, steps, warmup, nstreams, serial_value, graphs=False):
    """The headline steps with `nstreams` batches in flight, as a server
    running several instances of the model on one GPU would: step s runs
    batch s mod R in one hstu_stack_fwd call on stream s mod nstreams, each
    stream with a workspace of its own (R is a multiple of nstreams, so a
    batch always runs on the same stream and no two streams write the same
    output rows or pool pages).  Every step still runs the whole stack over
    its users; only consecutive steps overlap in time.  graphs: each batch's
    call is captured once into a HIP graph on its stream and the steps
    replay the graphs (one host call per step instead of one per kernel:
    the eager calls' host-side enqueueing, ~100 us per 3-layer step, would
    otherwise bound the overlapped steps)."""
    import torch
    if b.R % nstreams:
        raise ValueError("instances must be a multiple of the streams")
    P = ctypes.c_void_p
    streams = [torch.cuda.Stream() for _ in range(nstreams)]     # default priority
    wss = [torch.empty_like(b.ws) for _ in range(nstreams)]
    calls = []
    for i, io in enumerate(b.inst):
        a = list(io["stack_args"])
        a[-3] = P(wss[i % nstreams].data_ptr())
        a[-1] = P(streams[i % nstreams].cuda_stream)
        calls.append((tuple(a), streams[i % nstreams]))

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"hstu_stack_fwd failed: {rc}")

    torch.cuda.synchronize()
    if graphs:
        replays = []
        for a, st in calls:
            check(b.lib.hstu_stack_fwd(*a))          # once eagerly on the capture stream
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=st):
                check(b.lib.hstu_stack_fwd(*a))
            replays.append((g, st))
        torch.cuda.synchronize()

        def run(n):
            for s in range(n):
                g, st = replays[s % b.R]
                with torch.cuda.stream(st):
                    g.replay()
    else:
        def run(n):
            for s in range(n):
                check(b.lib.hstu_stack_fwd(*calls[s % b.R][0]))

    run(warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tokens = sum(b.inst[s % b.R]["T"] for s in range(steps))
    value = tokens / wall
    return dict(streams=nstreams, graphs=graphs, value=value, unit="new tokens/s",
                ms_per_step=1e3 * wall / steps, steps=steps, speedup_vs_serial=value / serial_value,
                note="wall time of the steps; each stream's calls are ordered, the streams' calls overlap")


def invariant_cost(b, steps, warmup, m):
    """The same timed steps with the batch-invariant flag set on every call
    (fixed 256-key attention pieces, one phase per item): its cost against
    the default split."""
    for io in b.inst:
        io["desc"].flags = b._lib.FLAG_BATCH_INVARIANT
    try:
        mi = time_stack(b, steps, warmup, events=False)
    finally:
        for io in b.inst:
            io["desc"].flags = 0
    ms = 1e3 * mi["wall"] / steps
    return dict(value=mi["tokens"] / mi["wall"], unit="new tokens/s", ms_per_step=ms,
                slowdown=ms / (1e3 * m["wall"] / m["steps"]))


def time_stack(b, steps, warmup, events=True):
    """Wall time of `steps` stack calls after `warmup` (each one
    hstu_stack_fwd call, synchronised on both sides), and, with events, a
    second pass over the same steps with runtime-stamped start/stop events
    around every stage kernel (kept out of the timed pass because enqueueing
    the events slows the host's submission of the launches)."""
    import torch
    for s in range(warmup):
        b.step(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        b.step(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    m = dict(wall=wall, steps=steps, tokens=sum(b.inst[s % b.R]["T"] for s in range(steps)), stage_ms=None)
    if not events:
        return m
    evs = b.make_events(steps)
    torch.cuda.synchronize()
    for s in range(steps):
        b.step(s, evs[s])
    torch.cuda.synchronize()
    stage_ms = np.zeros(b._lib.NUM_STAGES)
    hist_bytes = broad_bytes = flops = 0
    n_launch = 0
    attn_each, step_each = [], []
    for s in range(steps):
        io = b.inst[s % b.R]
        hb, bb, fl = b.attn_work(io)
        step_sum = 0.0
        for l in range(b.L):
            ev = evs[s][l]
            for k in range(b._lib.NUM_STAGES):
                ms = b.elapsed_ms(ev[2 * k], ev[2 * k + 1])
                stage_ms[k] += ms
                step_sum += ms
                if k == 2:
                    attn_each.append(1e3 * ms)
            hist_bytes += hb
            broad_bytes += bb
            flops += fl
            n_launch += 1
        step_each.append(1e3 * step_sum)
    m.update(stage_ms=stage_ms, hist_bytes=hist_bytes, broad_bytes=broad_bytes, flops=flops, n_launch=n_launch,
             attn_each=attn_each, step_each=step_each)
    return m


def roofline_of(m, traffic):
    """The attention kernel against HBM: the algorithmic bytes are every
    cached history key's K and V read once (4 * D bytes per key in bf16) per
    launch, over its mean duration from the event pass; the broader count
    (plus the new rows' K/V, the queries and one fp32 output) is kept beside
    it, and the MFMA position of the same launches (4 * D FLOP per
    query-key pair)."""
    attn_s = m["stage_ms"][2] / 1e3
    n = m["n_launch"]
    achieved = m["hist_bytes"] / attn_s / 1e9
    broad = m["broad_bytes"] / attn_s / 1e9
    return dict(kernel="paged_silu_attn", bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                frac=achieved / HBM_PEAK_GBS, traffic=traffic, mean_us=1e6 * attn_s / n,
                timing="hipExtLaunchKernel start/stop events per launch, second pass of the same steps",
                bytes_per_launch=m["hist_bytes"] / n,
                bytes_note="algorithmic: every cached history key's K and V row read once (4 * D bytes)",
                broad_bytes_per_launch=m["broad_bytes"] / n, broad_achieved=broad,
                broad_frac=broad / HBM_PEAK_GBS,
                mfma_tflops=m["flops"] / attn_s / 1e12, mfma_frac=m["flops"] / attn_s / 1e12 / BF16_PEAK_TFLOPS)


def roofline_mfma(m):
    """The attention kernel against the bf16 MFMA peak (4 * D FLOP per
    (query, key) pair over the causal and cached keys), for workloads whose
    attention is compute-bound (full recompute, long miss users)."""
    attn_s = m["stage_ms"][2] / 1e3
    n = m["n_launch"]
    achieved = m["flops"] / attn_s / 1e12
    return dict(kernel="paged_silu_attn", bound="mfma", achieved=achieved, peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                frac=achieved / BF16_PEAK_TFLOPS, traffic=None, mean_us=1e6 * attn_s / n,
                timing="hipExtLaunchKernel start/stop events per launch, second pass of the same steps",
                flops_per_launch=m["flops"] / n,
                flops_note="4 * D FLOP per (query, key) pair over the causal and cached keys")


def workload_record(args, name, steps, warmup, bound="hbm"):
    """One more configuration through the same stack path, as a record of
    the main line (its own batch, one instance)."""
    import torch
    from workloads import CONFIGS
    b = Bench(argparse.Namespace(workload=name, instances=1, seed=args.seed))
    m = time_stack(b, steps, warmup, events=True)
    rec = dict(workload=b.wl.name, value=m["tokens"] / m["wall"], unit="new tokens/s",
               ms_per_step=1e3 * m["wall"] / m["steps"], steps=m["steps"], layers=b.L, batch=b.B,
               hist=str(CONFIGS[name]["hist"]), new=str(CONFIGS[name]["new"]), page_size=b.wl.page_size,
               roofline=roofline_of(m, None) if bound == "hbm" else roofline_mfma(m))
    add_stages(rec, m, b, m["steps"])
    return b, rec


def workload_in_flight(args, name, steps, warmup, nstreams):
    """Configuration `name` with `nstreams` independent batches (its users
    drawn nstreams times over), timed with the steps serialised on one
    stream (eager calls) and then with the batches in flight on streams of
    their own (graph replays, see in_flight);
    the history K/V streamed per second of wall time (every layer's cached
    keys, 4 * D bytes each) is reported beside the token rates."""
    b = Bench(argparse.Namespace(workload=name, instances=nstreams, seed=args.seed, any_instances=True))
    m = time_stack(b, steps, warmup, events=False)
    serial = m["tokens"] / m["wall"]
    rec = in_flight(b, steps, warmup, nstreams, serial, graphs=True)
    hist_bytes = b.L * sum(b.attn_work(b.inst[s % b.R])[0] for s in range(steps))
    wall = rec["ms_per_step"] * steps / 1e3
    rec.update(serial_value=serial, serial_ms_per_step=1e3 * m["wall"] / steps,
               kv_stream_gbs=hist_bytes / wall / 1e9, kv_stream_frac=hist_bytes / wall / 1e9 / HBM_PEAK_GBS,
               serial_kv_stream_gbs=hist_bytes / m["wall"] / 1e9,
               kv_note="history K/V bytes of every layer over the wall time of the whole steps (all kernels)")
    return b, rec


def add_stages(out, m, b, steps):
    n = m["n_launch"]
    out["stages_us"] = {name: 1e3 * m["stage_ms"][k] / n for k, name in enumerate(b._lib.STAGES)}
    out["stages_note"] = ("per layer, from the layer-by-layer event pass, where prep runs in every layer; "
                          "the timed stack call runs it once per step")
    out["kernel_sum_ms_per_step"] = float(m["stage_ms"].sum() / steps)
    pct = lambda v: [float(np.percentile(v, q)) for q in (10, 50, 90)]
    out["percentiles_us"] = {"attn_launch_p10_p50_p90": pct(m["attn_each"]),
                             "step_kernels_p10_p50_p90": pct(m["step_each"]),
                             "note": "event pass; steps rotate over the instances' different batches"}


def cache_speedup(args, b, steps=6, warmup=2):
    """The cached step of the bench's first batch against the same users
    recomputed from scratch (each user's whole sequence, history and new
    rows, as new rows with nothing cached) through the same stack: the
    analogue, on one MI355X, of the pages' KV-hit versus no-cache latency
    ratios (context only)."""
    import torch
    from workloads import make_workload
    io = b.inst[0]
    for _ in range(warmup):
        b.step(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        b.step(0)
    torch.cuda.synchronize()
    cached = (time.perf_counter() - t0) / steps
    full = (io["hist"] + io["new_len"]).astype(int).tolist()
    wr = make_workload(b.wl.name, seed=args.seed + 1, B=len(full), hist=("const", 0), new=("fixed", full))
    br = Bench(args, wl=wr)
    mr = time_stack(br, steps, warmup, events=False)
    rec = mr["wall"] / steps
    del br
    torch.cuda.empty_cache()
    return dict(cached_ms_per_batch=1e3 * cached, recompute_ms_per_batch=1e3 * rec, speedup=rec / cached,
                users=len(full), cached_tokens=int(io["hist"].sum()), new_tokens=int(io["T"]),
                recompute_tokens=int(sum(full)))


if __name__ == "__main__":
    main()
