"""Seeded synthetic workloads for the HSTU layer forward over a paged KV cache.

The five workload shapes follow the benchmark setting of the NVIDIA blog post
"Deploying an HSTU generative recommender with NVIDIA Dynamo-Triton" (section
"HSTU serving latency benchmark": 3- and 8-layer HSTU, hidden 512, 4 heads,
BF16 weights and BF16 KV cache, long per-user histories), scaled out to a
serving-size mixed-hit case.  The blog's KuaiRand-1K data is not available, so
every tensor is drawn here from a fixed seed with the stated distributions.

Nothing in this file computes any part of the layer: it draws lengths, weights,
inputs, bias tables, cached history K/V values, page permutations and
timestamps, and lays out integer structure (prefix offsets, page tables).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

# ---------------------------------------------------------------------------
# Workload table, keyed by the workload's name.  `stream` is the first
# entropy word of its seed sequence.  Length specs:
#   ("fixed", [n0, n1, ...])  one value per user
#   ("const", v)              every user
#   ("uniform", lo, hi)       integers uniform in [lo, hi] inclusive
#   ("zipf", a, lo, hi)       numpy Generator.zipf(a), then clipped to [lo, hi]
# pos_mbits / ts_mbits are the mantissa-bit parameter of the log-linear
# bucket rule used by the relative-bias tables (fixed per workload).
# attn_scale is 1/N with N the workload's maximum total sequence length.
# ---------------------------------------------------------------------------
TINY_FP32 = "tiny-fp32-1layer-nocache"
B8_RECOMPUTE = "3layer-bf16-b8-full-recompute"
B8_KV_HIT = "3layer-bf16-b8-paged-kv-hit"
B8_KV_HIT_LONG = "8layer-bf16-b8-paged-kv-hit-long"
B64_SERVING = "8layer-bf16-b64-mixed-hit-serving"

CONFIGS: Dict[str, dict] = {
    TINY_FP32: dict(
        stream=1, dtype="f32", layers=1, B=2,
        D=64, H=2, d=32, hist=("const", 0), new=("fixed", [37, 64]),
        page_size=32, pool_pages=None, pos_buckets=32, pos_mbits=3,
        ts_buckets=0, ts_mbits=0, attn_scale=1.0 / 64, miss_frac=0.0,
    ),
    B8_RECOMPUTE: dict(
        stream=2, dtype="bf16", layers=3, B=8,
        D=512, H=4, d=128, hist=("const", 0), new=("uniform", 256, 4096),
        page_size=32, pool_pages=None, pos_buckets=128, pos_mbits=3,
        ts_buckets=0, ts_mbits=0, attn_scale=1.0 / 4096, miss_frac=0.0,
    ),
    B8_KV_HIT: dict(
        stream=3, dtype="bf16", layers=3, B=8,
        D=512, H=4, d=128, hist=("uniform", 256, 4096), new=("uniform", 16, 256),
        page_size=32, pool_pages=1 << 16, pos_buckets=128, pos_mbits=3,
        ts_buckets=0, ts_mbits=0, attn_scale=1.0 / 4096, miss_frac=0.0,
    ),
    B8_KV_HIT_LONG: dict(
        stream=4, dtype="bf16", layers=8, B=8,
        D=512, H=4, d=128, hist=("uniform", 4096, 16384), new=("const", 64),
        page_size=64, pool_pages=1 << 16, pos_buckets=256, pos_mbits=4,
        ts_buckets=0, ts_mbits=0, attn_scale=1.0 / 16448, miss_frac=0.0,
    ),
    B64_SERVING: dict(
        stream=5, dtype="bf16", layers=8, B=64,
        D=1024, H=8, d=128, hist=("zipf", 1.2, 32, 32768), new=("uniform", 1, 512),
        page_size=32, pool_pages=1 << 17, pos_buckets=256, pos_mbits=4,
        ts_buckets=64, ts_mbits=2, attn_scale=1.0 / 33280, miss_frac=0.3,
    ),
}

W_STD = 0.02        # W1, W2 ~ N(0, 0.02^2)
X_STD = 1.0         # X ~ N(0, 1)
BIAS_STD = 0.1      # bias buckets ~ N(0, 0.1^2)
# Cached history K/V entries (cache-hit workloads): i.i.d. normal with the
# first two moments of the values a layer of this width produces.
HIST_KV_MEAN = 0.05
HIST_KV_STD = 0.24
TS_GAP_MEAN = 4.0   # timestamp gaps are 1 + floor(Exp(mean 4))


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as
    float32.  This is only the storage format of bf16 inputs."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _draw_lengths(rng: np.random.Generator, spec, B: int) -> np.ndarray:
    kind = spec[0]
    if kind == "const":
        out = np.full(B, spec[1], dtype=np.int64)
    elif kind == "fixed":
        out = np.asarray(spec[1], dtype=np.int64)
        assert out.shape == (B,), (spec, B)
    elif kind == "uniform":
        out = rng.integers(spec[1], spec[2], size=B, endpoint=True)
    elif kind == "zipf":
        out = np.clip(rng.zipf(spec[1], size=B), spec[2], spec[3])
    else:
        raise ValueError(f"unknown length spec {spec}")
    return out.astype(np.int32)


@dataclasses.dataclass
class LayerInputs:
    """Per-layer parameters and cached state (all float32 / int32 arrays)."""
    w1: np.ndarray                 # [D, 4D]
    w2: np.ndarray                 # [D, D]
    pos_bias: np.ndarray           # [pos_buckets] float32
    ts_bias: Optional[np.ndarray]  # [ts_buckets] float32 or None
    hist_k: List[np.ndarray]       # per user [hist_len[u], D]
    hist_v: List[np.ndarray]       # per user [hist_len[u], D]
    page_table: np.ndarray         # [B, max_pages] int32, -1 = unused

    @property
    def w1t(self) -> np.ndarray:
        """W1 in out-features x in-features layout, [4D, D]."""
        return np.ascontiguousarray(self.w1.T)

    @property
    def w2t(self) -> np.ndarray:
        """W2 in out-features x in-features layout, [D, D]."""
        return np.ascontiguousarray(self.w2.T)


@dataclasses.dataclass
class Workload:
    name: str
    cfg: dict
    seed: int
    B: int
    D: int
    H: int
    d: int
    dtype: str
    layers: int
    page_size: int
    hist_len: np.ndarray           # [B] int32
    new_len: np.ndarray            # [B] int32
    new_offsets: np.ndarray        # [B+1] int32
    miss: np.ndarray               # [B] bool: history absent, full sequence computed
    x0: np.ndarray                 # [T, D] float32
    timestamps: Optional[List[np.ndarray]]  # per user int64 [hist+new]
    max_pages: int
    num_pool_pages: int
    _layer_seqs: list
    _page_perm: np.ndarray
    _layer_cache: dict = dataclasses.field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.new_offsets[-1])

    @property
    def pos_buckets(self) -> int:
        return self.cfg["pos_buckets"]

    @property
    def pos_mbits(self) -> int:
        return self.cfg["pos_mbits"]

    @property
    def ts_buckets(self) -> int:
        return self.cfg["ts_buckets"]

    @property
    def ts_mbits(self) -> int:
        return self.cfg["ts_mbits"]

    @property
    def attn_scale(self) -> float:
        return self.cfg["attn_scale"]

    def pages_per_user(self) -> np.ndarray:
        tot = self.hist_len.astype(np.int64) + self.new_len
        return (tot + self.page_size - 1) // self.page_size

    def ts_offsets(self) -> Optional[np.ndarray]:
        if self.timestamps is None:
            return None
        lens = np.array([len(t) for t in self.timestamps], dtype=np.int64)
        return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)

    def ts_flat(self) -> Optional[np.ndarray]:
        if self.timestamps is None:
            return None
        return np.concatenate(self.timestamps).astype(np.int64)

    def layer(self, l: int) -> LayerInputs:
        if l in self._layer_cache:
            return self._layer_cache[l]
        li = self._make_layer(l)
        self._layer_cache[l] = li
        return li

    def _make_layer(self, l: int) -> LayerInputs:
        D, B = self.D, self.B
        q = round_bf16 if self.dtype == "bf16" else (lambda a: a.astype(np.float32))
        s_w1, s_w2, s_pb, s_tb, s_kv = self._layer_seqs[l].spawn(5)
        w1 = q(np.random.default_rng(s_w1).normal(0.0, W_STD, size=(D, 4 * D)).astype(np.float32))
        w2 = q(np.random.default_rng(s_w2).normal(0.0, W_STD, size=(D, D)).astype(np.float32))
        pos_bias = np.random.default_rng(s_pb).normal(0.0, BIAS_STD, size=self.pos_buckets).astype(np.float32)
        ts_bias = None
        if self.ts_buckets > 0:
            ts_bias = np.random.default_rng(s_tb).normal(0.0, BIAS_STD, size=self.ts_buckets).astype(np.float32)
        rng_kv = np.random.default_rng(s_kv)
        hist_k, hist_v = [], []
        for u in range(B):
            c = int(self.hist_len[u])
            hk = rng_kv.normal(HIST_KV_MEAN, HIST_KV_STD, size=(c, D)).astype(np.float32)
            hv = rng_kv.normal(HIST_KV_MEAN, HIST_KV_STD, size=(c, D)).astype(np.float32)
            hist_k.append(q(hk))
            hist_v.append(q(hv))
        # Page ids: the seeded pool permutation, taken in order per
        # (layer, user, page index).  Layers never share a page.
        npu = self.pages_per_user()
        per_layer = int(npu.sum())
        base = l * per_layer
        pt = np.full((B, self.max_pages), -1, dtype=np.int32)
        pos = base
        for u in range(B):
            k = int(npu[u])
            pt[u, :k] = self._page_perm[pos:pos + k]
            pos += k
        return LayerInputs(w1=w1, w2=w2, pos_bias=pos_bias, ts_bias=ts_bias,
                           hist_k=hist_k, hist_v=hist_v, page_table=pt)


def make_workload(name: str, seed: int = 0, **over) -> Workload:
    """Draw workload `name` (a key of CONFIGS) from `seed`.  Keyword overrides replace
    entries of the workload table (e.g. B=3, hist=("uniform", 40, 90),
    layers=1, pool_pages=4096, max_pages=...) so that tests can run the same
    distributions at sizes the oracle finishes quickly."""
    cfg = dict(CONFIGS[name])
    max_pages_over = over.pop("max_pages", None)
    for k, v in over.items():
        if k not in cfg:
            raise KeyError(f"unknown workload field {k}")
        cfg[k] = v
    B, D, H, d = cfg["B"], cfg["D"], cfg["H"], cfg["d"]
    assert D == H * d
    ss = np.random.SeedSequence([cfg["stream"], seed])
    s_len, s_x, s_ts, s_miss, s_pages, s_layers = ss.spawn(6)
    rng_len = np.random.default_rng(s_len)
    hist = _draw_lengths(rng_len, cfg["hist"], B)
    new = _draw_lengths(rng_len, cfg["new"], B)
    miss = np.zeros(B, dtype=bool)
    if cfg["miss_frac"] > 0:
        k = int(round(cfg["miss_frac"] * B))
        sel = np.random.default_rng(s_miss).permutation(B)[:k]
        miss[sel] = True
        # A miss user's history is absent: its whole sequence is processed
        # as new tokens and appended.
        new = np.where(miss, hist + new, new).astype(np.int32)
        hist = np.where(miss, 0, hist).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(new.astype(np.int64))]).astype(np.int32)
    T = int(offsets[-1])
    xq = round_bf16 if cfg["dtype"] == "bf16" else (lambda a: a.astype(np.float32))
    x0 = xq(np.random.default_rng(s_x).normal(0.0, X_STD, size=(T, D)).astype(np.float32))
    timestamps = None
    if cfg["ts_buckets"] > 0:
        rng_ts = np.random.default_rng(s_ts)
        timestamps = []
        for u in range(B):
            L = int(hist[u]) + int(new[u])
            gaps = 1 + np.floor(rng_ts.exponential(TS_GAP_MEAN, size=L)).astype(np.int64)
            gaps[0] = 0
            timestamps.append(np.cumsum(gaps).astype(np.int64))
    ps = cfg["page_size"]
    npu = (hist.astype(np.int64) + new + ps - 1) // ps
    max_pages = int(max_pages_over) if max_pages_over is not None else max(1, int(npu.max()) if B else 1)
    assert max_pages >= (int(npu.max()) if B else 0)
    need = cfg["layers"] * int(npu.sum())
    if cfg["pool_pages"] is None:
        P = max(need, 1)
        perm = np.arange(P, dtype=np.int32)
    else:
        P = int(cfg["pool_pages"])
        if need > P:
            raise ValueError(f"pool of {P} pages too small for {need} pages")
        perm = np.random.default_rng(s_pages).permutation(P).astype(np.int32)
    return Workload(name=name, cfg=cfg, seed=seed, B=B, D=D, H=H, d=d,
                    dtype=cfg["dtype"], layers=cfg["layers"], page_size=ps,
                    hist_len=hist, new_len=new, new_offsets=offsets, miss=miss,
                    x0=x0, timestamps=timestamps, max_pages=max_pages,
                    num_pool_pages=P, _layer_seqs=s_layers.spawn(cfg["layers"]),
                    _page_perm=perm)


def expected_sizes(name: str) -> dict:
    """Closed-form expected lengths of a workload (for documentation only)."""
    cfg = CONFIGS[name]

    def mean(spec):
        if spec[0] == "const":
            return float(spec[1])
        if spec[0] == "fixed":
            return float(np.mean(spec[1]))
        if spec[0] == "uniform":
            return (spec[1] + spec[2]) / 2.0
        return math.nan
    return dict(hist=mean(cfg["hist"]), new=mean(cfg["new"]), B=cfg["B"])
