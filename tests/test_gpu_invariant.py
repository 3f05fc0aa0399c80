"""GPU tests of batch-invariant calls (desc flag FLAG_BATCH_INVARIANT).

With the flag every row a call produces is bit-identical whatever else is in
the batch and however the user's sequence was split into calls.  The cache
reuse of the NVIDIA blog's "Benefits" section (cached K/V reused, only the
new tokens computed) then gives exactly the rows of a full recompute:

* a two-layer stack over seven ragged users (one of them empty), recomputed in one call, against
  the same users fed in three incremental calls (history read from the
  pool, users with no rows in a call, a different batch in every call), for
  bf16 with and without the timestamp term and fp32: every row of every
  layer equal bit for bit;
* the same users one at a time against the batched call, bit for bit;
* the invariant call against the oracle (layer 0), to the usual tolerance.

The two runs of each comparison use pools of their own (different fill), so
no stale pool value can make them agree by accident.
"""
import numpy as np
import pytest
import torch

from gpu_util import EPS, tol_check, to_np
from hstu_jagged_silu_fwd_amd.stack import HSTUStack
from oracle import layer as olayer

pytestmark = pytest.mark.gpu

CASES = {
    "bf16-d128-ts": dict(dtype="bf16", H=2, d=128, ps=32, nb=64, mbits=3, tsb=32, tsm=2),
    "bf16-d64": dict(dtype="bf16", H=4, d=64, ps=64, nb=64, mbits=3, tsb=0, tsm=0),
    "f32-d32": dict(dtype="f32", H=2, d=32, ps=16, nb=32, mbits=2, tsb=0, tsm=0),
}
# Total positions per user.  The whole batch (4,402 rows) takes the large-M
# projection tiles and, without timestamps, the 8-wave attention layout; the
# incremental calls and single users take smaller tiles and, where a call
# has at most 96 new rows per user, the 16-wave layout, so the comparisons
# also hold across those forms.
LENS = np.array([700, 40, 1300, 257, 5, 0, 2100], np.int64)
CUTS = [np.array([300, 40, 513, 0, 2, 0, 1000]),              # rows [cut_{k-1}, cut_k) in call k
        np.array([650, 40, 1290, 256, 5, 0, 2050]),
        LENS]
NL = 2


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).cpu().numpy()


class Setup:
    """Seeded weights, inputs, timestamps and page tables of one case."""

    def __init__(self, c, seed=7):
        self.c = c
        self.B = len(LENS)
        self.D = c["H"] * c["d"]
        self.maxP = int((LENS.max() + c["ps"] - 1) // c["ps"]) + 1
        self.P = NL * self.B * self.maxP + 3           # the layers share one pool, on pages of their own
        rng = np.random.default_rng(seed)
        tq = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
        q = lambda a: torch.from_numpy(np.asarray(a, np.float32)).to(tq).float().numpy()
        D = self.D
        self.w1 = [q(rng.normal(0, 0.02, (D, 4 * D))) for _ in range(NL)]
        self.w2 = [q(rng.normal(0, 0.02, (D, D))) for _ in range(NL)]
        self.pb = [rng.normal(0, 0.1, c["nb"]).astype(np.float32) for _ in range(NL)]
        self.tb = [rng.normal(0, 0.1, c["tsb"]).astype(np.float32) for _ in range(NL)] if c["tsb"] else None
        pages = rng.permutation(self.P)[:NL * self.B * self.maxP].reshape(NL, self.B, self.maxP)
        self.pt = [pages[l].astype(np.int32) for l in range(NL)]
        self.x = [q(rng.normal(0, 1, (int(L), D))) for L in LENS]
        self.ts = [np.cumsum(1 + rng.integers(0, 9, int(L))).astype(np.int64) for L in LENS]

    def stack(self, fill):
        c = self.c
        st = HSTUStack(num_users=self.B, num_heads=c["H"], head_dim=c["d"], page_size=c["ps"],
                       num_pool_pages=self.P, max_pages_per_user=self.maxP, pos_buckets=c["nb"],
                       pos_mbits=c["mbits"], attn_scale=1.0 / float(LENS.max()), norm_eps=EPS,
                       dtype=c["dtype"], ts_buckets=c["tsb"], ts_mbits=c["tsm"], num_layers=NL,
                       pool_fill=fill, batch_invariant=True)
        for l in range(NL):
            st.set_layer(l, w1t=self.w1[l].T, w2t=self.w2[l].T, pos_bias=self.pb[l], page_table=self.pt[l],
                         ts_bias=None if self.tb is None else self.tb[l])
        return st

    def call(self, st, users, lo, hi):
        """Stack forward over rows [lo[u], hi[u]) of `users`, in that order
        (history lo[u]; page-table rows taken in the same order); returns
        every layer's output as raw bits, the outputs, and the row offsets."""
        x = np.concatenate([self.x[u][lo[u]:hi[u]] for u in users]).reshape(-1, self.D)
        n = np.array([hi[u] - lo[u] for u in users], np.int64)
        off = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        hist = np.array([lo[u] for u in users], np.int32)
        ts = tso = None
        if self.tb is not None:
            ts = np.concatenate([self.ts[u][:hi[u]] for u in users]).astype(np.int64)
            tso = np.concatenate([[0], np.cumsum([hi[u] for u in users])]).astype(np.int32)
        pts = [p[users] for p in self.pt]
        outs = st.forward(x, off, hist, timestamps=ts, ts_offsets=tso, return_all=True, page_tables=pts)
        assert st.read_status() == 0
        return [bits(o) for o in outs], outs, off


@pytest.mark.parametrize("case", list(CASES))
def test_invariant_cached_equals_full_recompute_bit_exact(case):
    print(f"case invariant cached == recompute {case}", flush=True)
    s = Setup(CASES[case])
    users = list(range(s.B))
    zero = np.zeros(s.B, np.int64)
    full, _, off_full = s.call(s.stack(0.0), users, zero, LENS)
    st = s.stack(5.0)
    got = [[None] * s.B for _ in range(NL)]
    lo = zero
    for k, hi in enumerate(CUTS):
        # a different batch each call: the users in another order, and users
        # with nothing new left out of the middle call
        order = users[::-1] if k == 1 else users
        if k == 1:
            order = [u for u in order if hi[u] > lo[u]]
        part, _, off = s.call(st, order, lo, hi)
        for l in range(NL):
            for j, u in enumerate(order):
                r = part[l][off[j]:off[j + 1]]
                got[l][u] = r if got[l][u] is None else np.concatenate([got[l][u], r])
        lo = hi
    for l in range(NL):
        for u in users:
            want = full[l][off_full[u]:off_full[u + 1]]
            have = got[l][u] if got[l][u] is not None else want[:0]
            assert have.shape == want.shape, (l, u)
            nd = int(np.count_nonzero(have != want))
            assert nd == 0, f"layer {l} user {u}: {nd} elements differ"


@pytest.mark.parametrize("case", list(CASES))
def test_invariant_batched_equals_one_user_at_a_time_bit_exact(case):
    print(f"case invariant batched == per user {case}", flush=True)
    s = Setup(CASES[case], seed=8)
    zero = np.zeros(s.B, np.int64)
    users = list(range(s.B))
    full, _, off_full = s.call(s.stack(0.0), users, zero, LENS)
    st1 = s.stack(-3.0)
    for u in users:
        if LENS[u] == 0:
            continue
        one, _, _ = s.call(st1, [u], zero, LENS)
        for l in range(NL):
            nd = int(np.count_nonzero(one[l] != full[l][off_full[u]:off_full[u + 1]]))
            assert nd == 0, f"layer {l} user {u}: {nd} elements differ"


@pytest.mark.parametrize("case", list(CASES))
def test_invariant_call_matches_the_oracle(case):
    print(f"case invariant vs oracle {case}", flush=True)
    c = CASES[case]
    s = Setup(c, seed=9)
    users = list(range(s.B))
    zero = np.zeros(s.B, np.int64)
    _, outs, _ = s.call(s.stack(0.0), users, zero, LENS)
    x = np.concatenate(s.x).reshape(-1, s.D)
    empty = [np.zeros((0, s.D))] * s.B
    ref = olayer.layer_forward(x, LENS, zero, empty, empty, s.w1[0], s.w2[0], s.pb[0], c["mbits"],
                               1.0 / float(LENS.max()), EPS, c["H"],
                               timestamps=s.ts if s.tb is not None else None,
                               ts_bias=None if s.tb is None else s.tb[0], ts_mbits=c["tsm"])
    tol_check(to_np(outs[0]), ref["y"], c["dtype"], f"invariant layer 0 {case}")
