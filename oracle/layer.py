"""fp64 numpy oracle of one HSTU layer over jagged per-user sequences with a
cached history prefix, and of a stack of such layers.  TEST INFRASTRUCTURE.

Definition (per layer, all arithmetic in float64 on the exact input values):

 1. Z = SiLU(X W1), SiLU(z) = z / (1 + exp(-z)).  U, V, Q, K are the four
    column blocks of width D, in that order; head h owns columns
    [h*d, (h+1)*d) of each block.  (Projection with SiLU: the layer's
    pointwise-transform step; pages: aitrends.kr 100093 "HSTU sequential
    modelling".  Block order and head layout are readings.)
 2. For user u with c cached history tokens and n new rows, the keys and
    values are [K_hist; K_new] and [V_hist; V_new] in position order
    (NVIDIA blog, "Why serving large sequential recommenders is hard": the
    cached history K/V is reused and only new tokens are computed).
 3. New row t sits at absolute position p = c + t.  For every key position
    j <= p (inclusive causal mask) and head h:
        s = <Q[t,h], K[j,h]> + pos_bias[b(p - j)]  (+ ts_bias[b_ts(ts[p] - ts[j])])
        a = SiLU(s) * attn_scale                     (no softmax)
        O[t,h] = sum_j a * V[j,h]
    (SiLU weighting replacing softmax and the relative attention bias:
    aitrends.kr 100093 "HSTU sequential modelling"; news.bpdata.com "HSTU".)
 4. Nrm = (O - mean) / sqrt(var + eps) over each row's D entries (population
    variance, no affine) -- reading of "row-normalised".
 5. Y = (Nrm * U) W2: elementwise gating before the output projection
    (same sections).
 6. In a stack, X_{l+1} = Y_l (no residual: reading).
 7. Candidates (optional): the last m_u new rows of user u are candidate
    items to be scored.  A candidate at position p attends to every key
    before the first candidate, cs = c + n - m_u, and to itself, not to the
    other candidates; rows before cs keep the plain causal mask.  (The pages
    list candidate items among the sequence's tokens, NVIDIA blog "Why use
    HSTU for generative recommendation", and give the workload's candidate
    count, section "Benchmark setup", but state no mask for them: this
    rule, that each candidate is scored as if it alone followed the
    history, is a reading.)
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from .buckets import bucket_np


def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def layer_norm_rows(o: np.ndarray, eps: float) -> np.ndarray:
    mu = o.mean(axis=1, keepdims=True)
    var = ((o - mu) ** 2).mean(axis=1, keepdims=True)
    return (o - mu) / np.sqrt(var + eps)


def project(x: np.ndarray, w1: np.ndarray):
    """Step 1: returns U, V, Q, K (float64, [T, D] each)."""
    D = w1.shape[0]
    z = silu(np.asarray(x, np.float64) @ np.asarray(w1, np.float64))
    return z[:, 0:D], z[:, D:2 * D], z[:, 2 * D:3 * D], z[:, 3 * D:4 * D]


def attention_user(q_rows: np.ndarray, t_rows: np.ndarray, k_all: np.ndarray,
                   v_all: np.ndarray, c: int, H: int, pos_bias: np.ndarray,
                   pos_mbits: int, attn_scale: float,
                   ts: Optional[np.ndarray] = None,
                   ts_bias: Optional[np.ndarray] = None, ts_mbits: int = 0,
                   q_block: int = 512, cand_start: Optional[int] = None) -> np.ndarray:
    """Step 3 for one user.  q_rows [m, D] are the queries of new rows with
    in-user indices t_rows [m]; k_all / v_all [c+n, D] hold history then new
    keys/values in position order; cand_start is the position of the first
    candidate (step 7; None = no candidates).  Returns the attention output
    [m, D]."""
    m, D = q_rows.shape
    d = D // H
    out = np.zeros((m, D), dtype=np.float64)
    pb = np.asarray(pos_bias, np.float64)
    tb = None if ts_bias is None else np.asarray(ts_bias, np.float64)
    for b0 in range(0, m, q_block):
        b1 = min(m, b0 + q_block)
        p = c + np.asarray(t_rows[b0:b1], dtype=np.int64)          # positions
        L = int(p.max()) + 1                                        # keys 0..max p
        j = np.arange(L, dtype=np.int64)
        delta = p[:, None] - j[None, :]
        keep = delta >= 0                                           # causal, inclusive
        if cand_start is not None:                                  # step 7
            keep &= (j[None, :] < cand_start) | (delta == 0)
        bias = pb[bucket_np(delta, pos_mbits, pb.shape[0])]
        if tb is not None:
            tsd = np.asarray(ts, np.int64)
            dts = tsd[p][:, None] - tsd[j][None, :]
            bias = bias + tb[bucket_np(dts, ts_mbits, tb.shape[0])]
        for h in range(H):
            cols = slice(h * d, (h + 1) * d)
            s = q_rows[b0:b1, cols] @ k_all[:L, cols].T + bias
            a = np.where(keep, silu(s) * attn_scale, 0.0)
            out[b0:b1, cols] = a @ v_all[:L, cols]
    return out


def layer_forward(x, new_len, hist_len, hist_k, hist_v, w1, w2, pos_bias,
                  pos_mbits, attn_scale, eps, H, timestamps=None, ts_bias=None,
                  ts_mbits=0, rows: Optional[Sequence[int]] = None,
                  q_block: int = 512, num_candidates=None) -> dict:
    """One layer over a jagged batch.

    x [T, D] holds the new rows of all users back to back (user u owns rows
    offsets[u] .. offsets[u+1]-1, offsets = prefix sums of new_len).
    hist_k / hist_v: per user [hist_len[u], D] cached history K / V in
    position order.  timestamps: per user int64 [hist_len[u] + new_len[u]]
    (or None).  rows: optional subset of global row indices whose attention
    and output are computed (all K/V are still computed); None = all rows.
    num_candidates: per user count of trailing candidate rows (step 7), or
    None for none.

    Returns float64 arrays: u, v, q, k [T, D]; rows [m]; o, nrm, g, y [m, D]
    (o already includes attn_scale)."""
    x = np.asarray(x, np.float64)
    T, D = x.shape
    new_len = np.asarray(new_len, np.int64)
    hist_len = np.asarray(hist_len, np.int64)
    offsets = np.concatenate([[0], np.cumsum(new_len)])
    assert offsets[-1] == T
    U, V, Q, K = project(x, w1)
    sel = np.arange(T) if rows is None else np.asarray(sorted(rows), dtype=np.int64)
    o = np.zeros((sel.shape[0], D), dtype=np.float64)
    for u in range(new_len.shape[0]):
        r0, r1 = int(offsets[u]), int(offsets[u + 1])
        mask = (sel >= r0) & (sel < r1)
        if not mask.any():
            continue
        c = int(hist_len[u])
        hk = np.asarray(hist_k[u], np.float64).reshape(c, D)
        hv = np.asarray(hist_v[u], np.float64).reshape(c, D)
        k_all = np.vstack([hk, K[r0:r1]])
        v_all = np.vstack([hv, V[r0:r1]])
        ridx = sel[mask]
        cs = None
        if num_candidates is not None:
            m_u = int(num_candidates[u])
            assert 0 <= m_u <= r1 - r0
            cs = c + (r1 - r0) - m_u
        o[mask] = attention_user(
            Q[ridx], ridx - r0, k_all, v_all, c, H, pos_bias, pos_mbits,
            attn_scale, None if timestamps is None else timestamps[u],
            ts_bias, ts_mbits, q_block, cs)
    nrm = layer_norm_rows(o, eps)
    g = nrm * U[sel]
    y = g @ np.asarray(w2, np.float64)
    return dict(u=U, v=V, q=Q, k=K, rows=sel, o=o, nrm=nrm, g=g, y=y)


def layer_forward_padded(x, new_len, hist_len, hist_k, hist_v, w1, w2,
                         pos_bias, pos_mbits, attn_scale, eps, H,
                         timestamps=None, ts_bias=None, ts_mbits=0,
                         num_candidates=None) -> np.ndarray:
    """Same layer computed on a per-user padded dense batch [B, Lmax, D] with
    explicit validity masks (an independent formulation used to pin the
    jagged indexing).  Candidates (step 7) are a per-position flag: a key
    flagged as a candidate is seen only by its own row.  Returns y [T, D] in
    jagged row order."""
    x = np.asarray(x, np.float64)
    T, D = x.shape
    d = D // H
    B = len(new_len)
    new_len = np.asarray(new_len, np.int64)
    hist_len = np.asarray(hist_len, np.int64)
    tot = hist_len + new_len
    Lmax = max(int(tot.max()) if B else 0, 1)
    offsets = np.concatenate([[0], np.cumsum(new_len)])
    U, V, Q, K = project(x, w1)
    Kp = np.zeros((B, Lmax, D))
    Vp = np.zeros((B, Lmax, D))
    Qp = np.zeros((B, Lmax, D))
    valid = np.zeros((B, Lmax), dtype=bool)
    is_new = np.zeros((B, Lmax), dtype=bool)
    is_cand = np.zeros((B, Lmax), dtype=bool)
    tsp = np.zeros((B, Lmax), dtype=np.int64)
    for u in range(B):
        c, n, r0 = int(hist_len[u]), int(new_len[u]), int(offsets[u])
        Kp[u, :c] = np.asarray(hist_k[u], np.float64).reshape(c, D)
        Vp[u, :c] = np.asarray(hist_v[u], np.float64).reshape(c, D)
        Kp[u, c:c + n] = K[r0:r0 + n]
        Vp[u, c:c + n] = V[r0:r0 + n]
        Qp[u, c:c + n] = Q[r0:r0 + n]
        valid[u, :c + n] = True
        is_new[u, c:c + n] = True
        if num_candidates is not None and int(num_candidates[u]) > 0:
            is_cand[u, c + n - int(num_candidates[u]):c + n] = True
        if timestamps is not None:
            tsp[u, :c + n] = timestamps[u]
    pos = np.arange(Lmax)
    delta = pos[:, None] - pos[None, :]                       # [Lq, Lk]
    bias = np.asarray(pos_bias, np.float64)[bucket_np(delta, pos_mbits, len(pos_bias))]
    O = np.zeros((B, Lmax, D))
    for u in range(B):
        bu = bias
        if ts_bias is not None:
            dts = tsp[u][:, None] - tsp[u][None, :]
            bu = bias + np.asarray(ts_bias, np.float64)[bucket_np(dts, ts_mbits, len(ts_bias))]
        m = (delta >= 0) & valid[u][None, :] & is_new[u][:, None]
        m &= ~is_cand[u][None, :] | (delta == 0)
        for h in range(H):
            cols = slice(h * d, (h + 1) * d)
            s = Qp[u][:, cols] @ Kp[u][:, cols].T + bu
            a = np.where(m, silu(s) * attn_scale, 0.0)
            O[u][:, cols] = a @ Vp[u][:, cols]
    o = np.zeros((T, D))
    for u in range(B):
        c, n, r0 = int(hist_len[u]), int(new_len[u]), int(offsets[u])
        o[r0:r0 + n] = O[u, c:c + n]
    return (layer_norm_rows(o, eps) * U) @ np.asarray(w2, np.float64)


def stack_forward(x0, new_len, hist_len, layers: List[dict], attn_scale, eps,
                  H, pos_mbits, timestamps=None, ts_mbits=0,
                  num_candidates=None) -> List[np.ndarray]:
    """A stack of layers, X_{l+1} = Y_l.  layers[l] holds w1, w2, pos_bias,
    ts_bias, hist_k, hist_v.  Returns [Y_0, ..., Y_{L-1}] (float64)."""
    xs = np.asarray(x0, np.float64)
    ys = []
    for li in layers:
        r = layer_forward(xs, new_len, hist_len, li["hist_k"], li["hist_v"],
                          li["w1"], li["w2"], li["pos_bias"], pos_mbits,
                          attn_scale, eps, H, timestamps, li.get("ts_bias"),
                          ts_mbits, num_candidates=num_candidates)
        ys.append(r["y"])
        xs = r["y"]
    return ys
