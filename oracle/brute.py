"""Scalar pure-Python brute force of the same layer, for tiny shapes only.
TEST INFRASTRUCTURE.  Every sum is an explicit loop over Python floats; it
shares nothing with oracle.layer except the bucket rule's scalar form.

Follows the definition stated in oracle.layer (pages: aitrends.kr 100093
"HSTU sequential modelling"; NVIDIA blog "Deploying an HSTU generative
recommender with NVIDIA Dynamo-Triton", "Why serving large sequential
recommenders is hard").
"""
from __future__ import annotations

import math

from .buckets import bucket


def _silu(z: float) -> float:
    if z < -700.0:
        return 0.0
    return z / (1.0 + math.exp(-z))


def layer_brute(x, new_len, hist_len, hist_k, hist_v, w1, w2, pos_bias,
                pos_mbits, attn_scale, eps, H, timestamps=None, ts_bias=None,
                ts_mbits=0, num_candidates=None):
    """Arguments as oracle.layer.layer_forward (nested lists or arrays).
    With num_candidates, row t of user u is a candidate when t >= n - m_u;
    a candidate skips the keys of every other candidate.
    Returns y as a list of rows (Python floats)."""
    T = len(x)
    D = len(w1)
    d = D // H
    z = [[0.0] * (4 * D) for _ in range(T)]
    for r in range(T):
        for col in range(4 * D):
            acc = 0.0
            for kk in range(D):
                acc += float(x[r][kk]) * float(w1[kk][col])
            z[r][col] = _silu(acc)
    Ublk = [row[0:D] for row in z]
    Vblk = [row[D:2 * D] for row in z]
    Qblk = [row[2 * D:3 * D] for row in z]
    Kblk = [row[3 * D:4 * D] for row in z]
    y = []
    r0 = 0
    for u in range(len(new_len)):
        c, n = int(hist_len[u]), int(new_len[u])
        keys = [[float(v) for v in hist_k[u][j]] for j in range(c)] + [Kblk[r0 + t] for t in range(n)]
        vals = [[float(v) for v in hist_v[u][j]] for j in range(c)] + [Vblk[r0 + t] for t in range(n)]
        m_u = 0 if num_candidates is None else int(num_candidates[u])
        for t in range(n):
            p = c + t
            o = [0.0] * D
            for h in range(H):
                for j in range(p + 1):
                    if t >= n - m_u and j >= c + n - m_u and j != p:
                        continue                    # another candidate's key
                    s = 0.0
                    for e in range(h * d, (h + 1) * d):
                        s += Qblk[r0 + t][e] * keys[j][e]
                    s += float(pos_bias[bucket(p - j, pos_mbits, len(pos_bias))])
                    if ts_bias is not None:
                        dt = int(timestamps[u][p]) - int(timestamps[u][j])
                        s += float(ts_bias[bucket(dt, ts_mbits, len(ts_bias))])
                    a = _silu(s) * attn_scale
                    for e in range(h * d, (h + 1) * d):
                        o[e] += a * vals[j][e]
            mu = sum(o) / D
            var = sum((v - mu) ** 2 for v in o) / D
            inv = 1.0 / math.sqrt(var + eps)
            g = [(o[e] - mu) * inv * Ublk[r0 + t][e] for e in range(D)]
            row = []
            for col in range(D):
                acc = 0.0
                for e in range(D):
                    acc += g[e] * float(w2[e][col])
                row.append(acc)
            y.append(row)
        r0 += n
    return y
