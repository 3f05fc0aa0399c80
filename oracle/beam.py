"""Reference of the beam-decode attention of Semantic-ID generative
recommendation over a shared context KV.  TEST INFRASTRUCTURE.

Pages: the Korean summary of the recsys-examples article (section on the
GR inference path) and the Hungarian article news.bpdata.com (section
"SID-GR inference"): a Semantic-ID request has a long user context (often
thousands of tokens), decodes only 2-3 Semantic-ID tokens, with wide beams
(128 or 256); the serving path keeps one request-level ContextKV shared by
every beam instead of copying it per beam, a short per-beam BeamKV for the
decoded tokens, and BeamPath bookkeeping of each beam's ancestry, and its
decode attention works on that layout directly.

The pages state no formula.  Readings (the plainest that the rest supports,
for a decoder built on a standard Qwen-style model):
  * attention is the usual scaled-dot-product softmax attention with grouped
    query heads: query head h reads KV head h // (Hq // Hkv);
  * at decode step t (0-based) beam w of request r holds one query token;
    its keys are the request's whole context (shared, ctx_len[r] tokens),
    then the BeamKV tokens on its path, one per earlier step s < t, taken
    from beam slot path[r, w, s] of step s, then its own token of step t
    (slot w of step t);
  * the context carries no mask beyond its length; the softmax runs over
    all ctx_len[r] + t + 1 keys.

Arrays: q [R, W, Hq, d]; ctx_k / ctx_v per request [c_r, Hkv, d];
beam_k / beam_v [R, S, W, Hkv, d] (S >= t + 1 steps); path [R, W, t].
"""
from __future__ import annotations

import numpy as np


def beam_keys(ctx_k, beam_k, path, r: int, w: int, t: int):
    """Key (or value) rows of beam w of request r at step t, in order:
    context, path tokens of steps 0..t-1, its own token of step t.
    Returns [ctx_len + t + 1, Hkv, d]."""
    rows = [np.asarray(ctx_k[r], np.float64)]
    for s in range(t):
        rows.append(np.asarray(beam_k[r, s, int(path[r, w, s])], np.float64)[None])
    rows.append(np.asarray(beam_k[r, t, w], np.float64)[None])
    return np.concatenate(rows, axis=0)


def beam_decode_attention(q, ctx_k, ctx_v, beam_k, beam_v, path, t: int, scale: float):
    """out [R, W, Hq, d] (float64)."""
    q = np.asarray(q, np.float64)
    R, W, Hq, d = q.shape
    Hkv = np.asarray(beam_k).shape[3]
    G = Hq // Hkv
    out = np.zeros_like(q)
    for r in range(R):
        for w in range(W):
            K = beam_keys(ctx_k, beam_k, path, r, w, t)
            V = beam_keys(ctx_v, beam_v, path, r, w, t)
            for h in range(Hq):
                g = h // G
                s = (K[:, g, :] @ q[r, w, h]) * scale
                p = np.exp(s - s.max())
                p /= p.sum()
                out[r, w, h] = p @ V[:, g, :]
    return out
