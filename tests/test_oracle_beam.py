"""Pins of the beam-decode attention oracle (oracle.beam).

* Against torch's scaled_dot_product_attention (float64, CPU) run on each
  beam's materialised key sequence -- the per-beam copy of the context that
  the shared layout avoids -- with the query heads' KV heads repeated.
* Path semantics: a BeamKV slot on no beam's path changes nothing; changing
  a slot on a path changes exactly the beams that descend from it.
* Closed forms: one key gives its value; equal values give that value;
  query heads sharing a KV head and a query give equal outputs; far-apart
  scores give the value of the best key (hard max), without overflow.
"""
import numpy as np
import pytest
import torch

from oracle.beam import beam_decode_attention, beam_keys


def case(seed, R=2, W=5, Hq=4, Hkv=2, d=16, ctx=(7, 0), t=2, S=4):
    rng = np.random.default_rng(seed)
    q = rng.normal(0, 1, size=(R, W, Hq, d))
    ctx_k = [rng.normal(0, 1, size=(c, Hkv, d)) for c in ctx]
    ctx_v = [rng.normal(0, 1, size=(c, Hkv, d)) for c in ctx]
    bk = rng.normal(0, 1, size=(R, S, W, Hkv, d))
    bv = rng.normal(0, 1, size=(R, S, W, Hkv, d))
    path = rng.integers(0, W, size=(R, W, t))
    return dict(q=q, ctx_k=ctx_k, ctx_v=ctx_v, beam_k=bk, beam_v=bv, path=path, t=t, scale=d ** -0.5)


@pytest.mark.parametrize("seed,t,ctx", [(0, 0, (5, 3)), (1, 1, (0, 9)), (2, 2, (7, 0)), (3, 3, (12, 4))])
def test_matches_sdpa_on_materialised_sequences(seed, t, ctx):
    kw = case(seed, t=t, ctx=ctx)
    out = beam_decode_attention(**kw)
    R, W, Hq, d = kw["q"].shape
    G = Hq // kw["beam_k"].shape[3]
    for r in range(R):
        for w in range(W):
            K = torch.from_numpy(beam_keys(kw["ctx_k"], kw["beam_k"], kw["path"], r, w, t))
            V = torch.from_numpy(beam_keys(kw["ctx_v"], kw["beam_v"], kw["path"], r, w, t))
            k = K.permute(1, 0, 2).repeat_interleave(G, dim=0)[None]       # [1, Hq, L, d]
            v = V.permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
            qq = torch.from_numpy(kw["q"][r, w])[None, :, None, :]         # [1, Hq, 1, d]
            ref = torch.nn.functional.scaled_dot_product_attention(qq, k, v, scale=kw["scale"])
            assert np.max(np.abs(ref[0, :, 0, :].numpy() - out[r, w])) < 1e-12


def test_path_slots_select_the_ancestors():
    kw = case(4, R=1, W=3, t=2, ctx=(6,))
    kw["path"] = np.array([[[1, 0], [1, 2], [0, 0]]])
    base = beam_decode_attention(**kw)
    # step 0 slot 2 and step 1 slot 1 lie on no path
    for s, slot in [(0, 2), (1, 1)]:
        bk = kw["beam_k"].copy()
        bv = kw["beam_v"].copy()
        bk[0, s, slot] += 5.0
        bv[0, s, slot] -= 3.0
        assert np.array_equal(beam_decode_attention(**dict(kw, beam_k=bk, beam_v=bv)), base)
    # step 1 slot 0 is on the paths of beams 0 and 2 only
    bv = kw["beam_v"].copy()
    bv[0, 1, 0] += 2.0
    moved = np.abs(beam_decode_attention(**dict(kw, beam_v=bv)) - base).max(axis=(2, 3))[0]
    assert moved[0] > 1e-6 and moved[2] > 1e-6 and moved[1] == 0.0
    # the current step's key is the beam's own slot
    bv = kw["beam_v"].copy()
    bv[0, 2, 1] += 2.0
    moved = np.abs(beam_decode_attention(**dict(kw, beam_v=bv)) - base).max(axis=(2, 3))[0]
    assert moved[1] > 1e-6 and moved[0] == 0.0 and moved[2] == 0.0


def test_closed_forms():
    kw = case(5, R=1, W=2, t=0, ctx=(0,))
    out = beam_decode_attention(**kw)                      # a single key: its value
    G = 2
    for w in range(2):
        for h in range(4):
            assert np.allclose(out[0, w, h], kw["beam_v"][0, 0, w, h // G], atol=1e-15)
    kw = case(6, R=1, W=3, t=2, ctx=(9,))
    c = np.linspace(-1, 1, 16)
    kw["ctx_v"] = [np.broadcast_to(c, kw["ctx_v"][0].shape).copy()]
    kw["beam_v"] = np.broadcast_to(c, kw["beam_v"].shape).copy()
    assert np.allclose(beam_decode_attention(**kw), c, atol=1e-14)


def test_grouped_heads_and_hard_max():
    kw = case(7, R=1, W=2, t=1, ctx=(10,))
    q = kw["q"].copy()
    q[:, :, 1] = q[:, :, 0]                              # heads 0 and 1 share KV head 0
    out = beam_decode_attention(**dict(kw, q=q))
    assert np.array_equal(out[:, :, 0], out[:, :, 1])
    q[:, :, 2] = q[:, :, 0]                              # head 2 reads KV head 1
    assert np.abs(beam_decode_attention(**dict(kw, q=q))[:, :, 2] - out[:, :, 0]).max() > 1e-3
    # huge scores: the output is the value of the best key, with no overflow
    big = dict(kw, q=kw["q"] * 1e4)
    out = beam_decode_attention(**big)
    assert np.all(np.isfinite(out))
    K = beam_keys(kw["ctx_k"], kw["beam_k"], kw["path"], 0, 1, 1)
    V = beam_keys(kw["ctx_v"], kw["beam_v"], kw["path"], 0, 1, 1)
    j = int(np.argmax(K[:, 0, :] @ kw["q"][0, 1, 0]))
    assert np.allclose(out[0, 1, 0], V[j, 0], atol=1e-9)
