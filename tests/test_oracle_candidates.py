"""Pins of the oracle's candidate rule and input preprocessing.

Candidate rule (oracle.layer step 7, a reading): a candidate row sees every
key before the first candidate and itself.  The pins do not restate that
mask; they check what it implies:
  * one candidate at the end is the plain causal layer (nothing to hide);
  * with a distance-independent position bias, a candidate's output equals
    the last row of the plain causal layer run on the history and the other
    new rows followed by that candidate alone (timestamps travel with it);
  * rows before the candidates do not change when the candidates are dropped;
  * a candidate's output does not move when another candidate's input does;
  * the scalar brute force and the padded-dense formulation agree with it.
Preprocessing: a hand-worked fixture pins the row order, the tables used and
the positions.
"""
import json
import os

import numpy as np
import pytest

from oracle import brute, layer, preprocess
from test_oracle import EPS, rel_err, small_case

HERE = os.path.dirname(__file__)


def _const_bias(kw):
    kw = dict(kw)
    kw["pos_bias"] = np.full_like(np.asarray(kw["pos_bias"], np.float64), 0.37)
    return kw


def _user_rows(kw, u):
    off = np.concatenate([[0], np.cumsum(kw["new_len"])])
    return int(off[u]), int(off[u + 1])


def _single_user(kw, u, rows, ts=None):
    """The case of user u alone with the given new-row indices (global)."""
    out = dict(kw)
    out["x"] = np.asarray(kw["x"])[rows]
    out["new_len"] = np.array([len(rows)])
    out["hist_len"] = np.array([kw["hist_len"][u]])
    out["hist_k"] = [kw["hist_k"][u]]
    out["hist_v"] = [kw["hist_v"][u]]
    if "timestamps" in kw:
        out["timestamps"] = [ts]
    return out


@pytest.mark.parametrize("ts", [False, True])
def test_candidates_brute_and_padded_agree(ts):
    news, hists = (0, 1, 5, 6, 3), (0, 3, 7, 2, 0)
    kw = small_case(3, B=5, news=news, hists=hists, ts=ts)
    m = np.array([0, 1, 3, 6, 2])
    y = layer.layer_forward(**kw, num_candidates=m)["y"]
    yb = np.array(brute.layer_brute(**kw, num_candidates=m))
    yp = layer.layer_forward_padded(**kw, num_candidates=m)
    assert rel_err(y, yb) < 1e-12
    assert rel_err(y, yp) < 1e-12
    # and they differ from the causal layer where a candidate has company
    yc = layer.layer_forward(**kw)["y"]
    r0, r1 = _user_rows(kw, 2)
    assert rel_err(y[r1 - 1], yc[r1 - 1]) > 1e-3


def test_one_candidate_is_causal_and_zero_is_none():
    kw = small_case(4, B=3, news=(4, 1, 6), hists=(5, 0, 3), ts=True)
    yc = layer.layer_forward(**kw)["y"]
    y0 = layer.layer_forward(**kw, num_candidates=[0, 0, 0])["y"]
    y1 = layer.layer_forward(**kw, num_candidates=[1, 1, 1])["y"]
    assert np.array_equal(y0, yc)
    assert rel_err(y1, yc) < 1e-14


@pytest.mark.parametrize("ts", [False, True])
def test_candidate_equals_alone_after_history(ts):
    news, hists, m = (7, 5, 3), (6, 0, 11), (3, 5, 2)
    kw = _const_bias(small_case(5, B=3, news=news, hists=hists, ts=ts))
    y = layer.layer_forward(**kw, num_candidates=m)["y"]
    for u in range(3):
        r0, r1 = _user_rows(kw, u)
        cs_row = r1 - m[u]
        c = int(hists[u])
        for i in range(m[u]):
            row = cs_row + i
            rows = list(range(r0, cs_row)) + [row]
            tsu = None
            if ts:
                full = np.asarray(kw["timestamps"][u])
                tsu = np.concatenate([full[:c + cs_row - r0], full[c + row - r0:c + row - r0 + 1]])
            alone = layer.layer_forward(**_single_user(kw, u, rows, tsu))["y"]
            assert rel_err(y[row], alone[-1]) < 1e-12, (u, i)


def test_rows_before_candidates_ignore_them():
    news, hists, m = (7, 5, 3), (6, 0, 11), (3, 2, 3)
    kw = small_case(6, B=3, news=news, hists=hists)
    y = layer.layer_forward(**kw, num_candidates=m)["y"]
    for u in range(3):
        r0, r1 = _user_rows(kw, u)
        rows = list(range(r0, r1 - m[u]))
        if not rows:
            continue
        pre = layer.layer_forward(**_single_user(kw, u, rows))["y"]
        assert rel_err(y[rows], pre) < 1e-12


def test_candidate_independent_of_other_candidates():
    news, hists, m = (6, 4), (9, 2), (4, 3)
    kw = small_case(7, B=2, news=news, hists=hists)
    y = layer.layer_forward(**kw, num_candidates=m)["y"]
    rng = np.random.default_rng(1)
    for u in range(2):
        r0, r1 = _user_rows(kw, u)
        for i in range(m[u]):
            row = r1 - m[u] + i
            kw2 = dict(kw)
            x2 = np.array(kw["x"], copy=True)
            others = [r for r in range(r1 - m[u], r1) if r != row]
            x2[others] = rng.normal(0, 3, size=(len(others), x2.shape[1]))
            kw2["x"] = x2
            y2 = layer.layer_forward(**kw2, num_candidates=m)["y"]
            assert rel_err(y2[row], y[row]) < 1e-13
            if others:
                assert rel_err(y2[others], y[others]) > 1e-3


def test_candidate_stack_equals_alone():
    """Through three layers: each layer's candidate rows read only history
    and non-candidate rows, so the whole stack scores a candidate as if it
    alone followed them."""
    rng = np.random.default_rng(8)
    D, H, L = 8, 2, 3
    news, hists, m = np.array([5, 4]), np.array([3, 6]), np.array([3, 4])
    T = int(news.sum())
    x0 = rng.normal(0, 1, size=(T, D))
    layers = []
    for _ in range(L):
        layers.append(dict(w1=rng.normal(0, 0.3, size=(D, 4 * D)), w2=rng.normal(0, 0.3, size=(D, D)),
                           pos_bias=np.full(16, -0.2),
                           hist_k=[rng.normal(0, 0.5, size=(int(c), D)) for c in hists],
                           hist_v=[rng.normal(0, 0.5, size=(int(c), D)) for c in hists]))
    ys = layer.stack_forward(x0, news, hists, layers, 1 / 16, EPS, H, 2, num_candidates=m)
    off = np.concatenate([[0], np.cumsum(news)])
    for u in range(2):
        r0, r1 = int(off[u]), int(off[u + 1])
        for i in range(int(m[u])):
            row = r1 - int(m[u]) + i
            rows = list(range(r0, r1 - int(m[u]))) + [row]
            lu = [dict(li, hist_k=[li["hist_k"][u]], hist_v=[li["hist_v"][u]]) for li in layers]
            alone = layer.stack_forward(x0[rows], [len(rows)], [hists[u]], lu, 1 / 16, EPS, H, 2)
            assert rel_err(ys[-1][row], alone[-1][-1]) < 1e-12


# ---- preprocessing ----

def _golden():
    with open(os.path.join(HERE, "golden", "preprocess_tokens.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("variant", ["with_actions", "without_actions"])
def test_preprocess_hand_worked(variant):
    g = _golden()
    t, b = g["tables"], g["batch"]
    acts = b["actions"] if variant == "with_actions" else None
    x, new_len, ncand = preprocess.preprocess(b["hist_len"], b["ctx"], b["items"], acts, b["cands"],
                                              t["item_emb"], t["action_emb"], t["ctx_emb"], t["pos_emb"])
    exp = g[variant]
    assert np.array_equal(x, np.asarray(exp["x"], np.float64))
    assert new_len.tolist() == exp["new_len"]
    assert ncand.tolist() == exp["num_candidates"]


def test_preprocess_sizes_of_the_benchmark_sequence():
    """6 context tokens, 4096 item/action pairs and 100 candidates make the
    8,298-token sequence of the pages' workload."""
    rng = np.random.default_rng(0)
    D = 4
    toks = preprocess.user_tokens(range(6), rng.integers(0, 9, 4096), rng.integers(0, 3, 4096),
                                  rng.integers(0, 9, 100))
    assert len(toks) == 8298
    kinds = [k for k, _ in toks]
    assert kinds[:6] == [preprocess.CONTEXT] * 6
    assert kinds[6:8198:2] == [preprocess.ITEM] * 4096 and kinds[7:8198:2] == [preprocess.ACTION] * 4096
    assert kinds[8198:] == [preprocess.ITEM] * 100
    del D
