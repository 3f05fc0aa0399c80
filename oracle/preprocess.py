"""Reference of the input preprocessing that builds a layer's rows from
categorical tokens.  TEST INFRASTRUCTURE.

The NVIDIA blog "Deploying an HSTU generative recommender with NVIDIA
Dynamo-Triton", section "Why use HSTU for generative recommendation", says
the ranking model's inputs are categorical tokens (context tokens for the
user side, item tokens, optional action tokens for the user's interaction
with each item), and that preprocessing looks the tokens' embeddings up,
interleaves item and action embeddings when action tokens are present,
appends the context and applies a positional encoding.  Its section
"Benchmark setup" sizes one sequence as history item/action pairs, up to
100 candidates and 6 context features.

Readings (the pages give no formula):
  * every token is one row: a history pair is two rows, the item's then the
    action's (without action tokens, one item row per history entry);
  * a user's new rows are its context tokens first, then its history
    entries, then its candidate items (the candidates last, where the
    candidate mask of oracle.layer expects them); a user whose context is
    already cached sends no context tokens;
  * row t of a user with c cached tokens sits at position p = c + t, and its
    input is   x = E[token] + pos_emb[p]   with one embedding table per token
    kind (context, item, action; candidates are items) and a learned position
    table (the positional encoding read as an added learned embedding).
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

CONTEXT, ITEM, ACTION = 0, 1, 2


def user_tokens(ctx_ids: Sequence[int], item_ids: Sequence[int],
                action_ids: Optional[Sequence[int]],
                cand_ids: Sequence[int]) -> List[Tuple[int, int]]:
    """The (kind, id) of one user's new rows in order."""
    toks = [(CONTEXT, int(i)) for i in ctx_ids]
    if action_ids is None:
        toks += [(ITEM, int(i)) for i in item_ids]
    else:
        assert len(action_ids) == len(item_ids)
        for it, ac in zip(item_ids, action_ids):
            toks.append((ITEM, int(it)))
            toks.append((ACTION, int(ac)))
    toks += [(ITEM, int(i)) for i in cand_ids]
    return toks


def preprocess(hist_len: Sequence[int], ctx: Sequence[Sequence[int]],
               items: Sequence[Sequence[int]],
               actions: Optional[Sequence[Sequence[int]]],
               cands: Sequence[Sequence[int]], item_emb, action_emb, ctx_emb,
               pos_emb):
    """A batch of users (lists indexed by user).  Returns x [T, D] float64
    (sums of the exact table values), new_len [B] and num_candidates [B]."""
    tables = {CONTEXT: np.asarray(ctx_emb, np.float64),
              ITEM: np.asarray(item_emb, np.float64),
              ACTION: None if action_emb is None else np.asarray(action_emb, np.float64)}
    pos = np.asarray(pos_emb, np.float64)
    D = pos.shape[1]
    rows, new_len, ncand = [], [], []
    for u in range(len(hist_len)):
        toks = user_tokens(ctx[u], items[u], None if actions is None else actions[u], cands[u])
        for t, (kind, i) in enumerate(toks):
            p = int(hist_len[u]) + t
            rows.append(tables[kind][i] + pos[p])
        new_len.append(len(toks))
        ncand.append(len(cands[u]))
    x = np.asarray(rows, np.float64).reshape(len(rows), D)
    return x, np.asarray(new_len, np.int64), np.asarray(ncand, np.int64)
