"""KV commit after acceptance — TEST INFRASTRUCTURE ONLY (see the package
docstring): the product path never imports this module.

The verify pass appended the keys and values of its T new positions to the
cache, rows ctx .. ctx+T-1 of every (sequence, KV head).  Once acceptance has
chosen what is kept, the cache holds the prefix followed by the accepted
positions only, and the rest is dropped:

* "LLM Primer VI — Chapitre 9 — Décodage spéculatif", §9.1: at the first
  divergence the engine commits to the target's own choice and throws the
  remaining candidates away;
* "Parallel Decoding" glossary, section "Limites du parallel decoding": tree
  attention needs an enlarged KV cache that holds the keys and values of
  every branch — after verification only one branch survives;
* "Décodage spéculatif : comment accélérer de 2 à 3 fois les réponses d'un
  LLM" (mc2informatique.fr), section "Comment fonctionne le décodage
  spéculatif ?", step 3: the validated tokens are kept.

Reading where the pages are silent: position 0 of
the new rows is the root (the last verified token) and is always kept; the
accepted path root = path[0], ..., path[l] (l = accept_len) is moved to rows
ctx .. ctx+l in path order and the cache length becomes ctx + l + 1; rows past
it are left as they are (dropped by the new length).  The emitted token that
ends the step (the correction, or the bonus token) has no key or value yet:
the next pass computes them.  A chain's accepted positions are already rows
ctx .. ctx+k, so its commit moves nothing.

``commit_kv`` is the definition written out: a gather of the path's rows.
"""
from __future__ import annotations

import numpy as np


def commit_kv(k: np.ndarray, v: np.ndarray, ctx: int, accept_len: np.ndarray,
              path: np.ndarray | None = None):
    """Return (k', v', new_len) after committing the accepted path.

    k, v        [B, Hkv, ctx+T, D] (any dtype; copied, not modified)
    accept_len  [B] accepted drafts l (tree: depth of the last accepted node;
                chain: number of accepted drafts)
    path        [B, T] node ids root..l then -1 (tree), or None (chain: the
                identity path 0..l)
    """
    k2, v2 = k.copy(), v.copy()
    B = k.shape[0]
    new_len = np.empty(B, dtype=np.int64)
    for b in range(B):
        l = int(accept_len[b])
        nodes = np.arange(l + 1) if path is None else np.asarray(path[b][: l + 1], dtype=np.int64)
        # every destination row reads its source from the input, so the order
        # of the copies does not matter
        k2[b, :, ctx: ctx + l + 1] = k[b][:, ctx + nodes]
        v2[b, :, ctx: ctx + l + 1] = v[b][:, ctx + nodes]
        new_len[b] = ctx + l + 1
    return k2, v2, new_len
