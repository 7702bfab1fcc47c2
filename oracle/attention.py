"""Verify-pass attention by its plain definition, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What is computed
----------------
"LLM Primer VI — Chapitre 9 — Décodage spéculatif", §9.1: the target runs a
single forward pass over the accepted prefix followed by the draft positions,
and because a transformer pass is parallel over positions it yields a
next-token distribution at every one of those positions.  Inside that pass each
draft position attends to the whole prefix and to the draft positions it
conditions on.  For a linear chain those are the earlier draft positions
(ordinary causal attention).  For a draft tree ("Parallel Decoding" glossary,
"Medusa" → "Tree attention", and "L'attention en arbre : la brique commune";
Primer §9.2 on EAGLE-2) a node conditions on its ancestors only, and the
attention mask encodes the tree.

Readings where the pages are silent:

* scale defaults to 1/sqrt(D) (scaled dot-product attention);
* Q and K arrive already position-encoded: no rotary step here;
* the K/V rows of the T new positions are appended after the ctx prefix rows
  before the call (the glossary's "Limites" section notes that tree attention
  needs an enlarged KV cache for the branches);
* grouped-query attention maps query head h to KV head h // (Hq // Hkv);
* every query sees at least itself, so no softmax row is empty.
"""
from __future__ import annotations

import numpy as np


def visible_tail_positions(parents, T: int) -> list[list[int]]:
    """For each draft position i, the draft positions whose keys it may see.

    A node sees itself and all of its ancestors (walked up through
    ``parents``).  ``parents=None`` is the linear chain, where position i
    sees every position 0..i.
    """
    if parents is None:
        return [list(range(i + 1)) for i in range(T)]
    out = []
    for i in range(T):
        seen = [i]
        j = int(parents[i])
        while j >= 0:
            seen.append(j)
            j = int(parents[j])
        out.append(sorted(seen))
    return out


def attend_one(qvec: np.ndarray, keys: np.ndarray, values: np.ndarray,
               scale: float) -> np.ndarray:
    """softmax(scale · keys·q) · values for one query over its visible keys."""
    s = (keys @ qvec) * scale
    s = s - s.max()
    e = np.exp(s)
    return (e / e.sum()) @ values


def visible_key_rows(ctx: int, tail_positions: list[int]) -> np.ndarray:
    """Row indices into the [ctx + T] key axis: the prefix, then the tail."""
    return np.concatenate([np.arange(ctx, dtype=np.int64),
                           ctx + np.asarray(tail_positions, dtype=np.int64)])


def verify_attention(q, k, v, ctx: int, parents=None, scale: float | None = None,
                     rows=None) -> np.ndarray:
    """Masked attention of the T draft positions against prefix + drafts.

    q:  [B, T, Hq, D]; k, v: [B, Hkv, ctx + T, D] (any real dtype; widened to
    float64, which is exact for fp32 and bf16 data).
    parents: None for a chain, else [B, T] ints, parents[b][0] == -1 and
    parents[b][i] < i.
    rows: optional list of (b, t, h) triples; when given only those outputs
    are computed (the others stay NaN) — used for sampled checks at full size.

    Returns O [B, T, Hq, D] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, Hq, D = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0 and k.shape[2] == ctx + T and v.shape == k.shape
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.full((B, T, Hq, D), np.nan)
    if rows is None:
        rows = [(b, t, h) for b in range(B) for t in range(T) for h in range(Hq)]
    vis_cache: dict = {}
    for (b, t, h) in rows:
        if b not in vis_cache:
            vis_cache[b] = visible_tail_positions(
                None if parents is None else parents[b], T)
        idx = visible_key_rows(ctx, vis_cache[b][t])
        kv = h // G
        out[b, t, h] = attend_one(q[b, t, h], k[b, kv][idx], v[b, kv][idx], scale)
    return out
