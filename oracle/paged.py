"""Verify attention over a paged KV cache — TEST INFRASTRUCTURE ONLY (see the
package docstring): the product path never imports this module.

"LLM Primer VI — Chapitre 9 — Décodage spéculatif", closing section "Ce que
prépare le Chapitre 9": paged KV is one of the runtime tools (with batching
and speculative decoding) that a serving engine wires together; the
"Parallel Decoding" glossary, section "Parallel decoding en production",
names vLLM, SGLang and TensorRT-LLM as engines that run speculation.  The
pages give the cache no layout.  Readings:

* the keys and values of every sequence live in fixed-size pages of
  ``page_size`` positions drawn from one shared pool; row j of sequence b's
  block table names the page that holds its positions
  j*page_size .. (j+1)*page_size - 1;
* a page holds all KV heads, laid out either head-major ("hnd":
  [pages, Hkv, page_size, D]) or position-major ("nhd": [pages, page_size,
  Hkv, D]);
* every sequence has a prefix length of its own, ctx_b; its T new positions
  follow the prefix (positions ctx_b .. ctx_b+T-1 of its logical cache), as in
  the contiguous case.

The operation is the contiguous one, unchanged: gather each sequence's logical
cache out of its pages, then apply :func:`oracle.attention.verify_attention`
to that sequence alone.
"""
from __future__ import annotations

import numpy as np

from .attention import verify_attention


def gather_sequence(pages: np.ndarray, table_row, length: int, layout: str) -> np.ndarray:
    """The first ``length`` positions of one sequence's cache, [Hkv, length, D].

    pages: [P, Hkv, ps, D] ("hnd") or [P, ps, Hkv, D] ("nhd").
    Position i sits in page table_row[i // ps] at offset i % ps.
    """
    if layout == "hnd":
        Hkv, ps, D = pages.shape[1], pages.shape[2], pages.shape[3]
    elif layout == "nhd":
        ps, Hkv, D = pages.shape[1], pages.shape[2], pages.shape[3]
    else:
        raise ValueError(f"unknown page layout {layout!r}")
    out = np.empty((Hkv, length, D), dtype=np.float64)
    for i in range(length):
        page, off = int(table_row[i // ps]), i % ps
        if layout == "hnd":
            out[:, i] = pages[page, :, off]
        else:
            out[:, i] = pages[page, off, :]
    return out


def verify_attention_paged(q, k_pages, v_pages, block_table, ctx_lens, parents=None,
                           layout: str = "hnd", scale: float | None = None,
                           rows=None) -> np.ndarray:
    """Masked verify attention of every sequence against its paged cache.

    q           [B, T, Hq, D]
    k_pages, v_pages  page pools in ``layout`` (see the module docstring)
    block_table [B, max_blocks] page ids
    ctx_lens    [B] prefix lengths ctx_b (sequence b's cache has ctx_b + T rows)
    parents     None (chain) or [B, T] as for ``verify_attention``
    rows        optional (b, t, h) triples to compute (others stay NaN)

    Returns O [B, T, Hq, D] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    kp = np.asarray(k_pages, dtype=np.float64)
    vp = np.asarray(v_pages, dtype=np.float64)
    B, T, Hq, D = q.shape
    out = np.full((B, T, Hq, D), np.nan)
    want = None if rows is None else {}
    if rows is not None:
        for (b, t, h) in rows:
            want.setdefault(b, []).append((0, t, h))
    for b in range(B):
        if want is not None and b not in want:
            continue
        ctx = int(ctx_lens[b])
        kb = gather_sequence(kp, block_table[b], ctx + T, layout)[None]
        vb = gather_sequence(vp, block_table[b], ctx + T, layout)[None]
        par = None if parents is None else np.asarray(parents)[b:b + 1]
        sub = None if want is None else want[b]
        out[b] = verify_attention(q[b:b + 1], kb, vb, ctx, parents=par, scale=scale,
                                  rows=sub)[0]
    return out
