"""n-gram (prompt-lookup) draft proposal — TEST INFRASTRUCTURE ONLY (see the
package docstring): the product path never imports this module.

"LLM Primer VI — Chapitre 9 — Décodage spéculatif", section "Pourquoi ce
chapitre existe": n-gram and suffix drafting are among the draft algorithms
the chapter covers; §9.3: the largest speedups are measured on highly
repetitive loads.  "Parallel Decoding" glossary, section "Parallel decoding en
production": TensorRT-LLM offers prompt lookup among its draft techniques.
The pages give no rule.  Reading (the plainest form of prompt lookup):

* the draft for a sequence comes from its own context c[0..L-1] (token ids);
* for n = n_max down to n_min, the last n tokens c[L-n..L-1] are searched
  for among the earlier n-grams c[e-n+1..e] with e <= L-2 (so that at least
  one token follows the occurrence); the first n with an occurrence wins;
* among its occurrences the most recent (largest e) is taken;
* the drafts are the tokens that followed it, c[e+1 .. min(e+N, L-1)]: up to
  N, fewer when the context ends first; no occurrence gives no draft.

``ngram_propose`` is that rule written out as a search from the longest n-gram
and the latest position down.
"""
from __future__ import annotations

import numpy as np


def ngram_propose(context, lengths, N: int, n_min: int, n_max: int):
    """Drafts for every sequence.

    context [B, L] token ids (positions >= lengths[b] ignored); lengths [B].
    Returns (num_drafts [B] int32, drafts [B, N] int32 padded with -1,
    match_end [B] int64, -1 without an occurrence).
    """
    ctx = np.asarray(context, dtype=np.int64)
    B = ctx.shape[0]
    num = np.zeros(B, dtype=np.int32)
    drafts = np.full((B, N), -1, dtype=np.int32)
    ends = np.full(B, -1, dtype=np.int64)
    for b in range(B):
        L = int(lengths[b])
        c = ctx[b, :L]
        found = None
        for n in range(n_max, n_min - 1, -1):
            if n > L - 1:
                continue                  # no earlier n-gram can end before L-1
            suffix = c[L - n:]
            for e in range(L - 2, n - 2, -1):
                if np.array_equal(c[e - n + 1: e + 1], suffix):
                    found = e
                    break
            if found is not None:
                break
        if found is None or N == 0:
            ends[b] = -1 if found is None else found
            continue
        cont = c[found + 1: min(found + N, L - 1) + 1]
        num[b] = len(cont)
        drafts[b, :len(cont)] = cont
        ends[b] = found
    return num, drafts, ends
