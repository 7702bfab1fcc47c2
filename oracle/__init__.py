"""CPU oracle for the speculative-decoding verify step — TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 numpy code written from the pages' description of the
target model's verification pass.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the product path
(``verify_pass_rejection_amd`` and its HIP library) never does, and the two
share no code.

Sources, cited by page title and section (no code is printed on the pages):

* "LLM Primer VI — Chapitre 9 — Décodage spéculatif" (actionbridge.io),
  §9.1 (the verification pass and the acceptance rule), §9.2 (EAGLE-2 draft
  trees checked under a custom mask), §9.3 (the α / speedup model).
* "Parallel Decoding" glossary entry (polydesk.ai), section "Medusa" with its
  "Tree attention" paragraph, and section "L'attention en arbre : la brique
  commune" (tree mask, root = last verified token, longest accepted path).
* "Décodage spéculatif : comment accélérer de 2 à 3 fois les réponses d'un
  LLM" (mc2informatique.fr), section "Comment fonctionne le décodage
  spéculatif ?", steps 2–3 (check the drafts in one pass; on a rejection,
  resume from that position with the target).

Modules:

* :mod:`oracle.attention` — masked verify attention by its plain definition.
* :mod:`oracle.accept`    — chain rejection sampling and greedy tree acceptance.
* :mod:`oracle.model`     — the α / expected-tokens / speedup closed forms.
* :mod:`oracle.commit`    — the KV commit of the accepted path (a gather).
* :mod:`oracle.paged`     — verify attention over a paged KV cache (a gather
  of each sequence's pages, then :mod:`oracle.attention`).
* :mod:`oracle.ngram`     — n-gram (prompt-lookup) draft proposal, a search
  from the longest n-gram and the latest position down.

Parity status: every function here is pinned by ``-m "not gpu"`` tests against
something other than itself (a library routine, a closed form, brute force,
stratified quadrature or a χ² law test); none is "parity unpinned".
"""
