"""The verification-overhead α and the speedup model, as closed forms.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"LLM Primer VI — Chapitre 9 — Décodage spéculatif", §9.3 gives the speedup of
one speculation round as the expected number of tokens a round yields divided
by (draft time / decode time + 1 + α·N), where α is the verification overhead
per extra position.  It draws two consequences: the best N is near 6–8 at
per-token acceptance 0.8 and near 10–12 at 0.9, and as acceptance tends to 1 the
speedup tends to 1/α.  §9.1 adds that a verify pass at N = 4 costs about
1.2–1.5 decode steps.

Readings: the expected token count includes the bonus
token drawn from p_N, so with a constant per-token acceptance a it is
1 + a + … + a^N; the draft time is the whole round's drafting time; α is
measured as (T_verify(N) − T_verify(0)) / (N · T_verify(0)).
"""
from __future__ import annotations

import numpy as np


def expected_tokens(a: float, N: int) -> float:
    """E[tokens per round] with constant per-token acceptance a: sum_{k<=N} a^k."""
    return float(sum(a ** k for k in range(N + 1)))


def expected_tokens_rows(betas) -> float:
    """E[tokens per round] with row-wise acceptance probabilities β_i:
    sum over k = 0..N of the product of the first k β's."""
    total, prod = 1.0, 1.0
    for beta in betas:
        prod *= float(beta)
        total += prod
    return total


def speedup(a: float, N: int, alpha: float, draft_ratio: float = 0.0) -> float:
    """Primer §9.3: E[tokens] / (T_draft/T_decode + 1 + α·N)."""
    return expected_tokens(a, N) / (draft_ratio + 1.0 + alpha * N)


def best_n(a: float, alpha: float, draft_ratio: float = 0.0, n_max: int = 64) -> int:
    """The draft length that maximises the §9.3 speedup."""
    values = [speedup(a, n, alpha, draft_ratio) for n in range(n_max + 1)]
    return int(np.argmax(values))


def verify_cost_ratio(alpha: float, N: int) -> float:
    """T_verify(N) / T_verify(0) under the §9.3 cost model: 1 + α·N."""
    return 1.0 + alpha * N


def alpha_from_times(t_verify_n: float, t_verify_0: float, N: int) -> float:
    """Measured α = (T_verify(N) − T_verify(0)) / (N · T_verify(0))."""
    return (t_verify_n - t_verify_0) / (N * t_verify_0)
