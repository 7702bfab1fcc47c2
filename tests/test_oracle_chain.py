"""Pins for oracle.accept.chain_accept against things other than itself.

The pages fix the law, not a listing: "LLM Primer VI — Chapitre 9 — Décodage
spéculatif", §9.1 (keep x with probability min(1, p(x)/q(x)), else draw from the
normalised (p − q)+; the output is distributed as pure target sampling; N + 1
positions, so a bonus token from p_N when all drafts are kept).

* stratified quadrature: with the uniform on an even grid of M points the
  fraction of outcomes equals the stated probability to within 1/M — for the
  ratio test, the residual draw, the bonus draw and the one-hot special cases
  (p and q computed here with scipy.special.softmax);
* N = 0 is inverse-CDF sampling from p_0 (numpy.searchsorted on the cumsum);
* χ² law tests, V = 16, 10^6 trials: the first emitted token follows p_0, also
  against 10^6 pure target draws (two-sample); the second follows p_1;
* exact enumeration on V = 3, N = 2: the law of (accepted length, emitted
  tokens) is prod_{i<k} min(p_i, q_i)(x_i) · (p_k − q_k)+(y) for k < N and
  prod_{i<N} min(p_i, q_i)(x_i) · p_N(y) for k = N; Monte Carlo of the oracle is
  χ²-tested against it, and E[tokens per round] against sum_k prod_{i<k} β_i.
"""
import itertools

import numpy as np
from scipy import stats
from scipy.special import softmax as sp_softmax

from oracle.accept import chain_accept
from oracle.model import expected_tokens_rows

CHI2_999_DF15 = 37.697   # scipy.stats.chi2.ppf(0.999, 15)


def grid(M):
    return (np.arange(M) + 0.5) / M


def uniform24(rng, shape):
    return rng.integers(1, 1 << 24, size=shape) / float(1 << 24)


def logits(rng, B, rows, V, sd=2.0):
    return rng.normal(0.0, sd, size=(B, rows, V))


def test_ratio_test_quadrature():
    rng = np.random.default_rng(1)
    V, M = 8, 4096
    zp = logits(rng, 1, 2, V)
    zq = zp[:, :1] + rng.normal(0, 1.0, size=(1, 1, V))
    p = sp_softmax(zp[0, 0]); q = sp_softmax(zq[0, 0])
    for x in range(V):
        res = chain_accept(np.repeat(zp, M, 0), np.repeat(zq, M, 0),
                           np.full((M, 1), x), grid(M)[:, None], np.full((M, 2), 0.5))
        frac = np.mean(res.num_accepted == 1)
        assert abs(frac - min(1.0, p[x] / q[x])) <= 1.0 / M
        kept = res.num_accepted == 1
        assert np.all(res.out_tokens[kept, 0] == x)


def test_residual_draw_quadrature():
    rng = np.random.default_rng(2)
    V, M = 12, 8192
    zp = logits(rng, 1, 2, V)
    zq = zp[:, :1] + rng.normal(0, 1.5, size=(1, 1, V))
    p = sp_softmax(zp[0, 0]); q = sp_softmax(zq[0, 0])
    x = int(np.argmax(q / p))                 # a token with p(x) < q(x)
    assert p[x] / q[x] < 0.99
    res = chain_accept(np.repeat(zp, M, 0), np.repeat(zq, M, 0), np.full((M, 1), x),
                       np.full((M, 1), 1 - 2.0 ** -24),
                       np.stack([grid(M), np.full(M, 0.5)], axis=1))
    assert np.all(res.num_accepted == 0)
    assert np.all(res.out_tokens[:, 1] == -1)
    w = np.maximum(p - q, 0)
    freq = np.bincount(res.out_tokens[:, 0], minlength=V) / M
    np.testing.assert_allclose(freq, w / w.sum(), atol=1.0 / M)


def test_bonus_draw_when_all_drafts_agree():
    rng = np.random.default_rng(3)
    V, N, M = 10, 3, 4096
    zp = logits(rng, 1, N + 1, V)
    zq = zp[:, :N].copy()                      # q = p: every ratio is exactly 1
    drafts = rng.integers(0, V, size=(M, N))
    ud = np.concatenate([np.full((M, N), 0.5), grid(M)[:, None]], axis=1)
    res = chain_accept(np.repeat(zp, M, 0), np.repeat(zq, M, 0), drafts,
                       uniform24(rng, (M, N)), ud)
    assert np.all(res.num_accepted == N)
    np.testing.assert_array_equal(res.out_tokens[:, :N], drafts)
    freq = np.bincount(res.out_tokens[:, N], minlength=V) / M
    np.testing.assert_allclose(freq, sp_softmax(zp[0, N]), atol=1.0 / M)


def test_zero_drafts_is_inverse_cdf_sampling():
    rng = np.random.default_rng(4)
    B, V = 2000, 37
    zp = logits(rng, B, 1, V)
    u = uniform24(rng, (B, 1))
    res = chain_accept(zp, np.zeros((B, 0, V)), np.zeros((B, 0), int), np.zeros((B, 0)), u)
    assert np.all(res.num_accepted == 0)
    for b in range(B):
        p = sp_softmax(zp[b, 0])
        c = np.cumsum(p)
        assert res.out_tokens[b, 0] == np.searchsorted(c, u[b, 0] * c[-1], side="right")


def test_one_hot_draft_distribution():
    """q one-hot at x: keep iff u < p(x); the residual is p without x, renormalised."""
    rng = np.random.default_rng(5)
    V, M, x = 9, 4096, 4
    zp = logits(rng, 1, 2, V)
    zq = np.full((1, 1, V), -np.inf); zq[0, 0, x] = 0.0
    p = sp_softmax(zp[0, 0])
    res = chain_accept(np.repeat(zp, M, 0), np.repeat(zq, M, 0), np.full((M, 1), x),
                       grid(M)[:, None], np.full((M, 2), 0.5))
    assert abs(np.mean(res.num_accepted == 1) - p[x]) <= 1.0 / M
    res = chain_accept(np.repeat(zp, M, 0), np.repeat(zq, M, 0), np.full((M, 1), x),
                       np.full((M, 1), 1 - 2.0 ** -24),
                       np.stack([grid(M), np.full(M, 0.5)], axis=1))
    assert np.all(res.num_accepted == 0)
    want = p.copy(); want[x] = 0; want /= want.sum()
    freq = np.bincount(res.out_tokens[:, 0], minlength=V) / M
    np.testing.assert_allclose(freq, want, atol=1.0 / M)


def test_one_hot_target_forces_its_token():
    rng = np.random.default_rng(6)
    B, N, V, ystar = 500, 3, 11, 7
    zp = np.full((B, N + 1, V), -np.inf); zp[:, :, ystar] = 1.0
    zq = logits(rng, B, N, V)
    drafts = rng.integers(0, V, size=(B, N))
    res = chain_accept(zp, zq, drafts, uniform24(rng, (B, N)), uniform24(rng, (B, N + 1)))
    for b in range(B):
        k = res.num_accepted[b]
        assert np.all(drafts[b, :k] == ystar)
        assert res.out_tokens[b, k] == ystar


def _mc(zp, zq, B, rng):
    N, V = zq.shape[1], zq.shape[2]
    q = sp_softmax(zq[0], axis=-1)
    drafts = np.stack([rng.choice(V, size=B, p=q[i]) for i in range(N)], axis=1)
    return chain_accept(np.broadcast_to(zp, (B,) + zp.shape[1:]),
                        np.broadcast_to(zq, (B,) + zq.shape[1:]), drafts,
                        uniform24(rng, (B, N)), uniform24(rng, (B, N + 1)))


def test_output_law_is_the_target_chi2():
    rng = np.random.default_rng(7)
    V, N, B = 16, 2, 1_000_000
    zp = logits(rng, 1, N + 1, V)
    zq = zp[:, :N] + rng.normal(0, 1.0, size=(1, N, V))
    res = _mc(zp, zq, B, rng)
    p0, p1 = sp_softmax(zp[0, 0]), sp_softmax(zp[0, 1])
    first = np.bincount(res.out_tokens[:, 0], minlength=V)
    assert stats.chisquare(first, B * p0).statistic < CHI2_999_DF15
    pure = np.bincount(rng.choice(V, size=B, p=p0), minlength=V)
    two = np.sum((first - pure) ** 2 / (first + pure))     # two-sample χ², equal sizes
    assert two < CHI2_999_DF15
    second = res.out_tokens[res.num_accepted >= 1, 1]
    obs = np.bincount(second, minlength=V)
    assert stats.chisquare(obs, obs.sum() * p1).statistic < CHI2_999_DF15


def exact_law(zp, zq):
    """Closed-form law of (k, emitted tokens) for fixed rows."""
    N, V = zq.shape[1], zq.shape[2]
    p = sp_softmax(zp[0], axis=-1); q = sp_softmax(zq[0], axis=-1)
    law = {}
    for k in range(N + 1):
        for xs in itertools.product(range(V), repeat=k):
            pre = np.prod([min(p[i, xs[i]], q[i, xs[i]]) for i in range(k)])
            last = np.maximum(p[k] - q[k], 0) if k < N else p[N]
            for y in range(V):
                law[(k,) + xs + (y,)] = pre * last[y]
    return law, p, q


def test_exact_enumeration_of_the_output_law():
    rng = np.random.default_rng(8)
    V, N, B = 3, 2, 400_000
    zp = logits(rng, 1, N + 1, V, sd=1.0)
    zq = zp[:, :N] + rng.normal(0, 1.0, size=(1, N, V))
    law, p, q = exact_law(zp, zq)
    assert abs(sum(law.values()) - 1) < 1e-12
    first = np.zeros(V)
    for key, pr in law.items():
        first[key[1]] += pr
    np.testing.assert_allclose(first, p[0], atol=1e-12)   # law preservation

    res = _mc(zp, zq, B, rng)
    keys = list(law)
    index = {kk: i for i, kk in enumerate(keys)}
    counts = np.zeros(len(keys))
    for b in range(B):
        k = int(res.num_accepted[b])
        counts[index[(k,) + tuple(int(t) for t in res.out_tokens[b, :k + 1])]] += 1
    expected = np.array([law[kk] for kk in keys]) * B
    assert np.all(counts[expected == 0] == 0)     # impossible outcomes never occur
    big = expected >= 5
    small = ~big & (expected > 0)
    obs, exp = counts[big], expected[big]
    if small.any():
        obs = np.append(obs, counts[small].sum())
        exp = np.append(exp, expected[small].sum())
    chi = np.sum((obs - exp) ** 2 / exp)
    assert chi < stats.chi2.ppf(0.999, len(obs) - 1)

    betas = [np.minimum(p[i], q[i]).sum() for i in range(N)]
    pk = [np.prod(betas[:k]) * (1 - betas[k]) for k in range(N)] + [np.prod(betas)]
    hist = np.bincount(res.num_accepted, minlength=N + 1) / B
    np.testing.assert_allclose(hist, pk, atol=5 * np.sqrt(0.25 / B))
    mean_tokens = np.mean(res.num_accepted + 1)
    se = np.std(res.num_accepted + 1) / np.sqrt(B)
    assert abs(mean_tokens - expected_tokens_rows(betas)) < 5 * se


def test_invalid_draft_token_is_rejected():
    rng = np.random.default_rng(9)
    zp = logits(rng, 2, 2, 5)
    zq = logits(rng, 2, 1, 5)
    res = chain_accept(zp, zq, np.array([[-1], [5]]), np.array([[1e-6], [1e-6]]),
                       np.array([[0.5, 0.5], [0.5, 0.5]]))
    assert np.all(res.num_accepted == 0)


def test_near_boundary_flag():
    zp = np.log(np.array([[[0.25, 0.75], [0.5, 0.5]]]))
    zq = np.log(np.array([[[0.5, 0.5]]]))
    # r = 0.25 / 0.5 = 0.5: a u within 1e-5 relative of it is flagged
    res = chain_accept(zp, zq, np.array([[0]]), np.array([[0.5 * (1 + 1e-6)]]),
                       np.array([[0.3, 0.3]]))
    assert res.near_boundary[0]
    res = chain_accept(zp, zq, np.array([[0]]), np.array([[0.4]]), np.array([[0.3, 0.3]]))
    assert not res.near_boundary[0]
    # the bonus draw from [0.5, 0.5] has its CDF boundary at 0.5
    res = chain_accept(zp, zq, np.array([[1]]), np.array([[0.1]]), np.array([[0.3, 0.5]]))
    assert res.num_accepted[0] == 1 and res.near_boundary[0]
