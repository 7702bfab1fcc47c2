"""Pins for oracle.accept.tree_accept_sampled against things other than itself.

The pages fix the law, not a multi-candidate listing ("LLM Primer VI —
Chapitre 9 — Décodage spéculatif", §9.1: the rule keeps the output distributed
as the target's own sampling; §9.2: the target picks among several draft
paths).  Pins:

* a tree in which every node has one child is a chain: the result equals
  ``chain_accept`` (pinned on its own) on the same rows and uniforms;
* χ² law tests: with the children of a node drawn independently from its q,
  the first emitted token follows p_root, and the token after an accepted
  node a follows p_a, for several candidates per node;
* special cases: q = p keeps the first child every time; a one-hot p is the
  only token ever emitted; an invalid token is never kept; a leaf root is
  inverse-CDF sampling from p_root (numpy.searchsorted);
* malformed parents: such a node is never visited.
"""
import numpy as np
from scipy import stats
from scipy.special import softmax as sp_softmax

from oracle.accept import chain_accept, tree_accept_sampled


def _uniforms(rng, shape):
    return rng.integers(1, 1 << 24, size=shape) / float(1 << 24)


def test_single_child_tree_is_the_chain():
    rng = np.random.default_rng(1)
    B, N, V = 40, 6, 12
    zp = rng.normal(0, 2.0, (B, N + 1, V))
    zq = zp[:, :N] + rng.normal(0, 1.0, (B, N, V))
    x = np.array([[rng.choice(V, p=sp_softmax(zq[b, i])) for i in range(N)] for b in range(B)])
    ua, ud = _uniforms(rng, (B, N)), _uniforms(rng, (B, N + 1))
    ch = chain_accept(zp, zq, x, ua, ud)
    # tree: node i+1 carries draft i; node n's draft row is the chain's row n
    T = N + 1
    parents = np.tile(np.arange(-1, N), (B, 1))
    tok = np.concatenate([np.zeros((B, 1), dtype=np.int64), x], axis=1)
    zq_t = np.concatenate([zq, rng.normal(0, 1.0, (B, 1, V))], axis=1)   # leaf row: unused
    ua_t = np.concatenate([np.full((B, 1), 0.5), ua], axis=1)
    tr = tree_accept_sampled(zp, zq_t, tok, parents, ua_t, ud)
    ok = ~(ch.near_boundary | tr.near_boundary)
    assert ok.sum() >= B - 2
    assert np.array_equal(tr.accept_len[ok], ch.num_accepted[ok])
    assert np.array_equal(tr.out_tokens[ok], ch.out_tokens[ok])
    for b in np.flatnonzero(ok):
        k = ch.num_accepted[b]
        assert list(tr.path[b, :k + 1]) == list(range(k + 1))
        assert np.all(tr.path[b, k + 1:] == -1)


def _law_trials(rng, zp, zq, parents, trials):
    """Fresh candidate draws (each node's children from its parent's q) and
    fresh uniforms in every trial; p/q logits shared by all trials."""
    T, V = zp.shape
    q = sp_softmax(zq, axis=-1)
    tok = np.zeros((trials, T), dtype=np.int64)
    for i in range(1, T):
        tok[:, i] = rng.choice(V, size=trials, p=q[parents[i]])
    zp_b = np.broadcast_to(zp, (trials, T, V))
    zq_b = np.broadcast_to(zq, (trials, T, V))
    par_b = np.broadcast_to(parents, (trials, T))
    return tree_accept_sampled(zp_b, zq_b, tok, par_b, _uniforms(rng, (trials, T)),
                               _uniforms(rng, (trials, T)))


def test_several_candidates_keep_the_target_law_chi2():
    rng = np.random.default_rng(2)
    V = 6
    # root with three children; children 1 and 2 with two leaf children each
    parents = np.array([-1, 0, 0, 0, 1, 1, 2, 2])
    T = len(parents)
    zp = rng.normal(0, 1.5, (T, V))
    zq = rng.normal(0, 1.5, (T, V))                       # far from p: many rejections
    p = sp_softmax(zp, axis=-1)
    trials = 100000
    r = _law_trials(rng, zp, zq, parents, trials)
    first = np.bincount(r.out_tokens[:, 0], minlength=V)
    crit = stats.chi2.ppf(0.999, V - 1)
    assert stats.chisquare(first, trials * p[0]).statistic < crit
    # the token after an accepted node a follows p_a
    for a in (1, 2):
        sel = r.path[:, 1] == a
        assert sel.sum() > 3000
        second = np.bincount(r.out_tokens[sel, 1], minlength=V)
        assert stats.chisquare(second, sel.sum() * p[a]).statistic < crit
    # the candidates matter: several are rejected and later ones kept
    assert np.mean(r.path[:, 1] == 3) > 0.02


def test_q_equal_to_p_keeps_the_first_child():
    rng = np.random.default_rng(3)
    B, V = 20, 9
    parents = np.tile(np.array([-1, 0, 0, 1, 1, 3]), (B, 1))
    T = parents.shape[1]
    z = rng.normal(0, 2.0, (B, T, V))
    tok = rng.integers(0, V, (B, T))
    r = tree_accept_sampled(z, z, tok, parents, _uniforms(rng, (B, T)), _uniforms(rng, (B, T)))
    for b in range(B):
        assert list(r.path[b, :4]) == [0, 1, 3, 5]
        assert r.accept_len[b] == 3


def test_one_hot_target_is_the_only_token_emitted():
    rng = np.random.default_rng(4)
    B, V, y = 30, 7, 5
    parents = np.tile(np.array([-1, 0, 0, 0]), (B, 1))
    zp = np.full((B, 4, V), -1e4)
    zp[:, :, y] = 0.0
    zq = rng.normal(0, 1.0, (B, 4, V))
    tok = rng.integers(0, V, (B, 4))
    r = tree_accept_sampled(zp, zq, tok, parents, _uniforms(rng, (B, 4)), _uniforms(rng, (B, 4)))
    for b in range(B):
        kids = [i for i in (1, 2, 3) if tok[b, i] == y]
        if kids:                       # the first child carrying y is kept
            assert r.path[b, 1] == kids[0] and r.out_tokens[b, 0] == y
        else:                          # every child rejected: the residual is one-hot on y
            assert r.accept_len[b] == 0 and r.out_tokens[b, 0] == y


def test_invalid_token_is_never_kept_and_leaf_root_is_inverse_cdf():
    rng = np.random.default_rng(5)
    B, V = 16, 10
    zp = rng.normal(0, 1.0, (B, 3, V))
    zq = zp.copy()                                 # a valid token would always be kept
    tok = np.tile(np.array([0, -1, V]), (B, 1))    # both children invalid
    parents = np.tile(np.array([-1, 0, 0]), (B, 1))
    ud = _uniforms(rng, (B, 3))
    r = tree_accept_sampled(zp, zq, tok, parents, _uniforms(rng, (B, 3)), ud)
    assert np.all(r.accept_len == 0)
    # q = p and two rejections: (p - q)+ sums to zero, which falls back to p
    p = sp_softmax(zp[:, 0], axis=-1)
    want = [np.searchsorted(np.cumsum(p[b]), ud[b, 0] * np.cumsum(p[b])[-1], side="right")
            for b in range(B)]
    assert list(r.out_tokens[:, 0]) == want
    # a root without children: plain inverse-CDF sampling from p_root
    leaf = tree_accept_sampled(zp[:, :1], zq[:, :1], tok[:, :1], parents[:, :1],
                               _uniforms(rng, (B, 1)), ud[:, :1])
    assert list(leaf.out_tokens[:, 0]) == want and np.all(leaf.path[:, 1:] == -1)


def test_malformed_parent_is_never_visited():
    rng = np.random.default_rng(6)
    B, V = 10, 8
    z = rng.normal(0, 1.0, (B, 4, V))
    tok = rng.integers(0, V, (B, 4))
    parents = np.tile(np.array([-1, 0, 3, 2]), (B, 1))   # node 2 points forward
    r = tree_accept_sampled(z, z, tok, parents, _uniforms(rng, (B, 4)), _uniforms(rng, (B, 4)))
    assert np.all(r.path[:, :2] == [0, 1]) and np.all(r.path[:, 2:] == -1)
