"""Pins of oracle.commit (KV commit after acceptance) against things other than
itself: the chain closed form (nothing moves), a brute-force walk from the
deepest accepted node up its parents, and the meaning of the committed cache
(a query over it attends to exactly the prefix plus the accepted branch).
"""
import numpy as np

from oracle.accept import tree_accept
from oracle.attention import attend_one
from oracle.commit import commit_kv
from verify_pass_rejection_amd import inputs as I


def _rand_kv(B=3, H=2, ctx=7, T=9, D=4, seed=0):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, H, ctx + T, D))
    v = rng.standard_normal((B, H, ctx + T, D))
    return k, v


def test_chain_commit_moves_nothing():
    k, v = _rand_kv()
    acc = np.array([0, 3, 8])
    k2, v2, n = commit_kv(k, v, 7, acc)
    assert np.array_equal(k2, k) and np.array_equal(v2, v)
    assert list(n) == [7 + 1, 7 + 4, 7 + 9]


def test_identity_path_equals_chain():
    k, v = _rand_kv(seed=1)
    acc = np.array([2, 0, 5])
    path = np.full((3, 9), -1)
    for b, l in enumerate(acc):
        path[b, : l + 1] = np.arange(l + 1)
    a = commit_kv(k, v, 7, acc, path)
    c = commit_kv(k, v, 7, acc)
    for x, y in zip(a, c):
        assert np.array_equal(x, y)


def _branch_brute(parents, leaf):
    """Ancestors-or-self of `leaf`, root first, by walking up the parents."""
    nodes = [leaf]
    while parents[nodes[-1]] >= 0:
        nodes.append(int(parents[nodes[-1]]))
    return nodes[::-1]


def test_tree_commit_against_a_walk_up_the_parents():
    rng = np.random.default_rng(3)
    B, H, ctx, T, D = 4, 2, 5, 12, 3
    k, v = _rand_kv(B, H, ctx, T, D, seed=3)
    parents = np.array([[-1] + [int(rng.integers(0, i)) for i in range(1, T)] for _ in range(B)])
    leaves = [int(rng.integers(0, T)) for _ in range(B)]
    path = np.full((B, T), -1)
    acc = np.zeros(B, dtype=int)
    for b in range(B):
        br = _branch_brute(parents[b], leaves[b])
        path[b, : len(br)] = br
        acc[b] = len(br) - 1
    k2, v2, n = commit_kv(k, v, ctx, acc, path)
    for b in range(B):
        br = _branch_brute(parents[b], leaves[b])
        for h in range(H):
            for i, node in enumerate(br):
                assert np.array_equal(k2[b, h, ctx + i], k[b, h, ctx + node])
                assert np.array_equal(v2[b, h, ctx + i], v[b, h, ctx + node])
            # the prefix and the rows past the new length are untouched
            assert np.array_equal(k2[b, h, :ctx], k[b, h, :ctx])
            assert np.array_equal(k2[b, h, ctx + len(br):], k[b, h, ctx + len(br):])
        assert n[b] == ctx + len(br)


def test_committed_cache_is_prefix_plus_accepted_branch():
    # A tree from the synthetic generator, accepted greedily; a fresh query over
    # the committed cache (its first new_len rows) must equal the same query over
    # the original cache restricted to the prefix and the accepted branch.
    w = I.WORKLOADS["eagle2_tree"].with_(B=2, T=20, Hq=4, Hkv=2, D=8, ctx=11, V=50,
                                         tree_widths=(1, 3, 6, 10), seed=21)
    d = I.make_tree_inputs(w)
    res = tree_accept(d["target_logits"].numpy(), d["tokens"].numpy(), d["parents"].numpy())
    rng = np.random.default_rng(4)
    k = rng.standard_normal((w.B, w.Hkv, w.ctx + w.T, w.D))
    v = rng.standard_normal((w.B, w.Hkv, w.ctx + w.T, w.D))
    k2, v2, n = commit_kv(k, v, w.ctx, res.accept_len, res.path)
    par = d["parents"].numpy()
    for b in range(w.B):
        l = int(res.accept_len[b])
        branch = _branch_brute(par[b], int(res.path[b, l]))
        rows = np.concatenate([np.arange(w.ctx), w.ctx + np.array(branch)])
        for h in range(w.Hkv):
            qv = rng.standard_normal(w.D)
            got = attend_one(qv, k2[b, h, : n[b]], v2[b, h, : n[b]], 0.3)
            want = attend_one(qv, k[b, h, rows], v[b, h, rows], 0.3)
            assert np.allclose(got, want, rtol=0, atol=1e-12)
