"""Pins for oracle.attention against things other than itself.

* torch's CPU scaled_dot_product_attention (a library routine) in float64, with
  the boolean mask built independently as the transitive closure of the parent
  relation (repeated boolean matrix products), GQA by repeat_interleave;
* a tree equals each root→leaf branch run as its own causal chain over the
  prefix plus that branch's K/V ("Parallel Decoding" glossary, "L'attention en
  arbre": every branch is a continuation, all checked in one masked pass);
* T = 1 is the ordinary single-query decode step (Primer ch. 9, §9.1: the
  pass over N + 1 positions; N = 0 is plain decoding);
* closed forms: Q = 0 averages the visible V rows; constant V rows return
  that constant.
"""
import numpy as np
import pytest
import torch

from oracle.attention import verify_attention


def random_tree(T, rng):
    return [-1] + [int(rng.integers(0, i)) for i in range(1, T)]


def closure_mask(parents, T):
    """Ancestor-or-self matrix via boolean powers of (I + A), A[i, parent(i)] = 1."""
    a = torch.eye(T, dtype=torch.float64)
    for i, p in enumerate(parents):
        if p >= 0:
            a[i, p] = 1.0
    reach = a.clone()
    for _ in range(T):
        reach = ((reach @ a) > 0).double()
    return reach > 0


def sdpa_reference(q, k, v, ctx, parents_per_b, scale):
    B, T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, T, Hq, D))
    for b in range(B):
        if parents_per_b is None:
            tail = torch.tril(torch.ones(T, T, dtype=torch.bool))
        else:
            tail = closure_mask(parents_per_b[b], T)
        mask = torch.cat([torch.ones(T, ctx, dtype=torch.bool), tail], dim=1)
        qb = torch.from_numpy(q[b]).permute(1, 0, 2)                 # [Hq, T, D]
        kb = torch.from_numpy(k[b]).repeat_interleave(G, dim=0)      # [Hq, L, D]
        vb = torch.from_numpy(v[b]).repeat_interleave(G, dim=0)
        o = torch.nn.functional.scaled_dot_product_attention(
            qb, kb, vb, attn_mask=mask, scale=scale)
        out[b] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("tree", [False, True])
@pytest.mark.parametrize("B,T,Hq,Hkv,D,ctx", [(2, 5, 4, 2, 16, 7), (1, 9, 6, 3, 8, 0),
                                             (3, 1, 2, 1, 4, 11), (1, 17, 8, 8, 32, 33)])
def test_matches_library_sdpa(tree, B, T, Hq, Hkv, D, ctx):
    rng = np.random.default_rng(B * 100 + T)
    q = rng.normal(size=(B, T, Hq, D))
    k = rng.normal(size=(B, Hkv, ctx + T, D))
    v = rng.normal(size=(B, Hkv, ctx + T, D))
    parents = [random_tree(T, rng) for _ in range(B)] if tree else None
    scale = 0.37
    got = verify_attention(q, k, v, ctx, parents=parents, scale=scale)
    want = sdpa_reference(q, k, v, ctx, parents, scale)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_default_scale_is_inverse_sqrt_d():
    rng = np.random.default_rng(3)
    q = rng.normal(size=(1, 3, 2, 16))
    k = rng.normal(size=(1, 2, 8, 16))
    v = rng.normal(size=(1, 2, 8, 16))
    got = verify_attention(q, k, v, 5)
    want = sdpa_reference(q, k, v, 5, None, None)     # torch's default: 1/sqrt(D)
    np.testing.assert_allclose(got, want, atol=1e-12)


def test_tree_equals_each_branch_as_a_causal_chain():
    rng = np.random.default_rng(7)
    T, Hq, Hkv, D, ctx = 12, 4, 2, 8, 9
    parents = random_tree(T, rng)
    q = rng.normal(size=(1, T, Hq, D))
    k = rng.normal(size=(1, Hkv, ctx + T, D))
    v = rng.normal(size=(1, Hkv, ctx + T, D))
    tree_out = verify_attention(q, k, v, ctx, parents=[parents])
    leaves = [i for i in range(T) if i not in parents]
    assert len(leaves) >= 2
    for leaf in leaves:
        branch = []
        n = leaf
        while n >= 0:
            branch.append(n)
            n = parents[n]
        branch.reverse()
        rows = list(range(ctx)) + [ctx + n for n in branch]
        chain_out = verify_attention(q[:, branch], k[:, :, rows], v[:, :, rows], ctx)
        np.testing.assert_array_equal(chain_out[0], tree_out[0, branch])


def test_chain_is_a_tree_with_consecutive_parents():
    rng = np.random.default_rng(8)
    T = 6
    q = rng.normal(size=(2, T, 4, 8))
    k = rng.normal(size=(2, 2, 10 + T, 8))
    v = rng.normal(size=(2, 2, 10 + T, 8))
    chain = verify_attention(q, k, v, 10)
    tree = verify_attention(q, k, v, 10, parents=[[-1] + list(range(T - 1))] * 2)
    np.testing.assert_array_equal(chain, tree)


def test_single_position_is_a_plain_decode_step():
    rng = np.random.default_rng(9)
    q = rng.normal(size=(2, 1, 8, 32))
    k = rng.normal(size=(2, 2, 41, 32))
    v = rng.normal(size=(2, 2, 41, 32))
    got = verify_attention(q, k, v, 40)
    for b in range(2):
        for h in range(8):
            o = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b, :, h]), torch.from_numpy(k[b, h // 4]),
                torch.from_numpy(v[b, h // 4]))
            np.testing.assert_allclose(got[b, 0, h], o[0].numpy(), atol=1e-12)


def test_zero_query_averages_the_visible_rows():
    rng = np.random.default_rng(10)
    T, ctx = 7, 5
    parents = [-1, 0, 0, 1, 1, 3, 2]
    q = np.zeros((1, T, 2, 4))
    k = rng.normal(size=(1, 1, ctx + T, 4))
    v = rng.normal(size=(1, 1, ctx + T, 4))
    got = verify_attention(q, k, v, ctx, parents=[parents])
    # visible tail rows written out by hand for this tree
    anc = {0: [0], 1: [0, 1], 2: [0, 2], 3: [0, 1, 3], 4: [0, 1, 4],
           5: [0, 1, 3, 5], 6: [0, 2, 6]}
    for i in range(T):
        rows = list(range(ctx)) + [ctx + a for a in anc[i]]
        np.testing.assert_allclose(got[0, i, 0], v[0, 0, rows].mean(axis=0), atol=1e-12)


def test_constant_values_come_back_unchanged():
    rng = np.random.default_rng(11)
    q = rng.normal(size=(1, 4, 2, 8)) * 5
    k = rng.normal(size=(1, 1, 20, 8))
    c = rng.normal(size=8)
    v = np.broadcast_to(c, (1, 1, 20, 8)).copy()
    got = verify_attention(q, k, v, 16, parents=[[-1, 0, 0, 2]])
    np.testing.assert_allclose(got, np.broadcast_to(c, got.shape), atol=1e-12)


def test_sampled_rows_match_full_output():
    rng = np.random.default_rng(12)
    q = rng.normal(size=(2, 3, 4, 8))
    k = rng.normal(size=(2, 2, 9, 8))
    v = rng.normal(size=(2, 2, 9, 8))
    full = verify_attention(q, k, v, 6)
    part = verify_attention(q, k, v, 6, rows=[(1, 2, 3), (0, 0, 1)])
    assert np.isnan(part[0, 1, 0]).all()
    np.testing.assert_array_equal(part[1, 2, 3], full[1, 2, 3])
    np.testing.assert_array_equal(part[0, 0, 1], full[0, 0, 1])
