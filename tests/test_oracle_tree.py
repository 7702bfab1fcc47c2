"""Pins for oracle.accept.tree_accept against things other than itself.

"Parallel Decoding" glossary, "L'attention en arbre : la brique commune": the
root is the last verified token, branches are candidate continuations, the
longest accepted path becomes the output; "LLM Primer VI — Chapitre 9", §9.1:
at the first divergence the target's own choice is committed.

* brute force: every root→leaf path is walked from the root while each node's
  token equals its parent's target choice; the longest agreeing prefix over all
  paths wins (ties: lowest final node id);
* a chain-shaped tree is textbook greedy verification of a draft chain;
* T = 1 is an argmax decode step;
* argmax ties resolve to the lowest token id (rows built with known ties).
"""
import numpy as np
import pytest

from oracle.accept import tree_accept


def brute_force(z, tokens, parents):
    T, V = z.shape
    best = None
    leaves = [i for i in range(T) if i not in parents[1:]]
    for leaf in leaves:
        path = [leaf]
        while path[-1] != 0:
            path.append(parents[path[-1]])
        path.reverse()
        kept = [0]
        for n in path[1:]:
            parent_choice = max(range(V), key=lambda t: (z[kept[-1], t], -t))
            if tokens[n] != parent_choice:
                break
            kept.append(n)
        key = (len(kept), -kept[-1])
        if best is None or key > best[0]:
            best = (key, kept)
    kept = best[1]
    final_choice = max(range(V), key=lambda t: (z[kept[-1], t], -t))
    return len(kept) - 1, kept, [tokens[n] for n in kept[1:]] + [final_choice]


@pytest.mark.parametrize("seed", range(40))
def test_matches_brute_force_on_small_trees(seed):
    rng = np.random.default_rng(seed)
    B, T = 3, int(rng.integers(1, 14))
    V = int(rng.integers(2, 5))
    z = rng.integers(-2, 3, size=(B, T, V)).astype(np.float32)   # many ties
    tokens = rng.integers(0, V, size=(B, T))
    parents = np.array([[-1] + [int(rng.integers(0, i)) for i in range(1, T)]
                        for _ in range(B)])
    res = tree_accept(z, tokens, parents)
    for b in range(B):
        depth, path, emitted = brute_force(z[b], list(tokens[b]), list(parents[b]))
        assert res.accept_len[b] == depth
        assert list(res.path[b, :depth + 1]) == path
        assert np.all(res.path[b, depth + 1:] == -1)
        assert list(res.out_tokens[b, :depth + 1]) == emitted
        assert np.all(res.out_tokens[b, depth + 1:] == -1)


def test_chain_tree_is_greedy_chain_verification():
    rng = np.random.default_rng(1)
    B, T, V = 50, 7, 3
    z = rng.normal(size=(B, T, V))
    tokens = rng.integers(0, V, size=(B, T))
    res = tree_accept(z, tokens, np.array([[-1] + list(range(T - 1))] * B))
    for b in range(B):
        n = 0
        while n + 1 < T and tokens[b, n + 1] == np.argmax(z[b, n]):
            n += 1
        assert res.accept_len[b] == n
        assert list(res.path[b, :n + 1]) == list(range(n + 1))
        assert res.out_tokens[b, n] == np.argmax(z[b, n])


def test_single_node_is_an_argmax_decode_step():
    rng = np.random.default_rng(2)
    z = rng.normal(size=(20, 1, 50))
    res = tree_accept(z, np.zeros((20, 1), int), np.full((20, 1), -1))
    assert np.all(res.accept_len == 0)
    assert np.all(res.path[:, 0] == 0)
    assert np.all(res.out_tokens[:, 0] == z[:, 0].argmax(-1))


def test_argmax_ties_go_to_the_lowest_token():
    z = np.zeros((1, 2, 10), dtype=np.float32)
    z[0, 0, [3, 7]] = 5.0                   # tie between tokens 3 and 7
    z[0, 1, [9, 2]] = 1.0                   # tie between tokens 2 and 9
    res = tree_accept(z, np.array([[0, 3]]), np.array([[-1, 0]]))
    assert res.accept_len[0] == 1
    assert list(res.out_tokens[0]) == [3, 2]
    res = tree_accept(z, np.array([[0, 7]]), np.array([[-1, 0]]))
    assert res.accept_len[0] == 0 and res.out_tokens[0, 0] == 3


def test_deepest_tie_goes_to_lowest_node_and_duplicate_siblings():
    z = np.full((1, 5, 4), 0.0)
    z[0, 0, 1] = 1.0                        # root's choice: token 1
    z[0, 1, 2] = 1.0; z[0, 2, 3] = 1.0
    tokens = np.array([[0, 1, 1, 0, 0]])    # nodes 1 and 2 are duplicate siblings
    parents = np.array([[-1, 0, 0, 1, 2]])
    res = tree_accept(z, tokens, parents)
    assert res.accept_len[0] == 1 and list(res.path[0, :2]) == [0, 1]
    assert list(res.out_tokens[0, :2]) == [1, 2]


def test_malformed_parent_is_never_accepted():
    z = np.zeros((1, 3, 2)); z[0, :, 1] = 1.0
    res = tree_accept(z, np.array([[0, 1, 1]]), np.array([[-1, 0, 5]]))
    assert res.accept_len[0] == 1 and list(res.path[0]) == [0, 1, -1]
