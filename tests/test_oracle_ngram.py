"""Pins of oracle.ngram against things other than itself: hand-worked
examples, a search written with the standard library's bytes.rfind on a
fixed-width encoding of the tokens (a different route to the most recent
occurrence), and properties every proposal must have (the proposed tokens
followed an occurrence of the context's last n tokens, and no longer n-gram or
later occurrence exists).
"""
import numpy as np
import pytest

from oracle.ngram import ngram_propose


def one(tokens, N=4, n_min=1, n_max=3):
    c = np.array([tokens])
    num, d, e = ngram_propose(c, [len(tokens)], N, n_min, n_max)
    return int(num[0]), [int(x) for x in d[0, :num[0]]], int(e[0])


def test_hand_worked_examples():
    # "abcabc": the suffix "abc" occurs ending at 2; "abc" follows, cut by the end
    assert one([1, 2, 3, 1, 2, 3]) == (3, [1, 2, 3], 2)
    # the longest n-gram wins over a more recent shorter one
    assert one([7, 8, 9, 5, 9, 0, 7, 8, 9], n_max=3) == (4, [5, 9, 0, 7], 2)
    # only a shorter n-gram occurs: "9" most recently at 4 (followed by 0)
    assert one([7, 8, 9, 5, 9, 0, 1, 9], n_max=3) == (3, [0, 1, 9], 4)
    # nothing repeats: no draft
    assert one([1, 2, 3, 4, 5]) == (0, [], -1)
    # n_min above every repeat: no draft
    assert one([1, 2, 1, 3, 1], n_min=2) == (0, [], -1)
    # constant run: the most recent occurrence ends at L-2, one token follows
    assert one([4, 4, 4, 4, 4], N=3, n_max=2) == (1, [4], 3)
    # N limits the drafts
    assert one([1, 2, 3, 4, 5, 6, 1], N=2) == (2, [2, 3], 0)
    # too short a context for any occurrence
    assert one([3]) == (0, [], -1)


def _rfind_reference(c, N, n_min, n_max):
    """Most recent earlier occurrence via bytes.rfind on 4-byte big-endian
    tokens (a match must sit on a token boundary and end before L-1)."""
    L = len(c)
    enc = b"".join(int(t).to_bytes(4, "big") for t in c)
    for n in range(n_max, n_min - 1, -1):
        if n > L - 1:
            continue
        suf = enc[4 * (L - n):]
        hay_end = 4 * (L - 1)                 # occurrences end at e <= L-2
        pos = enc.rfind(suf, 0, hay_end)
        while pos != -1 and pos % 4 != 0:
            pos = enc.rfind(suf, 0, pos + len(suf) - 1)
        if pos != -1:
            e = pos // 4 + n - 1
            cont = list(c[e + 1: min(e + N, L - 1) + 1])
            return len(cont), cont, e
    return 0, [], -1


@pytest.mark.parametrize("seed", range(6))
def test_matches_a_bytes_rfind_search(seed):
    rng = np.random.default_rng(seed)
    B, Lmax, N = 40, 120, 6
    # small vocabularies and copied spans make repeats of every length
    ctx = rng.integers(0, 5 + 3 * seed, (B, Lmax))
    for b in range(B):
        for _ in range(3):
            s, ln = rng.integers(0, Lmax - 20), rng.integers(2, 12)
            d = rng.integers(s + 1, Lmax - ln)
            ctx[b, d:d + ln] = ctx[b, s:s + ln]
    lens = rng.integers(1, Lmax + 1, B)
    num, drafts, ends = ngram_propose(ctx, lens, N, 1, 4)
    for b in range(B):
        want = _rfind_reference(ctx[b, :lens[b]], N, 1, 4)
        assert (int(num[b]), [int(x) for x in drafts[b, :num[b]]], int(ends[b])) == want
        assert np.all(drafts[b, num[b]:] == -1)


def test_proposal_properties():
    rng = np.random.default_rng(9)
    B, L, N, n_min, n_max = 64, 300, 8, 2, 5
    ctx = rng.integers(0, 6, (B, L))
    lens = np.full(B, L)
    num, drafts, ends = ngram_propose(ctx, lens, N, n_min, n_max)
    for b in range(B):
        c = ctx[b]
        e = int(ends[b])
        assert e >= 0                           # with 6 tokens, 2-grams always repeat
        # the longest n whose suffix occurs earlier
        n = max(k for k in range(n_min, n_max + 1)
                if any(np.array_equal(c[j - k + 1: j + 1], c[L - k:]) for j in range(k - 1, L - 1)))
        assert np.array_equal(c[e - n + 1: e + 1], c[L - n:])
        assert not any(np.array_equal(c[j - n + 1: j + 1], c[L - n:]) for j in range(e + 1, L - 1))
        assert num[b] == min(N, L - 1 - e)
        assert np.array_equal(drafts[b, :num[b]], c[e + 1: e + 1 + num[b]])
