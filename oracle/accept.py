"""Acceptance after the verify pass: chain rejection sampling and greedy trees.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Chain (``chain_accept``) — "LLM Primer VI — Chapitre 9 — Décodage spéculatif",
§9.1.  The drafts x_0..x_{N-1} were drawn from the draft distributions q_i.  The
target's pass gives p_0..p_N (one more position than there are drafts).  Going
along the chain, draft x_i is kept with probability min(1, p_i(x_i)/q_i(x_i));
at the first draft that is not kept the engine commits the target's own choice
there, drawn from the normalised positive part of p_i − q_i, and throws the
rest away.  This makes the emitted tokens distributed exactly as if the target
had sampled alone (also stated in the "Parallel Decoding" glossary, section
"Speculative Decoding", and in the mc2informatique article, step 3).  When every
draft is kept, the extra (N+1)-th distribution p_N supplies one more token.

Tree (``tree_accept``) — "Parallel Decoding" glossary, "L'attention en arbre :
la brique commune": the root is the last verified token, every branch is a
candidate continuation, and the longest accepted path becomes the output; the
Primer §9.2 says the target picks the best of several draft paths; §9.1 says the
engine commits to the target's own choice at the first divergence.  The check
is greedy (the mc2informatique article, step 2: do the drafts match the target's
own predictions).

Sampled tree (``tree_accept_sampled``) — the §9.1 rule applied to the several
candidates a tree offers for the same position, one after the other (its
docstring lists the readings).

Readings where the pages are silent:

* the ratio test is ``u < r`` with caller uniforms u in (0, 1); one u_accept per
  draft position and one u_draw per position, only the draw at the stopping
  row being used;
* q(x) = 0 gives r = +inf when p(x) > 0 and r = 0 otherwise;
* the inverse-CDF draw returns the smallest j with C_j > u·C_{V-1}, C the
  running sum in ascending token order; if rounding leaves no such j it
  returns the largest j with positive weight;
* a residual that sums to zero at a rejection (impossible in exact arithmetic)
  falls back to p itself;
* temperature τ divides the logits before the softmax (τ = 1 in every config);
* tree argmax ties go to the lowest token id; among equally deep accepted
  nodes the lowest node id wins; the accepted path need not reach a leaf.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

#: Relative half-width of the band around a decision boundary inside which an
#: fp32 implementation may legitimately decide the other way.
BOUNDARY_BAND = 1e-5


def softmax(logits, temperature: float = 1.0) -> np.ndarray:
    """Row softmax of logits / temperature in float64, max-subtracted."""
    z = np.asarray(logits, dtype=np.float64) / float(temperature)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def inverse_cdf(weights, u):
    """Draw from unnormalised non-negative weights with uniforms u, per row.

    weights [..., V], u [...].  Returns (y, lower, upper): y = min{j : C_j >
    u·C_{V-1}}, C the running sum in ascending token order, and the interval
    [C_{y-1}, C_y] / C_{V-1} of u-values that select y (used for flagging).
    If rounding leaves no crossing, y is the last token with positive weight.
    """
    w = np.asarray(weights, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    c = np.cumsum(w, axis=-1)
    total = c[..., -1]
    y = np.sum(c <= (u * total)[..., None], axis=-1)   # first index with C > u·total
    V = w.shape[-1]
    none = y >= V
    if np.any(none):
        last = V - 1 - np.argmax((w > 0)[..., ::-1], axis=-1)
        y = np.where(none, last, y)
    c_y = np.take_along_axis(c, y[..., None], axis=-1)[..., 0]
    c_before = np.where(y > 0, np.take_along_axis(c, np.maximum(y - 1, 0)[..., None],
                                                  axis=-1)[..., 0], 0.0)
    return y, c_before / total, c_y / total


@dataclass
class ChainResult:
    num_accepted: np.ndarray   # [B] int32
    out_tokens: np.ndarray     # [B, N+1] int32, -1 after the emitted tokens
    near_boundary: np.ndarray  # [B] bool: some used decision lies in the band


def chain_accept(target_logits, draft_logits, draft_tokens, u_accept, u_draw,
                 temperature: float = 1.0, band: float = BOUNDARY_BAND) -> ChainResult:
    """Rejection-sampling verification of a chain of N drafts, per sequence.

    target_logits [B, N+1, V], draft_logits [B, N, V], draft_tokens [B, N],
    u_accept [B, N], u_draw [B, N+1].  The steps follow the Primer §9.1 in its
    order: walk the chain, keep each draft while the ratio test passes, draw
    from the residual at the first failure, or from p_N when nothing failed.
    Sequences are independent; the walk runs for all of them at once.
    """
    zp = np.asarray(target_logits)
    zq = np.asarray(draft_logits)
    B, N1, V = zp.shape
    N = N1 - 1
    assert zq.shape == (B, N, V)
    x = np.asarray(draft_tokens, dtype=np.int64).reshape(B, N)
    ua = np.asarray(u_accept, dtype=np.float64).reshape(B, N)
    ud = np.asarray(u_draw, dtype=np.float64).reshape(B, N + 1)
    seq = np.arange(B)

    p = softmax(zp, temperature)                                  # [B, N+1, V]
    q = softmax(zq, temperature) if N else np.zeros((B, 0, V))    # [B, N, V]

    # Walk the chain: a sequence stops at its first failed ratio test.
    stop = np.full(B, N, dtype=np.int64)
    active = np.ones(B, dtype=bool)
    flag = np.zeros(B, dtype=bool)
    for i in range(N):
        xi = x[:, i]
        valid = (xi >= 0) & (xi < V)
        xc = np.where(valid, xi, 0)
        px = p[seq, i, xc]
        qx = q[seq, i, xc]
        # r = p(x)/q(x); q(x) = 0 gives +inf if p(x) > 0, else 0.
        with np.errstate(divide="ignore", invalid="ignore"):
            r = np.where(qx > 0, px / np.where(qx > 0, qx, 1.0),
                         np.where(px > 0, np.inf, 0.0))
        r = np.where(valid, r, 0.0)
        finite = np.isfinite(r)
        near = np.abs(ua[:, i] - np.where(finite, r, 0.0)) <= band * np.where(finite, r, 0.0)
        flag |= active & finite & near
        rejected = active & ~(ua[:, i] < r)
        stop[rejected] = i
        active &= ~rejected

    # The token committed at the stopping row: residual (p - q)+ after a
    # rejection, p_N after a full acceptance.
    p_stop = p[seq, stop]                                         # [B, V]
    if N:
        q_stop = q[seq, np.minimum(stop, N - 1)]
        w = np.where((stop < N)[:, None], np.maximum(p_stop - q_stop, 0.0), p_stop)
        empty = w.sum(axis=-1) == 0.0
        w[empty] = p_stop[empty]
    else:
        w = p_stop
    u = ud[seq, stop]
    y, lo, hi = inverse_cdf(w, u)
    flag |= (np.abs(u - lo) <= band * lo) | (np.abs(u - hi) <= band * hi)
    num = stop.astype(np.int32)
    col = np.arange(N + 1)[None, :]
    out = np.full((B, N + 1), -1, dtype=np.int32)
    kept = col[:, :N] < stop[:, None]
    out[:, :N][kept] = x[kept]
    out[seq, stop] = y
    return ChainResult(num, out, flag)


@dataclass
class TreeResult:
    accept_len: np.ndarray  # [B] int32: depth of the deepest accepted node
    path: np.ndarray        # [B, T] int32: node ids root..deepest, then -1
    out_tokens: np.ndarray  # [B, T] int32: path tokens (root excluded) + target's choice, then -1


def tree_accept(target_logits, tokens, parents) -> TreeResult:
    """Greedy verification of a draft tree (one target pass over all nodes).

    target_logits [B, T, V]: the target's logits at every node (node 0 = root,
    the last verified token); tokens [B, T]: the draft token each node carries
    (node 0's is ignored); parents [B, T]: parent node id, -1 for the root, and
    parents[i] < i.
    """
    z = np.asarray(target_logits)
    B, T, V = z.shape
    tok = np.asarray(tokens, dtype=np.int64).reshape(B, T)
    par = np.asarray(parents, dtype=np.int64).reshape(B, T)
    # The target's own choice at each node; np.argmax returns the first
    # (lowest) index among equal maxima.
    choice = np.argmax(z, axis=-1)

    accept_len = np.zeros(B, dtype=np.int32)
    path = np.full((B, T), -1, dtype=np.int32)
    out = np.full((B, T), -1, dtype=np.int32)
    for b in range(B):
        accepted = [True] + [False] * (T - 1)
        depth = [0] * T
        for i in range(1, T):
            pa = int(par[b, i])
            if not 0 <= pa < i:
                continue  # malformed parent: the node is never accepted
            depth[i] = depth[pa] + 1
            accepted[i] = accepted[pa] and tok[b, i] == choice[b, pa]
        best = 0
        for i in range(1, T):
            if accepted[i] and depth[i] > depth[best]:
                best = i
        nodes = []
        n = best
        while n >= 0:
            nodes.append(n)
            n = int(par[b, n]) if n > 0 else -1
        nodes.reverse()
        accept_len[b] = depth[best]
        path[b, :len(nodes)] = nodes
        emitted = [int(tok[b, n]) for n in nodes[1:]] + [int(choice[b, best])]
        out[b, :len(emitted)] = emitted
    return TreeResult(accept_len, path, out)


#: Relative error bound assumed for the probabilities of an implementation
#: that takes the sampled-tree decisions in float64 from exponentials rounded
#: to float32 (each p(v), q(v) within this factor of the exact value).
PROB_REL_ERR = 1e-6


@dataclass
class SampledTreeResult:
    accept_len: np.ndarray     # [B] int32: depth of the last accepted node
    path: np.ndarray           # [B, T] int32: node ids root..last, then -1
    out_tokens: np.ndarray     # [B, T] int32: path tokens (root excluded) + the drawn token, then -1
    near_boundary: np.ndarray  # [B] bool: some used decision lies within the error band


def tree_children(parents_row, T: int) -> list[list[int]]:
    """Children of every node in increasing id order; a node whose parent is
    not in [0, id) is nobody's child."""
    kids: list[list[int]] = [[] for _ in range(T)]
    for i in range(1, T):
        pa = int(parents_row[i])
        if 0 <= pa < i:
            kids[pa].append(i)
    return kids


def tree_accept_sampled(target_logits, draft_logits, tokens, parents, u_accept, u_draw,
                        temperature: float = 1.0, band: float = BOUNDARY_BAND,
                        eta: float = PROB_REL_ERR) -> SampledTreeResult:
    """Sampled (non-greedy) verification of a draft tree, per sequence.

    The Primer §9.2 has the target pick the best of several draft paths and
    §9.1 gives the one-candidate rule: keep a draft x with probability
    min(1, p(x)/q(x)), otherwise draw from the normalised (p - q)+.  With
    several candidates for the same position the rule is applied to them one
    after the other.  Readings (the pages give no multi-candidate rule):

    * the children of node n are the candidates for the token after n; they
      were drawn independently (with replacement) from q_n = softmax of
      draft_logits[b, n]; p_n = softmax of target_logits[b, n];
    * at node n the reference distribution starts as p_n; the children are
      tried in increasing id order; child i is kept iff u_accept[b, i] <
      ref(x_i) / q_n(x_i) (q = 0: +inf if ref(x) > 0, else 0; a token outside
      [0, V) gives 0); after each rejection ref becomes the normalised
      (ref - q_n)+ (a residual summing to zero falls back to p_n);
    * a kept child becomes the current node and the walk goes on from it;
    * when no child is kept (a leaf, or every child rejected) the emitted
      token is drawn from ref with u_draw[b, n] (``inverse_cdf``).

    Flags: a ratio test or a draw edge is flagged when its uniform lies within
    band (relative) plus the first-order error that probabilities accurate to
    ``eta`` (relative) can cause in that quantity, and a residual whose mass is
    within that error of zero is flagged (the emptiness test is a decision
    too); the residual is tracked as (p - c q)+ / Z for these bounds only.
    """
    zp = np.asarray(target_logits)
    zq = np.asarray(draft_logits)
    B, T, V = zp.shape
    assert zq.shape == (B, T, V)
    tok = np.asarray(tokens, dtype=np.int64).reshape(B, T)
    par = np.asarray(parents, dtype=np.int64).reshape(B, T)
    ua = np.asarray(u_accept, dtype=np.float64).reshape(B, T)
    ud = np.asarray(u_draw, dtype=np.float64).reshape(B, T)
    accept_len = np.zeros(B, dtype=np.int32)
    path = np.full((B, T), -1, dtype=np.int32)
    out = np.full((B, T), -1, dtype=np.int32)
    flag = np.zeros(B, dtype=bool)
    for b in range(B):
        kids = tree_children(par[b], T)
        n, nodes = 0, [0]
        while True:
            p = softmax(zp[b, n], temperature)
            q = softmax(zq[b, n], temperature)
            ref, c, Z = p.copy(), 0.0, 1.0
            kept = None
            for ch in kids[n]:
                x = int(tok[b, ch])
                if 0 <= x < V:
                    px, qx, rx = p[x], q[x], ref[x]
                    r = rx / qx if qx > 0 else (np.inf if rx > 0 else 0.0)
                else:
                    px = qx = rx = r = 0.0
                if np.isfinite(r) and qx > 0:
                    err = eta * ((px + c * qx) / (Z * qx) + r * ((1.0 + c) / Z + 1.0))
                    flag[b] |= abs(ua[b, ch] - r) <= band * r + err
                if ua[b, ch] < r:
                    kept = ch
                    break
                new = np.maximum(ref - q, 0.0)
                s = new.sum()
                if s > 0:
                    ref = new / s
                    c, Z = c + Z, Z * s
                    # an implementation may find a residual this small empty
                    flag[b] |= Z <= 2.0 * eta * (1.0 + c)
                else:
                    ref, c, Z = p.copy(), 0.0, 1.0
            if kept is None:
                break
            nodes.append(kept)
            n = kept
        u = ud[b, n]
        y, lo, hi = inverse_cdf(ref, u)
        err = 2.0 * eta * (1.0 + c) / Z
        flag[b] |= (abs(u - lo) <= band * lo + err) | (abs(u - hi) <= band * hi + err)
        accept_len[b] = len(nodes) - 1
        path[b, :len(nodes)] = nodes
        emitted = [int(tok[b, i]) for i in nodes[1:]] + [int(y)]
        out[b, :len(emitted)] = emitted
    return SampledTreeResult(accept_len, path, out, flag)
