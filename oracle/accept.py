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

import math
from dataclasses import dataclass, field

import numpy as np

#: Relative half-width of the band around a decision boundary inside which an
#: fp32 implementation may legitimately decide the other way, before the
#: decision's own error terms (the largest band the verification allows).
BOUNDARY_BAND = 1e-5

#: Unit roundoff of float32: one rounding moves a value by at most this, relative.
U32 = 2.0 ** -24
LN2 = math.log(2.0)
LOG2E = 1.0 / LN2
#: Relative error assumed for a float32 implementation's sums of non-negative
#: terms (a row's normaliser, the running sums of a CDF), beyond the errors of
#: the terms themselves: fixed summation trees of a few dozen roundings,
#: whose errors add up like a random walk (at most 4.2e-7 measured on rows of
#: 152064 tokens).
SUM_REL_ERR = 1e-6


@dataclass
class Flag:
    """A decision an implementation within the error model may take either
    way: the uniform u[index] (u_accept when kind is "accept", u_draw when it
    is "draw"; index is a chain row or a tree node) lies within `width` of
    `boundary`, the exact value it is compared with."""
    kind: str
    index: int
    boundary: float
    width: float
    # "draw" only: every positive-weight token whose interval of u-values
    # meets [u - width, u + width] (band_tokens)
    alt_tokens: tuple = ()


def row_stats(logits, temperature: float = 1.0):
    """Per row of logits: the maximum, l = log2 Σ 2^a with a = (z − max)·log2(e)/τ,
    and eps_s, a bound on the relative error of a float32 implementation's
    normaliser Σ 2^a: SUM_REL_ERR for the summation, plus, weighted by each
    term's mass, 2·U32 for its hardware exp2 and 8·U32·|a| of argument
    roundings (4·U32·|a| for the difference, the scale and the product, and as
    much again for the rescales from a partial sum's own maximum to the row's,
    whose arguments add up to at most |a|)."""
    z = np.asarray(logits, dtype=np.float64)
    zmax = z.max(axis=-1)
    a = (z - zmax[..., None]) * (LOG2E / float(temperature))
    e = np.exp2(a)
    s = e.sum(axis=-1)
    mean_abs_a = np.where(e > 0, e * np.abs(np.where(e > 0, a, 0.0)), 0.0).sum(axis=-1) / s
    return zmax, np.log2(s), SUM_REL_ERR + U32 * (2.0 + 8.0 * LN2 * mean_abs_a)


def prob_rel_err(a, l, eps_s, common: bool = True):
    """Relative error bound of a probability a float32 implementation computes
    as 2^(a − l), with a = (z − max)·log2(e)/τ and l the log2 of the row's
    normaliser (relative error eps_s).  Per token: the argument's roundings,
    U32·(4|a| + |a − l|) (difference, scale, product, the subtraction of l),
    times ln 2, and 3·U32 for the hardware exp2 and one more rounding of the
    result.  Common to the whole row (`common`): eps_s and the log2 of the
    normaliser, ln 2·2·U32·|l|; a draw from the row alone divides its running
    sums by their own total, where a factor common to every weight cancels."""
    a = np.where(np.isfinite(a), a, 0.0)
    e = LN2 * U32 * (4.0 * np.abs(a) + np.abs(a - l)) + 3.0 * U32
    if common:
        e = e + LN2 * U32 * 2.0 * np.abs(l) + eps_s
    return e


def ratio_rel_err(ap, lp, ep, aq, lq, eq):
    """Relative error bound of a ratio p(x)/q(x) a float32 implementation
    computes as 2^((ap − lp) − (aq − lq)) (a, l, eps_s as in row_stats and
    prob_rel_err, for the target row p and the draft row q): both
    probabilities' errors, ln 2·U32·|(ap − lp) − (aq − lq)| for the rounding of
    the difference, and 2·U32 for the hardware exp2."""
    d = (ap - lp) - (aq - lq)
    return (LN2 * U32 * (4 * np.abs(ap) + np.abs(ap - lp) + 2 * np.abs(lp)
                         + 4 * np.abs(aq) + np.abs(aq - lq) + 2 * np.abs(lq) + np.abs(d))
            + ep + eq + 2 * U32)


def weight_errors(zp_rows, zq_rows=None, temperature: float = 1.0):
    """Error bounds of a float32 implementation's draw weights, per row:
    zp_rows [..., V] target logits and zq_rows the matching draft rows, or
    None for a draw from p alone.  For p alone, dw_v = p_v · prob_rel_err
    without the row's common factor (it cancels against the total); for the
    residual (p − q)+, dw_v = p_v·e_p,v + q_v·e_q,v with the common factors
    (p and q have different ones), and 0 where p_v − q_v is negative by more
    than that (such a weight is zero in any implementation)."""
    k2 = LOG2E / float(temperature)
    zp_rows = np.asarray(zp_rows, dtype=np.float64)
    mp, lp, ep = row_stats(zp_rows, temperature)
    ap = (zp_rows - mp[..., None]) * k2
    p = softmax(zp_rows, temperature)
    common = zq_rows is not None
    dp = np.where(p > 0, p * prob_rel_err(ap, lp[..., None], ep[..., None], common), 0.0)
    if not common:
        return dp
    zq_rows = np.asarray(zq_rows, dtype=np.float64)
    mq, lq, eq = row_stats(zq_rows, temperature)
    aq = (zq_rows - mq[..., None]) * k2
    q = softmax(zq_rows, temperature)
    dq = np.where(q > 0, q * prob_rel_err(aq, lq[..., None], eq[..., None]), 0.0)
    return np.where(p - q > -(dp + dq), dp + dq, 0.0)


def edge_width(b, e_edge, e_tot, total, band: float = 0.0):
    """Half-width of the band around a CDF edge b = C/Z of a draw: band·b, the
    weights' errors (a weight's error bound e_v; e_edge the sum of those up to
    the edge, e_tot of all), which move b by at most ((1 − b)·e_edge + b·(e_tot
    − e_edge))/Z (the errors before the edge and past it pull it opposite
    ways), SUM_REL_ERR·b for the float32 running sum, and U32 for u·Z."""
    return (band * b + ((1 - b) * e_edge + b * (e_tot - e_edge)) / total
            + SUM_REL_ERR * b + U32)


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


def band_tokens(weights_row, u: float, width: float) -> tuple:
    """Every token a draw within `width` of u may land on: the tokens with
    positive weight whose interval [C_{j-1}, C_j] / C_{V-1} meets [u - width,
    u + width] (the decision-precision reading of a draw: the running sums
    are known only to within the edge widths, so any token the band reaches
    is a correct outcome, however small its own mass)."""
    w = np.asarray(weights_row, dtype=np.float64)
    c = np.cumsum(w)
    total = c[-1]
    if not total > 0:
        return ()
    hi = c / total
    lo = np.concatenate([[0.0], hi[:-1]])
    return tuple(int(j) for j in np.flatnonzero((w > 0) & (lo <= u + width) & (hi >= u - width)))


@dataclass
class ChainResult:
    num_accepted: np.ndarray     # [B] int32
    out_tokens: np.ndarray       # [B, N+1] int32, -1 after the emitted tokens
    near_boundary: np.ndarray    # [B] bool: some used decision is flagged
    flags: list = field(default_factory=list)   # per sequence, its flagged decisions (Flag)
    empty_ambiguous: np.ndarray = None  # [B] bool: the residual is within its error of empty


def chain_accept(target_logits, draft_logits, draft_tokens, u_accept, u_draw,
                 temperature: float = 1.0, band: float = BOUNDARY_BAND) -> ChainResult:
    """Rejection-sampling verification of a chain of N drafts, per sequence.

    target_logits [B, N+1, V], draft_logits [B, N, V], draft_tokens [B, N],
    u_accept [B, N], u_draw [B, N+1].  The steps follow the Primer §9.1 in its
    order: walk the chain, keep each draft while the ratio test passes, draw
    from the residual at the first failure, or from p_N when nothing failed.
    Sequences are independent; the walk runs for all of them at once.

    Flags (the decision-precision reading): a used decision is flagged when
    its uniform lies within band·b plus the decision's own error bound of its
    boundary b, for an implementation that computes each probability in
    float32 as 2^(a − l) (``prob_rel_err``): a ratio test r = p(x)/q(x) adds
    the two probabilities' errors (and 2·U32 for the exp2 of the difference);
    a CDF edge b = C/Z of the drawn row adds ((1 − b)·E + b·(E_total − E))/Z,
    E the summed error bounds of the weights up to the edge and E_total of
    all of them, plus SUM_REL_ERR·b for the running sum and U32 for u·Z.  A residual whose mass is within its error of zero
    is marked empty_ambiguous (an implementation may fall back to p there)
    unless the two rows are identical (then both sides find it empty).
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
    k2 = LOG2E / float(temperature)
    mp, lp, ep = row_stats(zp, temperature)                       # [B, N+1] each
    if N:
        mq, lq, eq = row_stats(zq, temperature)                   # [B, N] each
    flags = [[] for _ in range(B)]

    # Walk the chain: a sequence stops at its first failed ratio test.
    stop = np.full(B, N, dtype=np.int64)
    active = np.ones(B, dtype=bool)
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
        rf = np.where(finite, r, 0.0)
        ap = (zp[seq, i, xc] - mp[:, i]) * k2
        aq = (zq[seq, i, xc] - mq[:, i]) * k2
        with np.errstate(invalid="ignore"):
            eps_r = ratio_rel_err(ap, lp[:, i], ep[:, i], aq, lq[:, i], eq[:, i])
        width = np.where(finite & (rf > 0), band * rf + np.nan_to_num(eps_r) * rf, 0.0)
        near = active & finite & (rf > 0) & (np.abs(ua[:, i] - rf) <= width)
        for b in np.flatnonzero(near):
            flags[b].append(Flag("accept", i, float(rf[b]), float(width[b])))
        rejected = active & ~(ua[:, i] < r)
        stop[rejected] = i
        active &= ~rejected

    # The token committed at the stopping row: residual (p - q)+ after a
    # rejection, p_N after a full acceptance.
    p_stop = p[seq, stop]                                         # [B, V]
    zp_stop = zp[seq, stop]
    resid = stop < N
    dw = weight_errors(zp_stop, None, temperature)
    ambiguous = np.zeros(B, dtype=bool)
    if N:
        kq = np.minimum(stop, N - 1)
        q_stop = q[seq, kq]
        zq_stop = zq[seq, kq]
        w = np.where(resid[:, None], np.maximum(p_stop - q_stop, 0.0), p_stop)
        dw_res = weight_errors(zp_stop, zq_stop, temperature)
        mass = w.sum(axis=-1)
        identical = np.all(zp_stop == zq_stop, axis=-1)
        ambiguous = resid & ~identical & (mass <= dw_res.sum(axis=-1))
        empty = mass == 0.0
        w[empty] = p_stop[empty]
        dw = np.where((resid & ~empty)[:, None], dw_res, dw)
    else:
        w = p_stop
    u = ud[seq, stop]
    y, lo, hi = inverse_cdf(w, u)
    e_cum = np.cumsum(dw, axis=-1)
    e_tot = e_cum[:, -1]
    z_tot = w.sum(axis=-1)
    e_hi = e_cum[seq, y]
    e_lo = np.where(y > 0, e_cum[seq, np.maximum(y - 1, 0)], 0.0)
    w_hi = edge_width(hi, e_hi, e_tot, z_tot, band)
    w_lo = edge_width(lo, e_lo, e_tot, z_tot, band)
    near_lo = np.abs(u - lo) <= w_lo
    near_hi = np.abs(u - hi) <= w_hi
    for b in np.flatnonzero(near_lo | near_hi):
        alts = band_tokens(w[b], float(u[b]), float(max(w_lo[b], w_hi[b])))
        if near_lo[b]:
            flags[b].append(Flag("draw", int(stop[b]), float(lo[b]), float(w_lo[b]), alts))
        if near_hi[b]:
            flags[b].append(Flag("draw", int(stop[b]), float(hi[b]), float(w_hi[b]), alts))
    num = stop.astype(np.int32)
    col = np.arange(N + 1)[None, :]
    out = np.full((B, N + 1), -1, dtype=np.int32)
    kept = col[:, :N] < stop[:, None]
    out[:, :N][kept] = x[kept]
    out[seq, stop] = y
    flagged = np.array([len(f) > 0 for f in flags], dtype=bool) | ambiguous
    return ChainResult(num, out, flagged, flags, ambiguous)


def _nudged(flag: Flag, side: float):
    """The uniform moved to one side of a flagged decision's boundary, twice
    its width away; None when that side leaves (0, 1)."""
    v = flag.boundary + side * 2.0 * flag.width
    return v if 0.0 < v < 1.0 else None


def chain_admissible(target_logits, draft_logits, draft_tokens, u_accept, u_draw, b: int,
                     temperature: float = 1.0, band: float = BOUNDARY_BAND,
                     depth: int = 3) -> set:
    """The outcomes (num_accepted, out_tokens as a tuple) that sequence b may
    have under the error model: chain_accept's own; for every flagged ratio
    test the outcome with that test taken each way (its uniform moved to
    either side of the boundary), recursively to `depth` levels; for a
    flagged draw every token its band reaches (Flag.alt_tokens: the draw's
    uniform decides nothing else, so only the drawn token changes)."""
    sl = slice(b, b + 1)
    zp = np.asarray(target_logits)[sl]
    zq = np.asarray(draft_logits)[sl]
    x = np.asarray(draft_tokens)[sl]
    seen, outcomes = set(), set()

    def visit(ua, ud, d):
        key = (tuple(ua.ravel()), tuple(ud.ravel()))
        if key in seen:
            return
        seen.add(key)
        r = chain_accept(zp, zq, x, ua, ud, temperature, band)
        outcomes.add((int(r.num_accepted[0]), tuple(int(t) for t in r.out_tokens[0])))
        n = int(r.num_accepted[0])
        for f in r.flags[0]:
            if f.kind != "draw":
                continue
            for j in f.alt_tokens:
                toks = [int(t) for t in r.out_tokens[0]]
                toks[n] = j
                outcomes.add((n, tuple(toks)))
        if d == 0:
            return
        for f in r.flags[0]:
            for side in (-1.0, 1.0):
                v = _nudged(f, side)
                if v is None:
                    continue
                ua2, ud2 = ua.copy(), ud.copy()
                (ua2 if f.kind == "accept" else ud2)[0, f.index] = v
                visit(ua2, ud2, d - 1)

    visit(np.array(u_accept, dtype=np.float64)[sl], np.array(u_draw, dtype=np.float64)[sl],
          depth)
    return outcomes


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


@dataclass
class SampledTreeResult:
    accept_len: np.ndarray     # [B] int32: depth of the last accepted node
    path: np.ndarray           # [B, T] int32: node ids root..last, then -1
    out_tokens: np.ndarray     # [B, T] int32: path tokens (root excluded) + the drawn token, then -1
    near_boundary: np.ndarray  # [B] bool: some used decision is flagged
    flags: list = field(default_factory=list)   # per sequence, its flagged decisions (Flag)
    empty_ambiguous: np.ndarray = None  # [B] bool: a residual is within its error of empty


def tree_row_model(z, temperature: float = 1.0):
    """Error model of one row for an implementation that forms 2^a, a = (z −
    max)·log2(e)/τ, in float32 (the argument rounded three times: difference,
    scale, product; then the hardware exp2) and sums those terms in float64
    in groups of four float32 additions.  Returns (eps_s, term): eps_s bounds
    the relative error of the row's normaliser (U32·(3·ln 2·|a| + 2) per term,
    mass-weighted, 3·U32 for the groups, 2.5·U32 for rescaling partial sums
    with the hardware exp2), and term[v] the relative error of token v's
    float32 term times the float32 reciprocal normaliser, apart from factors
    common to the row (U32·(3·ln 2·|a_v| + 3): argument, exp2, the product)."""
    z = np.asarray(z, dtype=np.float64)
    a = (z - z.max()) * (LOG2E / float(temperature))
    e = np.exp2(a)
    fin = e > 0
    abs_a = np.abs(np.where(fin, a, 0.0))
    eps_s = U32 * (7.5 + 3.0 * LN2 * float((e * abs_a).sum() / e.sum()))
    term = np.where(fin, U32 * (3.0 * LN2 * abs_a + 3.0), 0.0)
    return eps_s, term


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
                        temperature: float = 1.0,
                        band: float = BOUNDARY_BAND) -> SampledTreeResult:
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

    Flags (the decision-precision reading): the residual after j rejections
    is (p − c_j q)+ / Z_j with c_0 = 0, Z_0 = 1, c_{j+1} = c_j + Z_j; for an
    implementation that reads the ratio tests' probabilities within 3·U32
    (and the normaliser's error) and sums float32 terms (``tree_row_model``)
    in float64, the errors of Z_j and c_j are carried along to first order,
    and a ratio test or draw edge is flagged when its uniform lies within
    band·b plus the propagated error of its boundary b.  A residual whose
    mass is within its error of zero is marked empty_ambiguous (the
    implementation may fall back to p there) unless the two rows are
    identical (then both sides find it empty).
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
    flags = [[] for _ in range(B)]
    ambiguous = np.zeros(B, dtype=bool)
    for b in range(B):
        kids = tree_children(par[b], T)
        n, nodes = 0, [0]
        while True:
            p = softmax(zp[b, n], temperature)
            q = softmax(zq[b, n], temperature)
            ref, c, Z = p.copy(), 0.0, 1.0
            # error model of this node's rows (see the docstring)
            es_p, term_p = tree_row_model(zp[b, n], temperature)
            es_q, term_q = tree_row_model(zq[b, n], temperature)
            identical = bool(np.array_equal(zp[b, n], zq[b, n]))
            tok_p = p * (term_p + 2.0 * U32 + es_p)      # + reciprocal rounding, subtraction
            tok_q = q * (term_q + 3.0 * U32 + es_q)      # + reciprocal, c and product roundings
            dc = dZ = 0.0
            kept = None
            for ch in kids[n]:
                x = int(tok[b, ch])
                if 0 <= x < V:
                    px, qx, rx = p[x], q[x], ref[x]
                    r = rx / qx if qx > 0 else (np.inf if rx > 0 else 0.0)
                else:
                    px = qx = rx = r = 0.0
                if np.isfinite(r) and qx > 0 and r > 0:
                    dpx = px * (3.0 * U32 + es_p)
                    dqx = qx * (3.0 * U32 + es_q)
                    dr = (dpx + c * dqx + qx * dc) / (Z * qx) + r * (dZ / Z + dqx / qx)
                    width = band * r + dr
                    if abs(ua[b, ch] - r) <= width:
                        flags[b].append(Flag("accept", ch, float(r), float(width)))
                if ua[b, ch] < r:
                    kept = ch
                    break
                new = np.maximum(ref - q, 0.0)
                s = new.sum()
                c_new, dc_new = c + Z, dc + dZ
                dwv = tok_p + c_new * tok_q + q * dc_new
                pos = p - c_new * q > -dwv
                dZ_new = float(dwv[pos].sum()) + 3.0 * U32 * Z * s
                if Z * s <= dZ_new and not identical:
                    ambiguous[b] = True           # an implementation may find it empty
                if s > 0:
                    ref = new / s
                    c, Z, dc, dZ = c_new, Z * s, dc_new, dZ_new
                else:
                    ref, c, Z, dc, dZ = p.copy(), 0.0, 1.0, 0.0, 0.0
            if kept is None:
                break
            nodes.append(kept)
            n = kept
        u = ud[b, n]
        y, lo, hi = inverse_cdf(ref, u)
        if c == 0.0:
            dw = p * term_p                       # a draw from p: the row's own factor cancels
        else:
            dw = tok_p + c * tok_q + q * dc
            dw = np.where(p - c * q > -dw, dw, 0.0)
        e_cum = np.cumsum(dw) / Z
        e_hi = e_cum[y]
        e_lo = e_cum[y - 1] if y > 0 else 0.0
        # b = C/total moves by (δC·(1 − b) − b·δ(total − C))/total
        w_hi = band * hi + (1 - hi) * e_hi + hi * (e_cum[-1] - e_hi)
        w_lo = band * lo + (1 - lo) * e_lo + lo * (e_cum[-1] - e_lo)
        if abs(u - lo) <= w_lo or abs(u - hi) <= w_hi:
            alts = band_tokens(ref, float(u), float(max(w_lo, w_hi)))
            if abs(u - lo) <= w_lo:
                flags[b].append(Flag("draw", n, float(lo), float(w_lo), alts))
            if abs(u - hi) <= w_hi:
                flags[b].append(Flag("draw", n, float(hi), float(w_hi), alts))
        accept_len[b] = len(nodes) - 1
        path[b, :len(nodes)] = nodes
        emitted = [int(tok[b, i]) for i in nodes[1:]] + [int(y)]
        out[b, :len(emitted)] = emitted
    flagged = np.array([len(f) > 0 for f in flags], dtype=bool) | ambiguous
    return SampledTreeResult(accept_len, path, out, flagged, flags, ambiguous)


def tree_sampled_admissible(target_logits, draft_logits, tokens, parents, u_accept, u_draw,
                            b: int, temperature: float = 1.0, band: float = BOUNDARY_BAND,
                            depth: int = 3) -> set:
    """The outcomes (accept_len, path, out_tokens, as tuples) that sequence b
    may have under the error model: tree_accept_sampled's own; for every
    flagged ratio test the outcome with that test taken each way (its uniform
    moved to either side of the boundary), recursively to `depth`; for a
    flagged draw every token its band reaches (Flag.alt_tokens)."""
    sl = slice(b, b + 1)
    zp = np.asarray(target_logits)[sl]
    zq = np.asarray(draft_logits)[sl]
    tok = np.asarray(tokens)[sl]
    par = np.asarray(parents)[sl]
    seen, outcomes = set(), set()

    def visit(ua, ud, d):
        key = (tuple(ua.ravel()), tuple(ud.ravel()))
        if key in seen:
            return
        seen.add(key)
        r = tree_accept_sampled(zp, zq, tok, par, ua, ud, temperature, band)
        outcomes.add((int(r.accept_len[0]), tuple(int(t) for t in r.path[0]),
                      tuple(int(t) for t in r.out_tokens[0])))
        n = int(r.accept_len[0])
        path_t = tuple(int(t) for t in r.path[0])
        for f in r.flags[0]:
            if f.kind != "draw":
                continue
            for j in f.alt_tokens:
                toks = [int(t) for t in r.out_tokens[0]]
                toks[n] = j
                outcomes.add((n, path_t, tuple(toks)))
        if d == 0:
            return
        for f in r.flags[0]:
            for side in (-1.0, 1.0):
                v = _nudged(f, side)
                if v is None:
                    continue
                ua2, ud2 = ua.copy(), ud.copy()
                (ua2 if f.kind == "accept" else ud2)[0, f.index] = v
                visit(ua2, ud2, d - 1)

    visit(np.array(u_accept, dtype=np.float64)[sl], np.array(u_draw, dtype=np.float64)[sl],
          depth)
    return outcomes
