"""Pins of the decision-precision model in oracle.accept against float32 arithmetic.

The pages fix no precision.  The oracle flags a decision when its uniform lies
within the error a float32 implementation may make in the quantity it is
compared with (a ratio p(x)/q(x), an edge C/Z of a draw's CDF), and offers
both outcomes there (chain_admissible, tree_sampled_admissible).  These tests
pin that model to something other than itself:

* float32 arithmetic emulated in numpy (every operation of a float32 array
  rounds) for the probabilities, ratios and draw weights the model covers:
  the observed float32-vs-float64 deviations must lie inside the model's
  bounds, and the bounds must not be loose (the largest deviation seen is at
  least 1/20 of the ratio bound, 1/100 of the CDF-edge and normaliser bounds,
  1/10 of the per-token bound);
* the summation allowance SUM_REL_ERR against float32 sums in the shape of a
  fixed reduction tree (sequential per-lane sums, a butterfly, sequential
  merges) and of a blocked inclusive scan: it must cover them with a 2x
  margin;
* constructed boundary cases: a uniform on a ratio or on a CDF edge is
  flagged, and the admissible set then holds the outcome on each side;
  a sequence with no flag has exactly one admissible outcome.
"""
import numpy as np
import pytest

from oracle.accept import (LOG2E, SUM_REL_ERR, U32, chain_accept, chain_admissible,
                           edge_width, ratio_rel_err, row_stats, softmax, tree_accept_sampled,
                           tree_row_model, tree_sampled_admissible, weight_errors)

F = np.float32


def fp32_log_probs(z, tau):
    """Float32 emulation of log2 p = a − l: c = fl(fl(log2 e)/τ), a = fl(fl(z −
    max)·c), terms fl(exp2(a)) summed in float64 (the summation is pinned
    separately), S rounded to float32, l = fl(log2 S), then fl(a − l)."""
    z32 = np.asarray(z, dtype=F)
    c = F(F(LOG2E) / F(tau))
    a = (z32 - z32.max(axis=-1, keepdims=True)) * c
    s = F(np.exp2(a).astype(np.float64).sum(axis=-1))
    l32 = np.log2(s)
    return a - l32[..., None]


def rows(seed, R, V, sd, noise):
    rng = np.random.default_rng(seed)
    zp = rng.normal(0.0, sd, (R, V)).astype(F).astype(np.float64)
    zq = (zp + rng.normal(0.0, noise, (R, V))).astype(F).astype(np.float64)
    return rng, zp, zq


@pytest.mark.parametrize("V,sd,noise,tau", [(152064, 3.0, 1.0, 1.0), (1024, 2.0, 0.5, 1.0),
                                            (32000, 3.0, 1.0, 0.7), (5000, 2.0, 1.0, 1.6)])
def test_ratio_bound_covers_float32(V, sd, noise, tau):
    rng, zp, zq = rows(11, 8, V, sd, noise)
    lp32, lq32 = fp32_log_probs(zp, tau), fp32_log_probs(zq, tau)
    p, q = softmax(zp, tau), softmax(zq, tau)
    mp, lp, ep = row_stats(zp, tau)
    mq, lq, eq = row_stats(zq, tau)
    k2 = LOG2E / tau
    worst = 0.0
    for r_ in range(zp.shape[0]):
        x = rng.choice(V, size=400, p=q[r_])                     # drafts drawn from q
        r64 = p[r_, x] / q[r_, x]
        r32 = np.exp2(lp32[r_, x] - lq32[r_, x]).astype(np.float64)
        bound = r64 * ratio_rel_err((zp[r_, x] - mp[r_]) * k2, lp[r_], ep[r_],
                                    (zq[r_, x] - mq[r_]) * k2, lq[r_], eq[r_])
        dev = np.abs(r32 - r64)
        assert np.all(dev <= bound)
        worst = max(worst, float(np.max(dev / bound)))
    assert worst > 0.05, f"bound loose: largest deviation is {worst:.2e} of it"


@pytest.mark.parametrize("V,sd,noise,tau,resid", [(152064, 3.0, 1.0, 1.0, True),
                                                  (152064, 3.0, 1.0, 1.0, False),
                                                  (1024, 2.0, 0.5, 1.0, True),
                                                  (32000, 2.0, 1.0, 2.0, False)])
def test_cdf_edge_bound_covers_float32(V, sd, noise, tau, resid):
    """Every edge C_y/Z of the draw weights, float32 weights (summed in
    float64 here) against float64, inside edge_width without its band and
    summation terms."""
    _, zp, zq = rows(12, 4, V, sd, noise)
    lp32, lq32 = fp32_log_probs(zp, tau), fp32_log_probs(zq, tau)
    p, q = softmax(zp, tau), softmax(zq, tau)
    if resid:
        w64 = np.maximum(p - q, 0.0)
        w32 = np.maximum(np.exp2(lp32) - np.exp2(lq32), F(0)).astype(np.float64)
        dw = weight_errors(zp, zq, tau)
    else:
        w64, w32 = p, np.exp2(lp32).astype(np.float64)
        dw = weight_errors(zp, None, tau)
    c64, c32 = np.cumsum(w64, -1), np.cumsum(w32, -1)
    b64 = c64 / c64[:, -1:]
    b32 = c32 / c32[:, -1:]
    e = np.cumsum(dw, -1)
    model = edge_width(b64, e, e[:, -1:], c64[:, -1:]) - SUM_REL_ERR * b64 - U32
    dev = np.abs(b32 - b64)
    assert np.all(dev <= model)
    pos = model > 0                           # the last edge is 1 on both sides
    assert float(np.max(dev[pos] / model[pos])) > 0.01


def test_summation_allowance_covers_float32_trees():
    """SUM_REL_ERR against float32 sums of 152064 positive terms in a fixed
    tree (32 sequential per lane, a 64-lane butterfly, 8 sequential partials
    per 16384-term chunk, a butterfly over the chunks), and against a blocked
    inclusive float32 scan (8 sequential per lane, a 64-lane doubling scan,
    16 sequential wave offsets, sequential carries over 8192-term chunks)."""
    rng = np.random.default_rng(13)
    V = 152064
    worst_sum = worst_scan = 0.0
    for _ in range(24):
        z = rng.normal(0.0, 3.0, V)
        t = np.exp2((z - z.max()) * LOG2E).astype(F)
        exact = t.astype(np.float64)
        # tree sum
        pad = np.zeros(10 * 16384, dtype=F)
        pad[:V] = t
        chunks = pad.reshape(10, 8, 512, 4).transpose(0, 2, 1, 3).reshape(10, 8, 64, 32)
        lane = np.zeros((10, 8, 64), dtype=F)
        for i in range(32):
            lane = lane + chunks[..., i]
        for off in (1, 2, 4, 8, 16, 32):
            lane = lane + lane[..., np.arange(64) ^ off]
        waves = lane[..., 0]
        acc = waves[:, 0]
        for wv in range(1, 8):
            acc = acc + waves[:, wv]
        ch = np.zeros(64, dtype=F)
        ch[:10] = acc
        for off in (1, 2, 4, 8, 16, 32):
            ch = ch + ch[np.arange(64) ^ off]
        worst_sum = max(worst_sum, abs(float(ch[0]) / exact.sum() - 1.0))
        # blocked scan
        pad = np.zeros(19 * 8192, dtype=F)
        pad[:V] = t
        blk = pad.reshape(19, 16, 64, 8)
        local = np.zeros_like(blk)
        run = np.zeros((19, 16, 64), dtype=F)
        for e in range(8):
            run = run + blk[..., e]
            local[..., e] = run
        incl = run.copy()
        for off in (1, 2, 4, 8, 16, 32):
            sh = np.zeros_like(incl)
            sh[..., off:] = incl[..., :-off]
            incl = incl + sh
        excl = np.zeros_like(incl)
        excl[..., 1:] = incl[..., :-1]
        woff = np.zeros((19, 16), dtype=F)
        accw = np.zeros(19, dtype=F)
        for wv in range(16):
            woff[:, wv] = accw
            accw = accw + incl[:, wv, 63]
        carry = np.zeros(19, dtype=F)
        cacc = F(0)
        for c in range(19):
            carry[c] = cacc
            cacc = cacc + accw[c]
        scan = (carry[:, None, None, None] + (woff[..., None, None] + excl[..., None])) + local
        c32 = scan.reshape(-1)[:V].astype(np.float64)
        c64 = np.cumsum(exact)
        big = c64 > 1e-3 * c64[-1]
        worst_scan = max(worst_scan, float(np.max(np.abs(c32[big] / c64[big] - 1.0))))
    assert worst_sum <= SUM_REL_ERR / 2 and worst_scan <= SUM_REL_ERR / 2, (worst_sum, worst_scan)


def test_tree_row_model_covers_float32():
    """tree_row_model: a float64 sum of float32 terms fl(exp2(fl(fl(z − m)·fl(k)))),
    in groups of four float32 additions, within eps_s of the exact normaliser;
    each float32 term times the float32 reciprocal normaliser within term + 2·U32
    + eps_s of the exact probability."""
    rng = np.random.default_rng(14)
    worst = worst_s = 0.0
    for V, sd, tau in ((32000, 3.0, 1.0), (40001, 2.0, 2.0), (999, 2.0, 0.7)):
        for _ in range(6):
            z = rng.normal(0.0, sd, V).astype(F).astype(np.float64)
            eps_s, term = tree_row_model(z, tau)
            z32 = z.astype(F)
            k2f = F(LOG2E / tau)
            t = np.exp2((z32 - z32.max()) * k2f)
            pad = np.zeros(-(-V // 4) * 4, dtype=F)
            pad[:V] = t
            g = pad.reshape(-1, 4)
            s = ((g[:, 0] + g[:, 1]) + (g[:, 2] + g[:, 3])).astype(np.float64).sum()
            exact = np.exp2((z - z.max()) * (LOG2E / tau)).sum()
            assert abs(s / exact - 1.0) <= eps_s
            worst_s = max(worst_s, abs(s / exact - 1.0) / eps_s)
            p = softmax(z, tau)
            p32 = (t * F(1.0 / s)).astype(np.float64)
            dev = np.abs(p32 / p - 1.0)
            bound = term + 2 * U32 + eps_s
            assert np.all(dev <= bound)
            worst = max(worst, float(np.max(dev / bound)))
    assert worst > 0.1 and worst_s > 0.01, (worst, worst_s)


def test_ratio_on_the_boundary_is_flagged_and_both_outcomes_admissible():
    zp = np.log(np.array([[[0.25, 0.75], [0.5, 0.5]]]))
    zq = np.log(np.array([[[0.5, 0.5]]]))
    x = np.array([[0]])
    # r = 0.25 / 0.5 = 0.5 exactly: u at r is flagged (band 0: the model alone)
    res = chain_accept(zp, zq, x, np.array([[0.5]]), np.array([[0.3, 0.3]]), band=0.0)
    assert res.near_boundary[0] and res.flags[0][0].kind == "accept"
    assert res.flags[0][0].index == 0 and abs(res.flags[0][0].boundary - 0.5) < 1e-15
    alts = chain_admissible(zp, zq, x, np.array([[0.5]]), np.array([[0.3, 0.3]]), 0,
                            band=0.0)
    # kept: x then the bonus draw from p_1 = [0.5, 0.5] at 0.3 -> token 0;
    # rejected: the residual (p_0 - q_0)+ = [0, 0.25] -> token 1
    assert alts == {(1, (0, 0)), (0, (1, -1))}
    # far from every boundary: one outcome, no flag
    res = chain_accept(zp, zq, x, np.array([[0.2]]), np.array([[0.3, 0.3]]), band=0.0)
    assert not res.near_boundary[0] and res.flags[0] == []
    assert chain_admissible(zp, zq, x, np.array([[0.2]]), np.array([[0.3, 0.3]]), 0) == \
        {(1, (0, 0))}


def test_cdf_edge_is_flagged_and_both_tokens_admissible():
    # N = 0: a draw from p_0 = [0.2, 0.3, 0.5]; u = 0.5 is the edge between
    # tokens 1 and 2
    zp = np.log(np.array([[[0.2, 0.3, 0.5]]]))
    zq = np.zeros((1, 0, 3))
    x = np.zeros((1, 0), dtype=np.int64)
    ua = np.zeros((1, 0))
    res = chain_accept(zp, zq, x, ua, np.array([[0.5]]), band=0.0)
    assert [f.kind for f in res.flags[0]] == ["draw"]
    assert chain_admissible(zp, zq, x, ua, np.array([[0.5]]), 0, band=0.0) == \
        {(0, (1,)), (0, (2,))}
    assert chain_admissible(zp, zq, x, ua, np.array([[0.45]]), 0, band=0.0) == {(0, (1,))}


def test_draw_band_reaches_a_token_narrower_than_the_band():
    # p_0 = [0.5, 2e-7, 0.5 - 2e-7]; u just below the edge at 0.5.  The band
    # around u (width about band·u) reaches token 1 (mass 2e-7, narrower than
    # the band) and the start of token 2: all three are admissible.  Moving u
    # twice the width past the edge lands on token 2 and never on token 1.
    zp = np.log(np.array([[[0.5, 2e-7, 0.5 - 2e-7]]]))
    zq = np.zeros((1, 0, 3))
    x = np.zeros((1, 0), dtype=np.int64)
    ua = np.zeros((1, 0))
    ud = np.array([[0.5 - 1e-7]])
    res = chain_accept(zp, zq, x, ua, ud, band=1e-6)
    assert int(res.out_tokens[0, 0]) == 0 and [f.kind for f in res.flags[0]] == ["draw"]
    assert chain_admissible(zp, zq, x, ua, ud, 0, band=1e-6) == {(0, (0,)), (0, (1,)), (0, (2,))}
    # far from the edge: token 0 alone
    assert chain_admissible(zp, zq, x, ua, np.array([[0.3]]), 0, band=1e-6) == {(0, (0,))}
    # the same draw at the root of a one-node tree
    tok = np.array([[0]])
    par = np.array([[-1]])
    alts = tree_sampled_admissible(zp, zp, tok, par, np.array([[0.5]]), ud, 0, band=1e-6)
    assert alts == {(0, (0,), (0,)), (0, (0,), (1,)), (0, (0,), (2,))}


def test_residual_near_empty_is_ambiguous_but_identical_rows_are_not():
    rng = np.random.default_rng(15)
    zp = rng.normal(0, 2.0, (2, 2, 50))
    zq = zp[:, :1].copy()
    zq[1, 0, 7] += 1e-9                       # differs from p by far less than its error
    res = chain_accept(zp, zq, np.array([[-1], [-1]]), np.array([[0.5], [0.5]]),
                       np.array([[0.4, 0.4], [0.4, 0.4]]))
    assert np.all(res.num_accepted == 0)
    assert not res.empty_ambiguous[0] and res.empty_ambiguous[1]


def test_sampled_tree_boundaries_and_admissible_outcomes():
    # root with two children; p_0 = [0.25, 0.75], q_0 = [0.5, 0.5]
    zp = np.log(np.array([[[0.25, 0.75], [0.5, 0.5], [0.5, 0.5]]]))
    zq = np.log(np.array([[[0.5, 0.5], [0.5, 0.5], [0.5, 0.5]]]))
    tok = np.array([[0, 0, 1]])
    par = np.array([[-1, 0, 0]])
    ud = np.array([[0.3, 0.3, 0.3]])
    # child 1 (token 0): r = 0.5; u on it -> flagged, both outcomes admissible
    ua = np.array([[0.5, 0.5, 0.99]])
    res = tree_accept_sampled(zp, zq, tok, par, ua, ud, band=0.0)
    assert res.flags[0] and res.flags[0][0].kind == "accept" and res.flags[0][0].index == 1
    alts = tree_sampled_admissible(zp, zq, tok, par, ua, ud, 0, band=0.0)
    # kept: node 1, then a draw from p_1 at 0.3 -> token 0.  Rejected: the
    # residual (p - q)+ = [0, 0.25] / 0.25 = [0, 1]; child 2 (token 1) has
    # r = 1 / 0.5 = 2 and is kept; node 2 is a leaf: draw from p_2 -> token 0
    assert (1, (0, 1, -1), (0, 0, -1)) in alts
    assert (1, (0, 2, -1), (1, 0, -1)) in alts
    assert len(alts) == 2
    ua = np.array([[0.5, 0.2, 0.99]])
    assert tree_sampled_admissible(zp, zq, tok, par, ua, ud, 0) == \
        {(1, (0, 1, -1), (0, 0, -1))}
