"""Pins of oracle.paged (verify attention over a paged KV cache) against
things other than its own gather: the seeded scatter of a contiguous cache
into a shuffled page pool (a separate routine, written the other way round)
followed by the contiguous oracle, which is pinned on its own; the special
cases of one page per sequence and of one position per page; invariance under
a relabelling of the physical pages; and NaN poison in everything no sequence
owns.  A planted mistake in the gather (a shifted in-page offset) must fail
the pins.
"""
import numpy as np
import pytest

import oracle.paged as OP
from oracle.attention import verify_attention
from verify_pass_rejection_amd import inputs as I


def _case(B=3, T=5, Hq=4, Hkv=2, D=8, ctx=13, seed=21):
    w = I.WORKLOADS["tiny_chain"].with_(B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, ctx=ctx, seed=seed)
    q, k, v = I.make_attention_inputs(w)
    return w, q.double().numpy(), k, v


def _tree_parents(B, T, seed):
    rng = np.random.default_rng(seed)
    return np.array([[-1] + [int(rng.integers(max(0, i - 3), i)) for i in range(1, T)]
                     for _ in range(B)])


@pytest.mark.parametrize("layout", ["hnd", "nhd"])
@pytest.mark.parametrize("ps", [1, 4, 16])
def test_shuffled_pages_equal_the_contiguous_cache(layout, ps):
    w, q, k, v = _case()
    par = _tree_parents(w.B, w.T, 3)
    kp, vp, bt = I.make_paged_kv(w, k, v, ps, layout)
    ctx = np.full(w.B, w.ctx)
    got = OP.verify_attention_paged(q, kp.numpy(), vp.numpy(), bt.numpy(), ctx, par, layout)
    want = verify_attention(q, k.double().numpy(), v.double().numpy(), w.ctx, parents=par)
    assert np.array_equal(got, want)


def test_one_page_per_sequence_is_the_contiguous_layout():
    # with page_size = ctx + T, head-major pages are exactly the [Hkv, L, D]
    # block of each sequence
    w, q, k, v = _case(seed=22)
    L = w.ctx + w.T
    kp = k.double().numpy()
    vp = v.double().numpy()
    table = np.arange(w.B)[:, None]
    got = OP.verify_attention_paged(q, kp, vp, table, np.full(w.B, w.ctx), None, "hnd")
    assert kp.shape[2] == L
    assert np.array_equal(got, verify_attention(q, kp, vp, w.ctx))


def test_ragged_lengths_equal_each_sequence_alone():
    w, q, k, v = _case(B=4, ctx=19, seed=23)
    lens = I.ragged_ctx_lens(w).numpy()
    assert lens[0] == w.ctx and lens[-1] == 0
    kp, vp, bt = I.make_paged_kv(w, k, v, 4, "hnd", lens)
    got = OP.verify_attention_paged(q, kp.numpy(), vp.numpy(), bt.numpy(), lens, None, "hnd")
    kd, vd = k.double().numpy(), v.double().numpy()
    for b in range(w.B):
        c = int(lens[b])
        want = verify_attention(q[b:b + 1], kd[b:b + 1, :, :c + w.T], vd[b:b + 1, :, :c + w.T], c)
        assert np.array_equal(got[b], want[0])
    assert np.all(np.isfinite(got))          # the NaN poison is never read


def test_relabelling_the_physical_pages_changes_nothing():
    w, q, k, v = _case(seed=24)
    kp, vp, bt = I.make_paged_kv(w, k, v, 4, "nhd")
    kp, vp, bt = kp.numpy(), vp.numpy(), bt.numpy()
    P = kp.shape[0]
    relabel = np.random.default_rng(5).permutation(P)      # old page p -> new page relabel[p]
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[relabel], vp2[relabel] = kp, vp
    ctx = np.full(w.B, w.ctx)
    a = OP.verify_attention_paged(q, kp, vp, bt, ctx, None, "nhd")
    b = OP.verify_attention_paged(q, kp2, vp2, relabel[bt], ctx, None, "nhd")
    assert np.array_equal(a, b)


def test_sampled_rows_match_the_full_output():
    w, q, k, v = _case(seed=25)
    kp, vp, bt = I.make_paged_kv(w, k, v, 8, "hnd")
    ctx = np.full(w.B, w.ctx)
    full = OP.verify_attention_paged(q, kp.numpy(), vp.numpy(), bt.numpy(), ctx)
    rows = [(0, 1, 3), (2, 4, 0)]
    part = OP.verify_attention_paged(q, kp.numpy(), vp.numpy(), bt.numpy(), ctx, rows=rows)
    for (b, t, h) in rows:
        assert np.array_equal(part[b, t, h], full[b, t, h])


def test_a_planted_offset_mistake_fails_the_pins(monkeypatch):
    real = OP.gather_sequence

    def shifted(pages, table_row, length, layout):
        out = real(pages, table_row, length, layout)
        return np.roll(out, 1, axis=1)       # every position reads its neighbour's row

    monkeypatch.setattr(OP, "gather_sequence", shifted)
    with pytest.raises(AssertionError):
        test_shuffled_pages_equal_the_contiguous_cache("hnd", 4)
