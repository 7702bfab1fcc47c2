"""GPU parity of spec_ngram_propose against oracle.ngram (bit-exact: token ids
and counts).  Histories: the seeded repetitive recipe, small vocabularies
(matches of every length), lengths that straddle the 4096-position tiles,
and the degenerate cases (empty, one token, a constant run, N = 0)."""
import numpy as np
import pytest
import torch

from gpu_support import device, i64, say
from oracle.ngram import ngram_propose
from verify_pass_rejection_amd import inputs as I
from verify_pass_rejection_amd import native as nat

pytestmark = pytest.mark.gpu


def compare(ctx, lens, N, n_min, n_max, label="", pass_lens=True):
    num, drafts = nat.spec_ngram_propose(ctx, N, n_min, n_max,
                                         context_lens=lens if pass_lens else None)
    torch.cuda.synchronize()
    L = ctx.shape[1]
    lens_h = i64(lens) if pass_lens else np.full(ctx.shape[0], L)
    want_n, want_d, _ = ngram_propose(i64(ctx), lens_h, N, n_min, n_max)
    num, drafts = i64(num), i64(drafts)
    say(label, f"B={ctx.shape[0]} L={L} N={N} n={n_min}..{n_max}",
        f"with drafts={int((want_n > 0).sum())} mean={want_n.mean():.2f}")
    assert np.array_equal(num, want_n)
    assert np.array_equal(drafts, want_d)


@pytest.mark.parametrize("kw,N,n_min,n_max", [
    (dict(B=16, ctx=5000), 8, 1, 4),
    (dict(B=16, ctx=9000, V=50), 8, 2, 6),          # small vocabulary: long matches
    (dict(B=8, ctx=4097, V=7), 5, 1, 16),           # the largest n-gram, 2 tiles
    (dict(B=8, ctx=8194, V=3), 63, 3, 3),           # tile edges, the most drafts
])
def test_matches_oracle(kw, N, n_min, n_max):
    dev = device()
    w = I.WORKLOADS["large_batch_chain"].with_(**kw, seed=51)
    ctx, lens = I.make_ngram_inputs(w, dev)
    compare(ctx, lens, N, n_min, n_max, label=str(kw))


def test_full_size_sampled_sequences():
    dev = device()
    w = I.WORKLOADS["large_batch_chain"]
    ctx, lens = I.make_ngram_inputs(w, dev)
    num, drafts = nat.spec_ngram_propose(ctx, 8, 1, 4, context_lens=lens)
    torch.cuda.synchronize()
    pick = [0, 1, 17, 33, 50, w.B - 1]
    want_n, want_d, _ = ngram_propose(i64(ctx[pick]), i64(lens[pick]), 8, 1, 4)
    say(f"full size: {int((i64(num) > 0).sum())} of {w.B} sequences with drafts")
    assert np.array_equal(i64(num)[pick], want_n)
    assert np.array_equal(i64(drafts)[pick], want_d)


def test_degenerate_histories():
    dev = device()
    g = torch.Generator().manual_seed(3)
    ctx = torch.randint(0, 4, (6, 20), generator=g, dtype=torch.int32)
    ctx[3] = 9                                       # a constant run
    lens = torch.tensor([0, 1, 2, 20, 5, 13], dtype=torch.int32)
    compare(ctx.to(dev), lens.to(dev), 4, 1, 3, label="short and constant")
    compare(ctx.to(dev), lens.to(dev), 0, 1, 3, label="N = 0")
    compare(ctx.to(dev), lens.to(dev), 4, 1, 3, label="lengths NULL", pass_lens=False)
    # no repeats at all
    ctx = torch.arange(0, 3 * 5000, dtype=torch.int32).view(3, 5000)
    compare(ctx.to(dev), torch.full((3,), 5000, dtype=torch.int32).to(dev), 8, 1, 4,
            label="no repeats")


@pytest.mark.parametrize("ctx_len,V,N,n_min,n_max", [
    (32768, 50, 8, 1, 4),        # the longest history one block holds
    (32769, 50, 8, 1, 4),        # one token more: the tiled two-kernel path
    (40000, 7, 63, 2, 16),       # tiled, the largest n-gram and the most drafts
    (32768, 2, 5, 1, 16),        # one block, two tokens: matches at almost every end
])
def test_history_length_paths(ctx_len, V, N, n_min, n_max):
    """Histories up to 32768 tokens are scanned by one block per sequence out
    of LDS, longer ones by tiles across blocks; both against the oracle."""
    dev = device()
    w = I.WORKLOADS["large_batch_chain"].with_(B=6, ctx=ctx_len, V=V, seed=61)
    ctx, lens = I.make_ngram_inputs(w, dev)
    compare(ctx, lens, N, n_min, n_max, label=f"L={ctx_len} V={V}")
    compare(ctx, lens, N, n_min, n_max, label=f"L={ctx_len} V={V} lengths NULL",
            pass_lens=False)

