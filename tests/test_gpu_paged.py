"""GPU parity of spec_verify_attention_paged.

* Equal prefix lengths: the paged kernel must be bit-identical to the
  contiguous spec_verify_attention on the same logical cache (same launch
  plan, same arithmetic; only the addresses differ), for every page size and
  both page layouts.  The contiguous kernel is itself parity-tested against
  the oracle.
* Ragged prefix lengths: compared element by element with oracle.paged at
  reduced sizes (several splits, so that short sequences leave whole splits
  empty), and on sampled rows at the full large-batch size.  Tolerances:
  max-abs 1e-4 for fp32 inputs, 2e-2 for bf16 K/V.

Everything in the page pool that no sequence owns is NaN, so a read of it
would show up as a non-finite output.
"""
import zlib

import numpy as np
import pytest
import torch

from gpu_support import assert_attention_close, device, f64, say
from oracle.paged import verify_attention_paged
from verify_pass_rejection_amd import inputs as I
from verify_pass_rejection_amd import native as nat

pytestmark = pytest.mark.gpu


def _parents(w, dev):
    if w.kind != "tree":
        return None
    return I.make_tree_inputs(w.with_(V=8), dev)["parents"]


def _equal_to_contiguous(w, page_size, layout, lens_given=False):
    dev = device()
    q, k, v = I.make_attention_inputs(w, dev)
    par = _parents(w, dev)
    kp, vp, bt = I.make_paged_kv(w, k, v, page_size, layout)
    lens = torch.full((w.B,), w.ctx, dtype=torch.int32, device=dev) if lens_given else None
    say(w.name, f"ps={page_size} {layout} B={w.B} T={w.T} ctx={w.ctx} D={w.D} {w.dtype}")
    want = nat.spec_verify_attention(q, k, v, w.ctx, parents=par)
    got = nat.spec_verify_attention_paged(q, kp, vp, bt, w.ctx, ctx_lens=lens, parents=par,
                                          layout=layout)
    torch.cuda.synchronize()
    assert torch.isfinite(got).all()
    assert torch.equal(got, want)


@pytest.mark.parametrize("page_size", [1, 16, 32, 256])
@pytest.mark.parametrize("layout", ["hnd", "nhd"])
def test_chain_bitwise_equal_to_contiguous(page_size, layout):
    w = I.WORKLOADS["large_batch_chain"].with_(B=3, ctx=1500, seed=31)
    _equal_to_contiguous(w, page_size, layout)


@pytest.mark.parametrize("name,kw,page_size", [
    ("eagle2_tree", dict(B=2, ctx=700), 16),                     # two row tiles per wave
    ("medusa70b_tree", dict(B=2, ctx=300), 8),                   # three row tiles, lagging waves
    ("llama3_8b_chain", dict(B=2, ctx=1000), 64),
    ("tiny_chain", dict(B=2), 4),                                # fp32: VALU kernel
    ("large_batch_chain", dict(B=2, T=8, Hq=16, Hkv=4, D=64, ctx=450), 2),   # D = 64
    ("large_batch_chain", dict(B=64, T=5, ctx=187), 16),         # one split per unit
])
def test_workloads_bitwise_equal_to_contiguous(name, kw, page_size):
    w = I.WORKLOADS[name].with_(**kw)
    _equal_to_contiguous(w, page_size, "hnd", lens_given=True)


def _ragged_case(w, page_size, layout, rows=None, atol=None):
    dev = device()
    q, k, v = I.make_attention_inputs(w, dev)
    par = _parents(w, dev)
    lens = I.ragged_ctx_lens(w, dev)
    kp, vp, bt = I.make_paged_kv(w, k, v, page_size, layout, lens.cpu())
    say(w.name, f"ragged ps={page_size} {layout} lens={lens.cpu().tolist()[:8]}")
    out = nat.spec_verify_attention_paged(q, kp, vp, bt, w.ctx, ctx_lens=lens, parents=par,
                                          layout=layout)
    torch.cuda.synchronize()
    parn = None if par is None else par.cpu().numpy()
    lens_n = lens.cpu().numpy()
    if rows is None:
        want = verify_attention_paged(f64(q), f64(kp), f64(vp), bt.cpu().numpy(), lens_n,
                                      parn, layout)
        got = f64(out)
    else:
        # per sampled sequence, only its own pages go to the host (relabelled
        # 0..n-1, which leaves the result unchanged)
        got, want = [], []
        for b in sorted({r[0] for r in rows}):
            n = (int(lens_n[b]) + w.T + page_size - 1) // page_size
            ids = bt[b, :n].long()
            sub = [(0, t, h) for (bb, t, h) in rows if bb == b]
            o = verify_attention_paged(
                f64(q[b:b + 1]), f64(kp[ids]), f64(vp[ids]), np.arange(n)[None], lens_n[b:b + 1],
                None if parn is None else parn[b:b + 1], layout, rows=sub)
            for (_, t, h) in sub:
                want.append(o[0, t, h])
                got.append(f64(out[b, t, h]))
        got, want = np.array(got), np.array(want)
    assert_attention_close(got, want, w.dtype, label=w.name, atol=atol)


@pytest.mark.parametrize("name,kw,page_size,layout", [
    ("large_batch_chain", dict(B=4, ctx=2000), 16, "hnd"),
    ("large_batch_chain", dict(B=5, ctx=1200), 1, "nhd"),
    ("eagle2_tree", dict(B=3, ctx=900), 32, "nhd"),
    ("medusa70b_tree", dict(B=3, ctx=400), 64, "hnd"),
    ("tiny_chain", dict(B=4, ctx=700), 8, "nhd"),                # fp32
    ("large_batch_chain", dict(B=4, T=32, Hq=64, Hkv=8, D=64, ctx=333), 4, "hnd"),
])
def test_ragged_lengths_elementwise(name, kw, page_size, layout):
    _ragged_case(I.WORKLOADS[name].with_(**kw), page_size, layout)


def test_full_size_ragged_sampled_rows():
    w = I.WORKLOADS["large_batch_chain"]
    rng = np.random.default_rng(zlib.crc32(b"paged"))
    rows = sorted({(int(rng.integers(w.B)), int(rng.integers(w.T)), int(rng.integers(w.Hq)))
                   for _ in range(16)})
    rows += [(0, w.T - 1, w.Hq - 1), (w.B - 1, 0, 0)]         # longest and empty prefix
    _ragged_case(w, 16, "hnd", rows=rows)
    torch.cuda.empty_cache()


def test_full_size_bitwise_equal_to_contiguous():
    _equal_to_contiguous(I.WORKLOADS["large_batch_chain"], 16, "hnd")
    torch.cuda.empty_cache()
