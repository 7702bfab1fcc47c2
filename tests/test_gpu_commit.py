"""GPU parity of spec_commit_kv against oracle.commit (bit-exact: a pure move).

Paths come from the oracle's greedy tree acceptance on the synthetic trees
(and from the GPU's own acceptance in one end-to-end case); chains move
nothing and only report the new length.
"""
import numpy as np
import pytest
import torch

from gpu_support import device, say
from oracle.accept import tree_accept
from oracle.commit import commit_kv
from verify_pass_rejection_amd import inputs as I
from verify_pass_rejection_amd import native as nat

pytestmark = pytest.mark.gpu


def _host(t):
    # bf16 has no numpy dtype: compare raw 16-bit patterns
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _tree_case(w):
    dev = device()
    _, k, v = I.make_attention_inputs(w, dev)
    d = I.make_tree_inputs(w.with_(V=64), dev)
    res = tree_accept(d["target_logits"].cpu().numpy(), d["tokens"].cpu().numpy(),
                      d["parents"].cpu().numpy())
    return k, v, res


@pytest.mark.parametrize("name,kw", [
    ("eagle2_reduced", dict(B=3, ctx=300)),
    ("medusa_reduced", dict(B=4, ctx=129)),
    ("eagle2_d64_f32", dict(B=2, ctx=77, D=64, dtype="f32")),
])
def test_tree_commit_matches_oracle(name, kw):
    base = "medusa70b_tree" if name.startswith("medusa") else "eagle2_tree"
    w = I.WORKLOADS[base].with_(**kw)
    k, v, res = _tree_case(w)
    want_k, want_v, want_n = commit_kv(_host(k), _host(v), w.ctx, res.accept_len, res.path)
    dev = k.device
    acc = torch.tensor(res.accept_len, dtype=torch.int32, device=dev)
    path = torch.tensor(res.path, dtype=torch.int32, device=dev)
    say(name, f"B={w.B} T={w.T} Hkv={w.Hkv} D={w.D} ctx={w.ctx} {w.dtype}",
        f"accept_len={list(res.accept_len)}")
    n = nat.spec_commit_kv(k, v, w.ctx, acc, path=path)
    torch.cuda.synchronize()
    assert np.array_equal(n.cpu().numpy(), want_n)
    assert np.array_equal(_host(k), want_k)
    assert np.array_equal(_host(v), want_v)


def test_chain_commit_moves_nothing():
    dev = device()
    w = I.WORKLOADS["large_batch_chain"].with_(B=3, ctx=50)
    _, k, v = I.make_attention_inputs(w, dev)
    k0, v0 = k.clone(), v.clone()
    acc = torch.tensor([0, 4, 8], dtype=torch.int32, device=dev)
    n = nat.spec_commit_kv(k, v, w.ctx, acc)
    torch.cuda.synchronize()
    assert n.tolist() == [51, 55, 59]
    assert torch.equal(k, k0) and torch.equal(v, v0)


def test_invalid_entries_and_clamped_length():
    dev = device()
    w = I.WORKLOADS["eagle2_tree"].with_(B=2, T=8, ctx=10, Hkv=2, Hq=4)
    _, k, v = I.make_attention_inputs(w, dev)
    k0 = k.clone()
    # sequence 0: path 0, 3, then an out-of-range entry (row 2 left as it is);
    # sequence 1: accept_len beyond T-1 is clamped to T-1 with the identity path
    path = torch.tensor([[0, 3, 99, -1, -1, -1, -1, -1], list(range(8))],
                        dtype=torch.int32, device=dev)
    acc = torch.tensor([2, 50], dtype=torch.int32, device=dev)
    n = nat.spec_commit_kv(k, v, w.ctx, acc, path=path)
    torch.cuda.synchronize()
    assert n.tolist() == [10 + 3, 10 + 8]
    assert torch.equal(k[0, :, 10], k0[0, :, 10])
    assert torch.equal(k[0, :, 11], k0[0, :, 13])
    assert torch.equal(k[0, :, 12], k0[0, :, 12])
    assert torch.equal(k[1], k0[1])


def test_end_to_end_with_gpu_acceptance_full_size():
    # medusa at its real size: the GPU's own tree acceptance feeds the commit
    dev = device()
    w = I.WORKLOADS["medusa70b_tree"]
    _, k, v = I.make_attention_inputs(w, dev)
    d = I.make_tree_inputs(w, dev)
    acc, path, _ = nat.spec_accept_tree(d["target_logits"], d["tokens"], d["parents"])
    rows = (w.ctx + path.clamp(min=0)).long()                    # [B, T]
    want_k = torch.stack([k[b][:, rows[b]] for b in range(w.B)])  # [B, Hkv, T, D]
    n = nat.spec_commit_kv(k, v, w.ctx, acc, path=path)
    torch.cuda.synchronize()
    for b in range(w.B):
        l = int(acc[b])
        assert int(n[b]) == w.ctx + l + 1
        assert torch.equal(k[b, :, w.ctx: w.ctx + l + 1], want_k[b, :, : l + 1])
    torch.cuda.empty_cache()
