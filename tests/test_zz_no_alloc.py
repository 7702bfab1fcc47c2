"""spec_accept_chain_noalloc through the C ABI against spec_accept_chain.

The allocation-free entry point runs the same kernels with their scratch in
the library's static device array instead of a caller workspace, so on the
same inputs both give identical accepted lengths and tokens.  Three calls in a
row: the full large-batch chain (64 sequences, N = 8, V = 152064), then
smaller problems (a ragged vocabulary on the scalar-load path, and N = 0) that
find the previous call's contents in the shared array; and the call captured
into a HIP graph and replayed.
"""
import pytest
import torch

from gpu_support import device, say
from verify_pass_rejection_amd import inputs as I
from verify_pass_rejection_amd import native as nat

pytestmark = pytest.mark.gpu


def noalloc_call(d, B, N, V, temperature=1.0):
    """The C entry point itself, with outputs pre-filled with a sentinel."""
    dev = d["target_logits"].device
    num = torch.full((B,), -9, dtype=torch.int32, device=dev)
    out = torch.full((B, N + 1), -9, dtype=torch.int32, device=dev)
    ptr = lambda t: t.data_ptr() if t.numel() else None     # noqa: E731
    st = nat.load().spec_accept_chain_noalloc(
        ptr(d["target_logits"]), ptr(d["draft_logits"]), ptr(d["draft_tokens"]),
        ptr(d["u_accept"]), ptr(d["u_draw"]), float(temperature), num.data_ptr(),
        out.data_ptr(), B, N, V, torch.cuda.current_stream().cuda_stream)
    assert st == nat.SPEC_OK, nat.status_string(st)
    return num, out


@pytest.mark.parametrize("order", ["large_first"])
def test_noalloc_matches_workspace_entry_point(order):
    dev = device()
    cases = [dict(), dict(B=8, T=4, V=1001, seed=61), dict(B=16, T=1, V=5000, seed=62)]
    for kw in cases:
        w = I.WORKLOADS["large_batch_chain"].with_(**kw)
        say("noalloc", f"B={w.B} N={w.N} V={w.V}")
        d = I.make_chain_inputs(w, dev)
        ws = torch.full((nat.spec_accept_chain_workspace(w.B, w.N, w.V),), 0xFF,
                        dtype=torch.uint8, device=dev)
        want = nat.spec_accept_chain(d["target_logits"], d["draft_logits"], d["draft_tokens"],
                                     d["u_accept"], d["u_draw"], workspace=ws)
        got = noalloc_call(d, w.B, w.N, w.V)
        torch.cuda.synchronize()
        say("noalloc", f"mean_accepted={want[0].float().mean().item():.3f}")
        assert torch.equal(got[0], want[0])
        assert torch.equal(got[1], want[1])
        del d, ws
        torch.cuda.empty_cache()


def test_noalloc_refuses_problems_beyond_the_scratch():
    device()
    st = nat.load().spec_accept_chain_noalloc(1 << 12, 1 << 12, 1 << 12, 1 << 12, 1 << 12, 1.0,
                                              1 << 12, 1 << 12, 4096, 8, 152064, None)
    assert st == nat.SPEC_ERR_WORKSPACE


def test_noalloc_replayed_from_a_captured_graph():
    """What the entry point is for: captured into a HIP graph with nothing
    allocated inside the capture, then replayed with the uniforms rewritten
    in place between replays; every replay matches spec_accept_chain run
    eagerly with a workspace on the same inputs."""
    dev = device()
    w = I.WORKLOADS["llama3_8b_chain"].with_(B=8, seed=63)
    d = I.make_chain_inputs(w, dev)
    B, N, V = w.B, w.N, w.V
    num = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty((B, N + 1), dtype=torch.int32, device=dev)
    ptr = lambda t: t.data_ptr()                             # noqa: E731

    def step():
        st = nat.load().spec_accept_chain_noalloc(
            ptr(d["target_logits"]), ptr(d["draft_logits"]), ptr(d["draft_tokens"]),
            ptr(d["u_accept"]), ptr(d["u_draw"]), 1.0, ptr(num), ptr(out), B, N, V,
            torch.cuda.current_stream().cuda_stream)
        assert st == nat.SPEC_OK, nat.status_string(st)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                               # first call outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    gen = torch.Generator(device=dev).manual_seed(64)
    for rep in range(4):
        if rep:
            d["u_accept"].copy_(I.uniforms(tuple(d["u_accept"].shape), gen, dev))
            d["u_draw"].copy_(I.uniforms(tuple(d["u_draw"].shape), gen, dev))
        g.replay()
        torch.cuda.synchronize()
        got = (num.clone(), out.clone())
        want = nat.spec_accept_chain(d["target_logits"], d["draft_logits"], d["draft_tokens"],
                                     d["u_accept"], d["u_draw"])
        torch.cuda.synchronize()
        say("noalloc graph", f"replay {rep} mean_accepted={want[0].float().mean().item():.3f}")
        assert torch.equal(got[0], want[0]) and torch.equal(got[1], want[1])
