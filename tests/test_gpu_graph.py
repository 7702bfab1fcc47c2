"""The verify step replayed from a captured HIP graph.

An entry point only enqueues kernels on the caller's stream (no allocation,
no memset, no host synchronisation), so a caller can capture a whole verify
step, attention then acceptance, into one graph and replay it; at small sizes
the step is bound by launch latency, which a graph removes.  Each test replays
its graph several times, rewrites the inputs in place between replays (the
graph reads them afresh), runs the same step eagerly after every replay, with
other torch work and synchronisations in between, and compares the replay's
outputs with the eager ones bit for bit.
"""
import pytest
import torch

from gpu_support import device, say
from verify_pass_rejection_amd import inputs as I
from verify_pass_rejection_amd import native as nat

pytestmark = pytest.mark.gpu

REPLAYS = 4


def capture(step):
    side = torch.cuda.Stream()                       # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                       # first run outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def workspace(nbytes, dev):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=dev)


def time_us(fn, reps=50):
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        e.synchronize()
        ts.append(s.elapsed_time(e) * 1e3)
    return sorted(ts)[reps // 2]


def replay_and_compare(name, step, outputs, perturb):
    g = capture(step)
    gen = torch.Generator(device=outputs[0].device).manual_seed(11)
    for rep in range(REPLAYS):
        if rep:
            perturb(rep, gen)
        say(name, f"replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outputs]
        for t in outputs:
            t.fill_(-7)                              # the eager run must rewrite them
        torch.randn(1 << 20, device=t.device).sum().item()   # unrelated eager work
        step()
        torch.cuda.synchronize()
        for a, b in zip(got, outputs):
            assert torch.equal(a, b), f"{name}: replay {rep} differs from the eager step"
    eager, graph = time_us(step), time_us(g.replay)
    say(name, f"step median: eager {eager:.1f} us, graph replay {graph:.1f} us")


def test_chain_step_graph_replay():
    dev = device()
    w = I.WORKLOADS["llama3_8b_chain"]
    q, k, v = I.make_attention_inputs(w, dev)
    d = I.make_chain_inputs(w, dev)
    B, T, Hq, D = q.shape
    Hkv, N = k.shape[1], T - 1
    out = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
    num = torch.empty(B, dtype=torch.int32, device=dev)
    toks = torch.empty((B, N + 1), dtype=torch.int32, device=dev)
    ws_a = workspace(nat.spec_verify_attention_workspace(B, T, Hq, Hkv, D, w.ctx), dev)
    ws_c = workspace(nat.spec_accept_chain_workspace(B, N, w.V), dev)

    def step():
        nat.spec_verify_attention(q, k, v, w.ctx, out=out, workspace=ws_a)
        nat.spec_accept_chain(d["target_logits"], d["draft_logits"], d["draft_tokens"],
                              d["u_accept"], d["u_draw"], num_accepted=num, out_tokens=toks,
                              workspace=ws_c)

    def perturb(rep, gen):
        q.neg_()                                     # exact in bf16
        d["u_accept"].copy_(I.uniforms(tuple(d["u_accept"].shape), gen, dev))
        d["u_draw"].copy_(I.uniforms(tuple(d["u_draw"].shape), gen, dev))

    replay_and_compare("chain step (llama3_8b_chain)", step, [out, num, toks], perturb)


def test_tree_step_graph_replay():
    dev = device()
    w = I.WORKLOADS["eagle2_tree"]
    q, k, v = I.make_attention_inputs(w, dev)
    d = I.make_tree_inputs(w, dev)
    B, T, Hq, D = q.shape
    Hkv, V = k.shape[1], w.V
    out = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
    al = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.empty((B, T), dtype=torch.int32, device=dev)
    toks = torch.empty((B, T), dtype=torch.int32, device=dev)
    ws_a = workspace(nat.spec_verify_attention_workspace(B, T, Hq, Hkv, D, w.ctx), dev)
    ws_t = workspace(nat.spec_accept_tree_workspace(B, T, V), dev)

    def step():
        nat.spec_verify_attention(q, k, v, w.ctx, parents=d["parents"], out=out, workspace=ws_a)
        nat.spec_accept_tree(d["target_logits"], d["tokens"], d["parents"], accept_len=al,
                             path=path, out_tokens=toks, workspace=ws_t)

    def perturb(rep, gen):
        q.neg_()
        # drop the plants of one sequence: its argmax path changes
        d["target_logits"][rep % B].mul_(-1.0)

    replay_and_compare("tree step (eagle2_tree)", step, [out, al, path, toks], perturb)
