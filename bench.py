"""Benchmark of the speculative-decoding verify step on one MI355X.

One step = one pass of the whole hot path over one batch: verify attention of
the N+1 draft positions against the KV cache (spec_verify_attention), then
rejection-sampling acceptance on every target/draft row (spec_accept_chain).
The workload is the large-batch chain: batch 64, N = 8 drafts, 32 query / 8 KV
heads, head_dim 128, bf16 KV with a 32768-token prefix, vocabulary 152064.

Printed: one JSON line with the step time, the achieved algorithmic HBM
bandwidth of the step, of attention and of acceptance, the per-position
verification overhead α = (T(N) − T(0)) / (N·T(0)) at N = 4 and 8 on the same
shape, a roofline entry for the attention kernel and the CPU oracle's rate on a
bounded sample of the same workload.  Beside the line's own figures: the
attention call over a paged copy of the same cache (pages of 16 positions),
the n-gram draft proposal over histories of the same batch and length, and
under "other_workloads" the other reference workloads at full size with the
cache flushed between steps (the Llama-3-8B-shaped chain with its alpha at
N = 4 and 8, the EAGLE-2 and Medusa trees with their matrix rate, KV commit
and sampled acceptance, and the tiny fp32 chain).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("verify-step µs + achieved HBM GB/s (attn, sampler) at N=4/8; α overhead")
HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0      # dense bf16 matrix peak (no sparsity)
WORKLOAD = "large_batch_chain"
ATTN_SOURCE = os.path.join(ROOT, "verify_pass_rejection_amd", "csrc", "attention.hip")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attention_large_batch_chain_hbm_traffic.txt")
COPY_CALIBRATION_BYTES = 1 << 30     # one plain copy of 1 GiB (read 1 GiB, write 1 GiB)


def attention_bytes(w) -> int:
    """Algorithmic bytes of one attention call: K and V of all ctx+T keys once,
    Q once, the fp32 output once."""
    esz = 4 if w.dtype == "f32" else 2
    kv = 2 * w.B * w.Hkv * w.L * w.D * esz
    return kv + w.B * w.T * w.Hq * w.D * esz + w.B * w.T * w.Hq * w.D * 4


def attention_flops(w) -> int:
    return 4 * w.D * (w.Hq // w.Hkv) * w.T * w.L * w.B * w.Hkv


def sampler_bytes(w) -> int:
    """Algorithmic bytes of acceptance: every logit once — target and draft rows
    for a chain, one target row per node for a tree."""
    if w.kind == "tree":
        return w.T * w.V * 4 * w.B
    return (2 * w.N + 1) * w.V * 4 * w.B


def alpha(t_n: float, t_0: float, n: int) -> float:
    """Per-position verification overhead (T(N) − T(0)) / (N·T(0))."""
    return (t_n - t_0) / (n * t_0)


class Step:
    """Device-resident inputs, outputs and workspaces for one workload."""

    def __init__(self, w, dev):
        import torch
        from verify_pass_rejection_amd import inputs as I
        from verify_pass_rejection_amd import native as nat
        self.w, self.nat = w, nat
        self.q, self.k, self.v = I.make_attention_inputs(w, dev)
        self.tree = w.kind == "tree"
        self.d = I.make_tree_inputs(w, dev) if self.tree else I.make_chain_inputs(w, dev)
        self.parents = self.d["parents"] if self.tree else None
        self.out = torch.empty((w.B, w.T, w.Hq, w.D), dtype=torch.float32, device=dev)
        self.num = torch.empty(w.B, dtype=torch.int32, device=dev)
        self.tok = torch.empty((w.B, w.T), dtype=torch.int32, device=dev)
        self.path = torch.empty((w.B, w.T), dtype=torch.int32, device=dev)
        self.new_len = torch.empty(w.B, dtype=torch.int32, device=dev)   # KV commit output
        dt = nat.SPEC_BF16 if w.dtype == "bf16" else nat.SPEC_F32
        self.ws_a = torch.empty(nat.spec_verify_attention_workspace(
            w.B, w.T, w.Hq, w.Hkv, w.D, w.ctx, dt), dtype=torch.uint8, device=dev)
        ws = (nat.spec_accept_tree_workspace(w.B, w.T, w.V) if self.tree
              else nat.spec_accept_chain_workspace(w.B, w.N, w.V))
        self.ws_c = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def attention(self):
        self.nat.spec_verify_attention(self.q, self.k, self.v, self.w.ctx, parents=self.parents,
                                       out=self.out, workspace=self.ws_a)

    def accept(self):
        d = self.d
        if self.tree:
            self.nat.spec_accept_tree(d["target_logits"], d["tokens"], d["parents"],
                                      accept_len=self.num, path=self.path, out_tokens=self.tok,
                                      workspace=self.ws_c)
        else:
            self.nat.spec_accept_chain(d["target_logits"], d["draft_logits"],
                                       d["draft_tokens"], d["u_accept"], d["u_draw"],
                                       num_accepted=self.num, out_tokens=self.tok,
                                       workspace=self.ws_c)

    def __call__(self):
        self.attention()
        self.accept()


def pct(xs, q: float) -> float:
    """q-quantile of xs (nearest rank)."""
    ys = sorted(xs)
    return ys[min(len(ys) - 1, max(0, int(round(q * (len(ys) - 1)))))]


def evict(flush):
    """Reads the whole buffer (larger than L2 + MALL) on the launch stream, so
    that the next call finds none of its inputs in a cache.  A read leaves
    clean lines: rewriting the buffer instead leaves dirty ones whose
    write-back then competes with the next call's reads (measured: medusa
    tree attention 106.5 us after a rewrite, 97.5 us after a read)."""
    import torch
    flush.view(torch.int32).sum()


def time_steps(step, steps: int, warmup: int, flush=None):
    """Warm up, then time exactly `steps` steps; per-call times from events on
    the stream the library launches on (torch's current stream).  With
    `flush` (a device buffer larger than L2 + MALL), the buffer is read before
    every step, outside the events, so that no step finds its inputs in a
    cache; the step time is then the sum of the per-call event times."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(steps):
        if flush is not None:
            evict(flush)
        ev[i][0].record()
        step.attention()
        ev[i][1].record()
        step.accept()
        ev[i][2].record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    attn = [e[0].elapsed_time(e[1]) for e in ev]
    acc = [e[1].elapsed_time(e[2]) for e in ev]
    tot = [e[0].elapsed_time(e[2]) for e in ev]
    per_step = start.elapsed_time(end) / steps if flush is None else sum(tot) / steps
    return dict(ms_per_step=per_step, wall_s=wall,
                attn_ms=sum(attn) / steps, accept_ms=sum(acc) / steps,
                attn_min_ms=min(attn), accept_min_ms=min(acc),
                attn_pct_ms=[pct(attn, q) for q in (0.1, 0.5, 0.9)],
                accept_pct_ms=[pct(acc, q) for q in (0.1, 0.5, 0.9)])


def time_commit(step, steps: int, flush=None):
    """spec_commit_kv after the tree acceptance of the last timed step (runs
    last: it rewrites the new positions of K/V in place; repeating it with the
    same path moves the same rows again, the same work).  Timed per call with
    events, flush as for the step: the flush read before each call also keeps
    the host's launch out of the event pair, as for the other per-call figures
    (a loop of back-to-back calls measures the Python binding instead)."""
    import torch
    w, nat = step.w, step.nat
    run = lambda: nat.spec_commit_kv(step.k, step.v, w.ctx, step.num, path=step.path,  # noqa: E731
                                     new_len=step.new_len)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        if flush is not None:
            evict(flush)
        ev[i][0].record()
        run()
        ev[i][1].record()
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) * 1e3 for a, b in ev]
    us = pct(ts, 0.5)
    esize = 2 if w.dtype == "bf16" else 4
    rows = int((step.num.clamp(0, w.T - 1) + 1).sum()) * w.Hkv
    moved = rows * w.D * esize * 2 * 2          # K and V rows, read and written
    return {"us": round(us, 2), "us_p10_p50_p90": [round(pct(ts, q), 2) for q in (0.1, 0.5, 0.9)],
            "bytes_moved": moved, "GBps": round(moved / (us * 1e-6) / 1e9, 2),
            "note": "latency-bound: a few hundred KB per call"}


def time_paged(step, steps: int, flush=None, page_size: int = 16, layout: str = "hnd"):
    """Attention over a paged copy of the same cache (spec_verify_attention_paged:
    pages of page_size positions in a shuffled pool, every prefix at ctx) and
    the contiguous call, each timed per call with events in 3 interleaved
    rounds (median of the round medians); the two outputs must be
    bit-identical."""
    import torch
    from verify_pass_rejection_amd import inputs as I
    w, nat = step.w, step.nat
    kp, vp, bt = I.make_paged_kv(w, step.k, step.v, page_size, layout)
    out = torch.empty_like(step.out)

    def paged():
        nat.spec_verify_attention_paged(step.q, kp, vp, bt, w.ctx, parents=step.parents,
                                        layout=layout, out=out, workspace=step.ws_a)

    def per_call(fn, n):
        for _ in range(2):
            fn()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        for i in range(n):
            if flush is not None:
                evict(flush)
            ev[i][0].record()
            fn()
            ev[i][1].record()
        torch.cuda.synchronize()
        return pct([a.elapsed_time(b) for a, b in ev], 0.5)

    rounds = {"paged": [], "contiguous": []}
    for _ in range(3):
        rounds["contiguous"].append(per_call(step.attention, max(10, steps // 3)))
        rounds["paged"].append(per_call(paged, max(10, steps // 3)))
    same = bool(torch.equal(out, step.out))
    del kp, vp, bt
    torch.cuda.empty_cache()
    ab = attention_bytes(w)
    us = pct(rounds["paged"], 0.5) * 1e3
    us_c = pct(rounds["contiguous"], 0.5) * 1e3
    return {"page_size": page_size, "layout": layout, "us": round(us, 2),
            "GBps": round(ab / (us * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round(ab / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "contiguous_us": round(us_c, 2), "bitwise_equal_to_contiguous": same}


def time_sampled_tree(w, dev, steps: int, flush=None):
    """spec_accept_tree_sampled on the same tree shape with draft rows (draft
    logits = target + N(0, 1) noise, children drawn from their parent's q),
    timed per call with events; flush as for the step.  Bytes of the
    statistics pass: every target row and the draft row of every node with
    children, once."""
    import torch
    from verify_pass_rejection_amd import inputs as I
    from verify_pass_rejection_amd import native as nat
    d = I.make_sampled_tree_inputs(w, dev)
    args = (d["target_logits"], d["draft_logits"], d["tokens"], d["parents"], d["u_accept"],
            d["u_draw"])
    al, path, out = nat.spec_accept_tree_sampled(*args)
    ws = torch.empty(max(1, nat.spec_accept_tree_sampled_workspace(w.B, w.T, w.V)),
                     dtype=torch.uint8, device=dev)
    run = lambda: nat.spec_accept_tree_sampled(*args, accept_len=al, path=path,  # noqa: E731
                                               out_tokens=out, workspace=ws)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        if flush is not None:
            evict(flush)
        ev[i][0].record()
        run()
        ev[i][1].record()
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) * 1e3 for a, b in ev]
    par = d["parents"].cpu()
    internal = sum(len(set(int(x) for x in par[b, 1:].tolist() if x >= 0)) for b in range(w.B))
    stats_bytes = (w.B * w.T + internal) * w.V * 4
    us = pct(ts, 0.5)
    return {"us": round(us, 2), "us_p10_p50_p90": [round(pct(ts, q), 2) for q in (0.1, 0.5, 0.9)],
            "mean_accepted": round(float(al.float().mean()), 3),
            "statistics_pass_bytes": stats_bytes,
            "note": "one block per sequence walks the tree; latency-bound beyond the "
                    "statistics pass"}


def time_ngram(w, dev, steps: int, flush=None, n_min: int = 1, n_max: int = 4):
    """spec_ngram_propose for the workload's batch: histories of ctx tokens
    (the seeded repetitive recipe, lengths in [ctx/2, ctx]), N = the
    workload's draft count; per-call events.  The histories (a few MB) would
    stay in the caches, so a 512 MB buffer is read before every call whatever
    the workload's own inputs: that keeps them cold and the host's launch out
    of the event pair (back-to-back calls time the Python binding instead).
    Bytes: every history token once."""
    import torch
    from verify_pass_rejection_amd import inputs as I
    from verify_pass_rejection_amd import native as nat
    if flush is None:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    ctx, lens = I.make_ngram_inputs(w, dev)
    num, drafts = nat.spec_ngram_propose(ctx, w.N, n_min, n_max, context_lens=lens)
    ws = torch.empty(max(1, nat.spec_ngram_propose_workspace(w.B, w.ctx)), dtype=torch.uint8,
                     device=dev)
    run = lambda: nat.spec_ngram_propose(ctx, w.N, n_min, n_max, context_lens=lens,  # noqa: E731
                                         num_drafts=num, drafts=drafts, workspace=ws)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        if flush is not None:
            evict(flush)
        ev[i][0].record()
        run()
        ev[i][1].record()
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) * 1e3 for a, b in ev]
    us = pct(ts, 0.5)
    nbytes = int(lens.long().sum()) * 4
    return {"us": round(us, 2), "us_p10_p50_p90": [round(pct(ts, q), 2) for q in (0.1, 0.5, 0.9)],
            "bytes": nbytes, "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "n_min": n_min, "n_max": n_max,
            "mean_drafts": round(float(num.float().mean()), 3),
            "note": "latency-bound: a few MB per call"}


def host_info():
    """CPU model and RAM of the host, from /proc."""
    model, ram = "unknown", 0
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal"):
                ram = int(line.split()[1]) * 1024
                break
    except OSError:
        pass
    return model, ram


def cpu_baseline(w, step, budget_s: float = 20.0, max_workers: int = 16):
    """The fp64 oracle on a bounded sample of the same workload, spread over
    the host's cores: one worker thread per core (at most max_workers, the
    host share of one GPU), BLAS held to one thread in each, every task one
    independent unit — a (sequence, KV head) attention unit over the whole
    prefix, or one sequence's chain acceptance over its 2N + 1 rows.
    Sequences are taken in order, a group of them at a time, until the budget
    is spent; the rate is the algorithmic bytes of the sequences done per
    second, host copies included."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from oracle.accept import chain_accept
    from oracle.attention import verify_attention

    workers = max(1, min(len(os.sched_getaffinity(0)), max_workers))
    G = w.Hq // w.Hkv
    d = step.d

    def f64(t):
        return t.to(torch.float64).numpy()

    def attention_unit(host, g):
        q, k, v = host
        verify_attention(f64(q[:, :, g * G:(g + 1) * G]), f64(k[:, g:g + 1]),
                         f64(v[:, g:g + 1]), w.ctx)

    def acceptance(host):
        zp, zq, x, ua, ud = host
        chain_accept(f64(zp), f64(zq), x.numpy(), f64(ua), f64(ud))

    group = max(1, workers // w.Hkv)
    n_seq = 0
    t0 = time.perf_counter()
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        while n_seq < w.B and time.perf_counter() - t0 < budget_s:
            seqs = range(n_seq, min(w.B, n_seq + group))
            futs = []
            for b in seqs:
                sl = slice(b, b + 1)
                host = (step.q[sl].cpu(), step.k[sl].cpu(), step.v[sl].cpu())
                futs += [ex.submit(attention_unit, host, g) for g in range(w.Hkv)]
                acc = (d["target_logits"][sl].cpu(), d["draft_logits"][sl].cpu(),
                       d["draft_tokens"][sl].cpu(), d["u_accept"][sl].cpu(),
                       d["u_draw"][sl].cpu())
                futs.append(ex.submit(acceptance, acc))
            for f in futs:
                f.result()
            n_seq += len(seqs)
    dt = time.perf_counter() - t0
    per_seq = (attention_bytes(w) + sampler_bytes(w)) / w.B
    model, ram = host_info()
    return {"value": round(per_seq * n_seq / dt / 1e9, 4), "unit": "GB/s", "cores": workers,
            "kind": "oracle",
            "sample": f"{n_seq} of {w.B} sequences of {w.name} (attention for all {w.Hq} heads "
                      f"x {w.T} positions over ctx {w.ctx}, then chain acceptance over "
                      f"{2 * w.N + 1} rows of V={w.V}); {workers} worker threads, one "
                      f"(sequence, KV head) unit or one sequence's acceptance per task, BLAS "
                      f"one thread each; host copies included; {dt:.1f} s",
            "host_cpus_visible": os.cpu_count(), "cpu_model": model, "host_ram_bytes": ram}


def source_sha256(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic():
    """HBM bytes per attention launch from the committed PMC summary, or None
    if there is none or the kernel source changed since it was taken.

    traffic = FETCH_SIZE * (copy bytes / copy FETCH_SIZE)
            + WRITE_SIZE * (copy bytes / copy WRITE_SIZE), per dispatch.
    """
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    kv = {}
    for line in open(TRAFFIC_PROFILE):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    try:
        if kv.get("attention_source_sha256") != source_sha256(ATTN_SOURCE):
            return None
        copy = float(kv["copy_bytes"])
        fetch = float(kv["attention_fetch_kib"]) * copy / float(kv["copy_fetch_kib"])
        write = float(kv["attention_write_kib"]) * copy / float(kv["copy_write_kib"])
        return int(round(fetch + write))
    except (KeyError, ValueError, ZeroDivisionError):
        return None


def copy_calibration(dev):
    """A plain device copy of a known size, for scaling the HBM byte counters."""
    import torch
    n = COPY_CALIBRATION_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def measure_alpha(w, dev, step, rounds: int, flush=None):
    """alpha at N = 4 and 8 on the workload's shape: T(N) for N = 0, 4, 8 and
    the workload's own N, interleaved two steps at a time over many rounds
    (the box's speed drifts by a few per cent over seconds, more than alpha
    itself); the median step time of each N enters alpha."""
    import torch
    ns = sorted({0, 4, 8, w.N})
    steps_n = {n: (step if n == w.N else Step(w.with_(T=n + 1), dev)) for n in ns}
    for n in ns:
        time_steps(steps_n[n], 1, 2, flush)
    per_n = {n: [] for n in ns}
    for _ in range(rounds):
        for n in ns:
            per_n[n].append(time_steps(steps_n[n], 2, 0, flush)["ms_per_step"])
    times = {n: pct(per_n[n], 0.5) for n in ns}
    steps_n = None
    torch.cuda.empty_cache()
    out = {f"alpha_N{n}": round(alpha(times[n], times[0], n), 4) for n in ns if n > 0}
    out["verify_step_us_by_N"] = {str(n): round(times[n] * 1e3, 2) for n in ns}
    return out


def flush_buffer(w, dev):
    """A 512 MB buffer to read between steps when the workload's inputs could
    stay in L2 + the 256 MB MALL (everything below 2 GB), else None."""
    import torch
    if attention_bytes(w) + sampler_bytes(w) < (2 << 30):
        return torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    return None


def step_figures(w, step, t):
    """Per-call figures of a timed workload: step, attention and acceptance
    times (mean and p10/p50/p90), algorithmic GB/s and fractions of the HBM
    peak, and the attention call's matrix rate against the bf16 MFMA peak."""
    ab, sb = attention_bytes(w), sampler_bytes(w)
    attn_gbps = ab / (t["attn_ms"] * 1e-3) / 1e9
    samp_gbps = sb / (t["accept_ms"] * 1e-3) / 1e9
    attn_tflops = attention_flops(w) / (t["attn_ms"] * 1e-3) / 1e12
    return {
        "verify_step_us": round(t["ms_per_step"] * 1e3, 2),
        "attn_us": round(t["attn_ms"] * 1e3, 2),
        "sampler_us": round(t["accept_ms"] * 1e3, 2),
        "attn_us_p10_p50_p90": [round(x * 1e3, 2) for x in t["attn_pct_ms"]],
        "sampler_us_p10_p50_p90": [round(x * 1e3, 2) for x in t["accept_pct_ms"]],
        "acceptance": "greedy tree" if w.kind == "tree" else "chain rejection sampling",
        "mean_accepted": round(float(step.num.float().mean()), 3),
        "attn_bytes": ab, "sampler_bytes": sb,
        "attn_GBps": round(attn_gbps, 1),
        "sampler_GBps": round(samp_gbps, 1),
        "attn_frac_hbm_peak": round(attn_gbps / HBM_PEAK_GBPS, 4),
        "sampler_frac_hbm_peak": round(samp_gbps / HBM_PEAK_GBPS, 4),
        "attn_TFLOPs": round(attn_tflops, 2),
        "attn_frac_bf16_mfma_peak": (round(attn_tflops / BF16_MFMA_PEAK_TFLOPS, 4)
                                     if w.dtype == "bf16" else None),
    }


def time_graph_replay(step, steps: int):
    """Back-to-back steps (attention then acceptance) with the inputs resident,
    eager against replays of the step captured once into a HIP graph through
    torch's graph API: one event pair around `steps` steps, in three
    alternating rounds, median per-step time of each.  On launch-bound shapes
    the host's launches set the eager rate and a replay removes them.  The
    replay's outputs are compared bit for bit with an eager step's."""
    import torch
    side = torch.cuda.Stream()                  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                  # first run outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
        step()
    torch.cuda.synchronize()

    def loop(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / steps

    eager, replay = [], []
    for _ in range(3):
        eager.append(loop(step))
        replay.append(loop(g.replay))
    g.replay()
    torch.cuda.synchronize()
    replayed = [t.clone() for t in (step.out, step.num, step.tok, step.path)]
    step()
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in zip(replayed, (step.out, step.num, step.tok,
                                                            step.path)))
    del g
    return {"eager_us": round(pct(eager, 0.5), 2), "graph_replay_us": round(pct(replay, 0.5), 2),
            "steps_per_round": steps, "bitwise_equal_to_eager": bool(same),
            "note": "back-to-back steps, inputs cache-resident"}


def measure_config(name, dev, steps: int, warmup: int, with_alpha: bool):
    """One of the other reference workloads at its full size, cache flushed
    between steps: the step figures, alpha on chains, and for trees the KV
    commit and the sampled (non-greedy) acceptance of the same tree shape."""
    import torch
    from verify_pass_rejection_amd import inputs as I
    w = I.WORKLOADS[name]
    flush = flush_buffer(w, dev)
    step = Step(w, dev)
    t = time_steps(step, steps, warmup, flush)
    out = {"config": {"batch": w.B, "N_or_T": w.N if w.kind == "chain" else w.T, "Hq": w.Hq,
                      "Hkv": w.Hkv, "head_dim": w.D, "ctx": w.ctx, "vocab": w.V,
                      "kv_dtype": w.dtype},
           "cache_flush_between_steps": flush is not None, **step_figures(w, step, t)}
    if w.dtype == "f32":
        out["note"] = "launch-bound correctness workload (1 MB of attention bytes)"
    if with_alpha and w.kind == "chain":
        out.update(measure_alpha(w, dev, step, max(40, steps), flush))
    out["back_to_back"] = time_graph_replay(step, steps)
    if w.kind == "tree":
        out["kv_commit"] = time_commit(step, steps, flush)
        out["sampled_tree_acceptance"] = time_sampled_tree(w, dev, steps, flush)
    del step, flush
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-alpha", action="store_true")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the paged-KV attention timing")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the headline workload, not the other reference workloads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling byte counters)")
    ap.add_argument("--workload", default=WORKLOAD,
                    help="reference workload to time (the bench line uses large_batch_chain; "
                         "the others are for per-kernel measurement)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the verify step shards with no exchange over batch or KV heads)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from verify_pass_rejection_amd import inputs as I

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(dev)
    w = I.WORKLOADS[args.workload]
    flush = flush_buffer(w, dev)
    step = Step(w, dev)
    t = time_steps(step, args.steps, args.warmup, flush)
    fig = step_figures(w, step, t)
    ab, sb = attention_bytes(w), sampler_bytes(w)
    step_gbps = (ab + sb) / (t["ms_per_step"] * 1e-3) / 1e9
    attn_gbps = fig["attn_GBps"]

    alphas = {}
    if not args.no_alpha and w.kind == "chain":
        alphas = measure_alpha(w, dev, step, max(40, args.steps), flush)

    paged = None if args.no_paged else time_paged(step, args.steps, flush)

    ngram = time_ngram(w, dev, args.steps, flush) if w.kind == "chain" and w.N > 0 else None

    commit = sampled = None
    if w.kind == "tree":
        commit = time_commit(step, args.steps, flush)
        sampled = time_sampled_tree(w, dev, args.steps, flush)

    cpu = None
    if not args.no_cpu_baseline and w.kind == "chain":
        cpu = cpu_baseline(w, step)
    flushed = flush is not None
    del step, flush
    torch.cuda.empty_cache()

    configs = {}
    if not args.no_configs:
        for name in I.WORKLOADS:
            if name != w.name:
                configs[name] = measure_config(name, dev, args.steps, args.warmup,
                                               with_alpha=not args.no_alpha)

    line = {
        "metric": METRIC,
        "value": round(step_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; stands in for the pages' unnamed chat/code workloads)",
        "config": {"workload": w.name, "batch": w.B, "N": w.N, "Hq": w.Hq, "Hkv": w.Hkv,
                   "head_dim": w.D, "ctx": w.ctx, "vocab": w.V, "kv_dtype": w.dtype},
        **fig,
        "cache_flush_between_steps": flushed,
        **alphas,
        "roofline": {"bound": "hbm", "achieved": attn_gbps, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(attn_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic() if w.name == WORKLOAD else None,
                     "kernel": ("attn_mfma_kernel (spec_verify_attention: one launch, one "
                                "split per (sequence, KV head))" if w.name == WORKLOAD else
                                "spec_verify_attention call: attn_mfma_kernel, or attn_valu_kernel "
                                "for fp32, plus attn_combine_kernel when the keys are split"),
                     "algorithmic_bytes_per_launch": ab},
        "cpu_baseline": cpu,
    }
    if paged is not None:
        line["paged_attention"] = paged
    if commit is not None:
        line["kv_commit"] = commit
    if sampled is not None:
        line["sampled_tree_acceptance"] = sampled
    if ngram is not None:
        line["ngram_proposal"] = ngram
    if configs:
        line["other_workloads"] = configs
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
