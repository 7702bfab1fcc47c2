"""Seeded synthetic workloads for the verify step.

This module holds the workload shapes and the seeded generators that feed
both the HIP path and the CPU oracle.  It holds none of the verify step's own
arithmetic: no softmax, no ratio test, no inverse-CDF draw, no argmax.  Draft
tokens are drawn from q with the Gumbel-max trick (argmax of logits plus
Gumbel noise); this stands in for the drafter, which is outside the verify
step.  Tree tokens are planted by raising one logit of the parent's row rather
than by reading the row's argmax.

The pages benchmark on unnamed chat and code workloads ("LLM Primer VI —
Chapitre 9 — Décodage spéculatif", §9.2) and name no dataset; these seeded
inputs stand in for them.

Every tensor comes from its own named substream so that changing one input's
recipe does not move the others.  A generator's stream depends on the device
(torch's CPU and GPU generators differ); tests that compare against the oracle
generate once and copy the same tensors to the host.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

# Named substreams: a per-input offset added to the workload seed.
_STREAMS = {"q": 1, "k": 2, "v": 3, "target": 4, "draft_noise": 5,
            "draft_gumbel": 6, "u_accept": 7, "u_draw": 8, "tree": 9,
            "tree_tokens": 10, "ctx_lens": 11, "pages": 12, "stree_gumbel": 13,
            "ngram": 14}

#: Spike written into a parent's logit row at the planted child's token, in
#: units of the logit standard deviation (8σ is never reached by N(0, σ²)
#: samples in practice, so the planted token is that row's maximum).
PLANT_SIGMAS = 8.0


@dataclass(frozen=True)
class Workload:
    """One verify-step workload.

    kind: "chain" (N drafts, T = N + 1 query positions) or "tree" (T nodes,
    node 0 the root).  Q is [B, T, Hq, D]; K and V are [B, Hkv, ctx + T, D];
    logits are fp32 [B, rows, V].
    """
    name: str
    kind: str
    B: int
    T: int
    Hq: int
    Hkv: int
    D: int
    ctx: int
    dtype: str            # "f32" or "bf16" (Q, K and V)
    V: int
    target_sd: float
    draft_noise_sd: float = 0.0
    tree: str = ""        # "eagle2" or "medusa"
    tree_widths: tuple = field(default_factory=tuple)
    plant_prob: float = 0.8
    temperature: float = 1.0
    seed: int = 0

    @property
    def N(self) -> int:
        return self.T - 1

    @property
    def L(self) -> int:
        return self.ctx + self.T

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


#: The five reference workloads.  "~N(0, s)" in their descriptions is read
#: with s the standard deviation.
WORKLOADS = {
    "tiny_chain": Workload(
        "tiny_chain", "chain", B=1, T=5, Hq=8, Hkv=8, D=64, ctx=256, dtype="f32",
        V=1024, target_sd=2.0, draft_noise_sd=0.5, seed=1),
    "llama3_8b_chain": Workload(
        "llama3_8b_chain", "chain", B=1, T=6, Hq=32, Hkv=8, D=128, ctx=4096,
        dtype="bf16", V=128256, target_sd=3.0, draft_noise_sd=1.0, seed=2),
    "eagle2_tree": Workload(
        "eagle2_tree", "tree", B=8, T=64, Hq=32, Hkv=8, D=128, ctx=8192, dtype="bf16",
        V=32000, target_sd=3.0, tree="eagle2", tree_widths=(1, 4, 12, 12, 12, 12, 11),
        seed=3),
    "medusa70b_tree": Workload(
        "medusa70b_tree", "tree", B=32, T=42, Hq=64, Hkv=8, D=128, ctx=2048,
        dtype="bf16", V=32000, target_sd=3.0, tree="medusa", tree_widths=(4, 3, 2, 1),
        seed=4),
    "large_batch_chain": Workload(
        "large_batch_chain", "chain", B=64, T=9, Hq=32, Hkv=8, D=128, ctx=32768,
        dtype="bf16", V=152064, target_sd=3.0, draft_noise_sd=1.0, seed=5),
}


def _gen(w: Workload, stream: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 1000 + _STREAMS[stream])
    return g


def uniforms(shape, g: torch.Generator, device) -> torch.Tensor:
    """fp32 uniforms k / 2^24 with k uniform in [1, 2^24 - 1]: exact, never 0 or 1."""
    k = torch.randint(1, 1 << 24, shape, generator=g, device=device, dtype=torch.int64)
    return (k.to(torch.float64) / float(1 << 24)).to(torch.float32)


def _normal(shape, g, device, dtype, sd=1.0, chunk_dim0=True) -> torch.Tensor:
    """N(0, sd²) samples, generated in fp32 one leading slice at a time (to
    bound temporary memory for multi-GB tensors) and then cast."""
    out = torch.empty(shape, dtype=dtype, device=device)
    for i in range(shape[0]):
        x = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32)
        if sd != 1.0:
            x.mul_(sd)
        out[i].copy_(x)
    return out


def make_attention_inputs(w: Workload, device="cpu"):
    """q [B,T,Hq,D], k and v [B,Hkv,ctx+T,D] in the workload's dtype, N(0, 1)."""
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    q = _normal((w.B, w.T, w.Hq, w.D), _gen(w, "q", device), device, dt)
    k = _normal((w.B, w.Hkv, w.L, w.D), _gen(w, "k", device), device, dt)
    v = _normal((w.B, w.Hkv, w.L, w.D), _gen(w, "v", device), device, dt)
    return q, k, v


def make_chain_inputs(w: Workload, device="cpu"):
    """Logits, drafts and uniforms for chain acceptance.

    target logits ~ N(0, target_sd²); draft logits = target rows 0..N-1 plus
    N(0, draft_noise_sd²) noise; draft tokens ~ softmax(draft/τ) by Gumbel-max;
    u_accept [B, N] and u_draw [B, N+1] uniforms k / 2^24.
    """
    B, N, V = w.B, w.N, w.V
    target = _normal((B, N + 1, V), _gen(w, "target", device), device, torch.float32,
                     sd=w.target_sd)
    noise = _normal((B, max(N, 1), V), _gen(w, "draft_noise", device), device,
                    torch.float32, sd=w.draft_noise_sd)[:, :N]
    draft = (target[:, :N] + noise).contiguous()
    gumbel_u = uniforms((B, N, V), _gen(w, "draft_gumbel", device), device)
    gumbel = -torch.log(-torch.log(gumbel_u.double()))
    tokens = torch.argmax(draft.double() / w.temperature + gumbel, dim=-1).to(torch.int32)
    u_accept = uniforms((B, N), _gen(w, "u_accept", device), device)
    u_draw = uniforms((B, N + 1), _gen(w, "u_draw", device), device)
    return dict(target_logits=target, draft_logits=draft, draft_tokens=tokens.contiguous(),
                u_accept=u_accept, u_draw=u_draw)


def eagle2_parents(widths, g: torch.Generator) -> list[int]:
    """Nodes numbered depth by depth; each node's parent is uniform over the
    previous depth's nodes (so parent < child)."""
    parents = [-1]
    start_prev, n_prev = 0, 1
    for width in widths[1:]:
        picks = torch.randint(0, n_prev, (width,), generator=g).tolist()
        parents += [start_prev + p for p in picks]
        start_prev, n_prev = len(parents) - width, width
    return parents


def medusa_parents(topk, T: int, g: torch.Generator) -> list[int]:
    """A random prefix-closed, rank-ordered T-node subtree (root included) of
    the full template in which a depth-d node has topk[d] ranked children;
    re-drawn until it reaches the template's full depth.  Nodes are numbered
    depth by depth, children in rank order."""
    depth_max = len(topk)
    while True:
        # node = (depth, parent_node, rank); the root is (0, -1, 0)
        nodes = [(0, -1, 0)]
        children = {0: []}
        while len(nodes) < T:
            frontier = []
            for i, (d, _, _) in enumerate(nodes):
                if d < depth_max and len(children[i]) < topk[d]:
                    frontier.append(i)   # next child of i has rank len(children[i])
            pick = frontier[int(torch.randint(0, len(frontier), (1,), generator=g))]
            d = nodes[pick][0] + 1
            nodes.append((d, pick, len(children[pick])))
            children[len(nodes) - 1] = []
            children[pick].append(len(nodes) - 1)
        if max(n[0] for n in nodes) == depth_max:
            break
    # Renumber depth by depth, children in (new parent id, rank) order.
    order = [0]
    new_id = {0: 0}
    for d in range(1, depth_max + 1):
        level = [i for i, n in enumerate(nodes) if n[0] == d]
        level.sort(key=lambda i: (new_id[nodes[i][1]], nodes[i][2]))
        for i in level:
            new_id[i] = len(order)
            order.append(i)
    return [-1] + [new_id[nodes[i][1]] for i in order[1:]]


def make_tree_inputs(w: Workload, device="cpu"):
    """Parents, node tokens and target logits [B, T, V] for greedy tree acceptance.

    eagle2: a fresh tree per sequence; medusa: one tree shared by the batch.
    For every node with children, with probability plant_prob its lowest-id
    child carries a random token t and the node's logit row gets the value
    PLANT_SIGMAS·σ at t (making t that row's maximum); its other children get
    random tokens different from t.  Without a plant all children are random.
    """
    B, T, V = w.B, w.T, w.V
    gt = _gen(w, "tree", "cpu")
    if w.tree == "eagle2":
        assert sum(w.tree_widths) == T
        par = [eagle2_parents(w.tree_widths, gt) for _ in range(B)]
    elif w.tree == "medusa":
        one = medusa_parents(w.tree_widths, T, gt)
        par = [one for _ in range(B)]
    else:
        par = [[-1] + list(range(T - 1)) for _ in range(B)]   # chain
    parents = torch.tensor(par, dtype=torch.int32)

    logits = _normal((B, T, V), _gen(w, "target", device), device, torch.float32,
                     sd=w.target_sd)
    gk = _gen(w, "tree_tokens", "cpu")
    tokens = torch.randint(0, V, (B, T), generator=gk, dtype=torch.int64)
    plant_u = torch.rand((B, T), generator=gk, dtype=torch.float64)
    spike = PLANT_SIGMAS * w.target_sd
    for b in range(B):
        kids: dict[int, list[int]] = {}
        for i in range(1, T):
            kids.setdefault(par[b][i], []).append(i)
        for node, ch in kids.items():
            first = ch[0]
            planted = bool(plant_u[b, node] < w.plant_prob)
            t = int(tokens[b, first])
            if planted:
                logits[b, node, t] = spike
            for c in ch[1:]:
                # siblings get other tokens (with one token there is no other)
                while V > 1 and int(tokens[b, c]) == t:
                    tokens[b, c] = int(torch.randint(0, V, (1,), generator=gk))
    return dict(target_logits=logits, tokens=tokens.to(torch.int32).to(device),
                parents=parents.to(device))


def make_sampled_tree_inputs(w: Workload, device="cpu", draft_noise_sd: float = 1.0):
    """Inputs for sampled (non-greedy) tree acceptance.

    parents: as make_tree_inputs (eagle2 / medusa shapes); target logits
    [B, T, V] ~ N(0, target_sd²); draft logits = target + N(0, draft_noise_sd²)
    (row n is the draft's distribution for node n's children); each node's
    token is drawn from its parent's draft row by Gumbel-max (independently,
    so siblings may repeat a token); u_accept and u_draw [B, T] uniforms.
    """
    B, T, V = w.B, w.T, w.V
    parents = make_tree_inputs(w.with_(V=8), "cpu")["parents"]
    target = _normal((B, T, V), _gen(w, "target", device), device, torch.float32,
                     sd=w.target_sd)
    noise = _normal((B, T, V), _gen(w, "draft_noise", device), device, torch.float32,
                    sd=draft_noise_sd)
    draft = target + noise
    del noise
    par = parents.to(device).long()
    g = _gen(w, "stree_gumbel", device)
    tokens = torch.zeros((B, T), dtype=torch.int64, device=device)
    for b in range(B):
        # one Gumbel row per node, added to its parent's draft row
        gu = uniforms((T, V), g, device).double()
        rows = draft[b, par[b].clamp(min=0)].double() / w.temperature
        tokens[b] = torch.argmax(rows - torch.log(-torch.log(gu)), dim=-1)
    tokens[:, 0] = 0
    return dict(target_logits=target, draft_logits=draft.contiguous(),
                tokens=tokens.to(torch.int32), parents=par.to(torch.int32),
                u_accept=uniforms((B, T), _gen(w, "u_accept", device), device),
                u_draw=uniforms((B, T), _gen(w, "u_draw", device), device))


def make_ngram_inputs(w: Workload, device="cpu", copy_prob: float = 0.5,
                      span=(16, 256)):
    """Token histories [B, ctx] int32 for n-gram drafting, and lengths [B].

    A history is built span by span (span lengths uniform in ``span``): the
    first span is fresh, each later one is, with probability copy_prob, a
    copy of an earlier stretch of the same history, else fresh tokens
    uniform over the vocabulary — a repetitive load with prompt-lookup hits.
    Lengths are uniform in [ctx/2, ctx], sequence 0 at ctx.
    """
    g = torch.Generator().manual_seed(w.seed * 1000 + _STREAMS["ngram"])
    B, L, V = w.B, w.ctx, w.V
    ctx = torch.empty((B, L), dtype=torch.int64)
    for b in range(B):
        pos = 0
        while pos < L:
            n = min(L - pos, int(torch.randint(span[0], span[1] + 1, (1,), generator=g)))
            if pos >= span[0] and float(torch.rand((1,), generator=g)) < copy_prob:
                src = int(torch.randint(0, pos - min(n, pos) + 1, (1,), generator=g))
                n = min(n, pos - src)
                ctx[b, pos:pos + n] = ctx[b, src:src + n]
            else:
                ctx[b, pos:pos + n] = torch.randint(0, V, (n,), generator=g)
            pos += n
    lens = torch.randint(max(1, L // 2), L + 1, (B,), generator=g)
    lens[0] = L
    return ctx.to(torch.int32).to(device), lens.to(torch.int32).to(device)


def ragged_ctx_lens(w: Workload, device="cpu") -> torch.Tensor:
    """Per-sequence prefix lengths [B] int32 for a paged cache: uniform in
    [0, ctx], with sequence 0 at ctx (the longest) and, for B >= 3, the last
    sequence at 0 (no prefix)."""
    g = _gen(w, "ctx_lens", "cpu")
    lens = torch.randint(0, w.ctx + 1, (w.B,), generator=g, dtype=torch.int64)
    lens[0] = w.ctx
    if w.B >= 3:
        lens[-1] = 0
    return lens.to(torch.int32).to(device)


def make_paged_kv(w: Workload, k: torch.Tensor, v: torch.Tensor, page_size: int,
                  layout: str = "hnd", ctx_lens=None, spare_pages: int = 3):
    """Scatter contiguous K/V [B, Hkv, ctx+T, D] into a shuffled page pool.

    Sequence b keeps its first ctx_lens[b] + T rows (all ctx + T rows when
    ctx_lens is None).  Its j-th block of page_size rows goes to the page that
    a seeded permutation of the pool assigns it; block_table[b][j] names that
    page.  The pool holds spare_pages pages more than the sequences use.
    Everything no sequence owns is NaN: rows past a sequence's length in its
    last page, the spare pages, and the page that the unused block-table
    entries (past each sequence's last block) point at.

    Returns (k_pages, v_pages, block_table [B, max_blocks] int32) on k's
    device; pages are [P, Hkv, page_size, D] ("hnd") or [P, page_size, Hkv,
    D] ("nhd").
    """
    B, Hkv, L, D = k.shape
    T = w.T
    lens = [L - T] * B if ctx_lens is None else [int(x) for x in ctx_lens]
    nblk = [(c + T + page_size - 1) // page_size for c in lens]
    max_blocks = (L + page_size - 1) // page_size
    used = sum(nblk)
    pool = used + max(1, spare_pages)
    perm = torch.randperm(pool, generator=_gen(w, "pages", "cpu"))
    poison = int(perm[used])                      # a spare page: stale entries point here
    table = torch.full((B, max_blocks), poison, dtype=torch.int32)
    shape = (pool, Hkv, page_size, D) if layout == "hnd" else (pool, page_size, Hkv, D)
    if layout not in ("hnd", "nhd"):
        raise ValueError(f"unknown page layout {layout!r}")
    pages = []
    for src in (k, v):
        dst = torch.full(shape, float("nan"), dtype=src.dtype, device=src.device)
        at = 0
        for b in range(B):
            n, rows = nblk[b], lens[b] + T
            ids = perm[at: at + n]
            at += n
            table[b, :n] = ids.to(torch.int32)
            blk = torch.full((Hkv, n * page_size, D), float("nan"), dtype=src.dtype,
                             device=src.device)
            blk[:, :rows] = src[b, :, :rows]
            blk = blk.view(Hkv, n, page_size, D).permute(1, 0, 2, 3)   # [n, Hkv, ps, D]
            if layout == "nhd":
                blk = blk.permute(0, 2, 1, 3)                          # [n, ps, Hkv, D]
            dst[ids.to(src.device)] = blk
        pages.append(dst)
    return pages[0], pages[1], table.to(k.device)


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)
