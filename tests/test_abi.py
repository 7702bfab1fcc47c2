"""The C-ABI library on the host: it loads, exports every function
include/spec_verify.h declares, and rejects bad arguments before launching
anything (no GPU needed: every call here fails validation or is empty)."""
import os
import re
import subprocess

import pytest

from verify_pass_rejection_amd import native as nat

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")
FAKE = 0x1000          # a non-NULL pointer that must never be dereferenced
OK, NULL, SHAPE, UNSUP, WS, HIP = range(6)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = nat.load()
    decl = declared_functions()
    assert len(decl) == 15
    for name in decl:
        assert hasattr(lib, name), name
    assert sorted(nat.exported_symbols()) == decl
    dyn = subprocess.run(["nm", "-D", "--defined-only", nat.library_path()],
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (spec_[a-z_]+)$", dyn, flags=re.M))
    assert exported == set(decl)


def test_status_strings():
    for s in range(6):
        assert nat.status_string(s)
    assert nat.status_string(99) == "unknown status"


def attn(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, parents=None, out=FAKE, B=2, T=5, Hq=8, Hkv=2, D=128,
             ctx=100, dtype=1, scale=0.1, ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return nat.load().spec_verify_attention(a["q"], a["k"], a["v"], a["parents"], a["out"],
                                            a["B"], a["T"], a["Hq"], a["Hkv"], a["D"], a["ctx"],
                                            a["dtype"], a["scale"], a["ws"], a["ws_bytes"],
                                            a["stream"])


def test_attention_validation():
    assert attn(q=None) == NULL
    assert attn(out=None) == NULL
    assert attn(ws=None) == NULL
    assert attn(Hq=7) == SHAPE
    assert attn(B=-1) == SHAPE
    assert attn(ctx=-3) == SHAPE
    assert attn(T=65) == UNSUP
    assert attn(D=96) == UNSUP
    assert attn(dtype=7) == UNSUP
    assert attn(scale=float("nan")) == SHAPE
    assert attn(scale=0.0) == SHAPE
    assert attn(scale=-0.5) == SHAPE
    assert attn(ws_bytes=16) == WS
    assert attn(q=FAKE + 4) == UNSUP         # 16-byte loads and stores need alignment
    assert attn(out=FAKE + 8) == UNSUP
    assert attn(B=1 << 30, Hkv=2) == UNSUP   # B*Hkv past int32 block ids
    assert attn(B=(1 << 30) - 1, Hkv=2, q=None) == NULL
    assert attn(ctx=(1 << 24) - 5, T=5) == UNSUP   # (ctx+T)*D = 2^31: K/V element index
    assert attn(ctx=(1 << 24) - 6, T=5, q=None) == NULL
    assert attn(ctx=(1 << 31) - 2, T=5) == UNSUP    # ctx + T past int32, no overflow
    assert attn(B=0, q=None) == OK          # empty problem: nothing launched
    assert attn(T=0, q=None) == OK


def test_attention_workspace_sizes():
    f = nat.spec_verify_attention_workspace
    big = f(64, 9, 32, 8, 128, 32768, nat.SPEC_BF16)
    assert big > 0 and big % 256 == 0
    assert f(1, 5, 8, 8, 64, 256, nat.SPEC_F32) > 0
    assert f(1, 5, 8, 3, 64, 256, nat.SPEC_F32) == 0    # invalid shape
    assert f(0, 5, 8, 8, 64, 256, nat.SPEC_F32) == 0
    # the workspace holds at least one partial (D floats + max and sum) per row and split
    assert f(2, 6, 32, 8, 128, 4096, nat.SPEC_BF16) >= 2 * 8 * 24 * 130 * 4


def paged(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, parents=None, out=FAKE, B=2, T=5, Hq=8,
             Hkv=2, D=128, max_ctx=100, ps=16, P=20, mb=7, layout=0, dtype=1, scale=0.1,
             ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return nat.load().spec_verify_attention_paged(
        a["q"], a["k"], a["v"], a["bt"], a["lens"], a["parents"], a["out"], a["B"], a["T"],
        a["Hq"], a["Hkv"], a["D"], a["max_ctx"], a["ps"], a["P"], a["mb"], a["layout"],
        a["dtype"], a["scale"], a["ws"], a["ws_bytes"], a["stream"])


def test_paged_attention_validation():
    assert paged(q=None) == NULL
    assert paged(k=None) == NULL
    assert paged(bt=None) == NULL
    assert paged(ws=None) == NULL
    assert paged(Hq=7) == SHAPE
    assert paged(max_ctx=-1) == SHAPE
    assert paged(ps=0) == SHAPE
    assert paged(P=0) == SHAPE
    assert paged(mb=6) == SHAPE               # 6 * 16 < 100 + 5: the table is too short
    assert paged(ps=24) == UNSUP              # page sizes are powers of two
    assert paged(ps=1 << 21) == UNSUP
    assert paged(layout=2) == UNSUP
    assert paged(T=65) == UNSUP
    assert paged(D=96) == UNSUP
    assert paged(scale=0.0) == SHAPE
    assert paged(ws_bytes=16) == WS
    assert paged(k=FAKE + 2) == UNSUP         # 16-byte loads need alignment
    assert paged(B=0, q=None) == OK
    assert paged(T=0, q=None) == OK
    f = nat.spec_verify_attention_paged_workspace
    assert f(64, 9, 32, 8, 128, 32768, nat.SPEC_BF16) == \
        nat.spec_verify_attention_workspace(64, 9, 32, 8, 128, 32768, nat.SPEC_BF16)


def chain(**kw):
    a = dict(t=FAKE, d=FAKE, x=FAKE, ua=FAKE, ud=FAKE, tau=1.0, na=FAKE, out=FAKE,
             B=4, N=3, V=1000, ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return nat.load().spec_accept_chain(a["t"], a["d"], a["x"], a["ua"], a["ud"], a["tau"],
                                        a["na"], a["out"], a["B"], a["N"], a["V"], a["ws"],
                                        a["ws_bytes"], a["stream"])


def test_chain_validation():
    assert chain(t=None) == NULL
    assert chain(d=None) == NULL
    assert chain(ud=None) == NULL
    assert chain(na=None) == NULL
    assert chain(tau=0.0) == SHAPE
    assert chain(tau=-1.0) == SHAPE
    assert chain(tau=float("inf")) == SHAPE
    assert chain(V=0) == SHAPE
    assert chain(N=-1) == SHAPE
    assert chain(N=64) == UNSUP
    assert chain(V=(1 << 24) + 1) == UNSUP
    assert chain(ws_bytes=8) == WS
    assert chain(B=1 << 29, N=3) == UNSUP    # B*(2N+1) past int32 block ids
    assert chain(B=(2**31 - 1) // 7, N=3, t=None) == NULL
    assert chain(B=0, t=None) == OK
    # N = 0 needs no draft rows, tokens or accept uniforms
    assert chain(N=0, d=None, x=None, ua=None, ws_bytes=8) == WS


def chain_noalloc(**kw):
    a = dict(t=FAKE, d=FAKE, x=FAKE, ua=FAKE, ud=FAKE, tau=1.0, na=FAKE, out=FAKE,
             B=4, N=3, V=1000, stream=None)
    a.update(kw)
    return nat.load().spec_accept_chain_noalloc(a["t"], a["d"], a["x"], a["ua"], a["ud"],
                                                a["tau"], a["na"], a["out"], a["B"], a["N"],
                                                a["V"], a["stream"])


def test_chain_noalloc_validation():
    """The same checks as spec_accept_chain, and problems whose workspace
    would exceed the static scratch are refused before any HIP call."""
    assert chain_noalloc(t=None) == NULL
    assert chain_noalloc(d=None) == NULL
    assert chain_noalloc(ud=None) == NULL
    assert chain_noalloc(out=None) == NULL
    assert chain_noalloc(tau=0.0) == SHAPE
    assert chain_noalloc(V=0) == SHAPE
    assert chain_noalloc(N=64) == UNSUP
    assert chain_noalloc(B=1 << 29, N=3) == UNSUP
    assert chain_noalloc(B=0, t=None) == OK
    limit = nat.CHAIN_NOALLOC_SCRATCH_BYTES
    assert nat.spec_accept_chain_workspace(64, 8, 152064) <= limit       # the large batch fits
    assert nat.spec_accept_chain_workspace(1024, 8, 152064) <= limit
    assert nat.spec_accept_chain_workspace(4096, 8, 152064) > limit
    assert chain_noalloc(B=4096, N=8, V=152064) == WS
    assert chain_noalloc(B=64, N=63, V=1 << 24) == WS
    header = open(HEADER).read()
    assert f"#define SPEC_CHAIN_NOALLOC_SCRATCH_BYTES ((size_t){limit >> 20} << 20)" in header


def test_chain_workspace_sizes():
    f = nat.spec_accept_chain_workspace
    assert f(64, 8, 152064) >= 64 * 17 * 8
    assert f(0, 8, 100) == 0 and f(1, -1, 100) == 0


def tree(**kw):
    a = dict(z=FAKE, tok=FAKE, par=FAKE, al=FAKE, path=FAKE, out=FAKE, B=2, T=10, V=500,
             ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return nat.load().spec_accept_tree(a["z"], a["tok"], a["par"], a["al"], a["path"], a["out"],
                                       a["B"], a["T"], a["V"], a["ws"], a["ws_bytes"], a["stream"])


def test_tree_validation():
    assert tree(par=None) == NULL
    assert tree(path=None) == NULL
    assert tree(T=65) == UNSUP
    assert tree(V=0) == SHAPE
    assert tree(ws_bytes=4) == WS
    assert tree(B=1 << 27, T=16) == UNSUP    # B*T past int32 block ids
    assert tree(B=(1 << 27) - 1, T=16, par=None) == NULL
    assert tree(B=0, z=None) == OK
    assert nat.spec_accept_tree_workspace(8, 64, 32000) > 0


def test_python_binding_checks_tensors_before_calling():
    import torch
    q = torch.zeros(1, 2, 4, 64)
    with pytest.raises(ValueError):
        nat.spec_verify_attention(q, torch.zeros(1, 2, 9, 64), torch.zeros(1, 2, 10, 64), ctx=8)
    with pytest.raises(TypeError):
        nat.spec_accept_chain(torch.zeros(1, 2, 5), torch.zeros(1, 1, 5), torch.zeros(1, 1),
                              torch.zeros(1, 1), torch.zeros(1, 2))


def commit(**kw):
    a = dict(k=FAKE, v=FAKE, path=FAKE, acc=FAKE, new_len=FAKE, B=2, T=9, Hkv=8, D=128,
             ctx=100, dtype=1, stream=None)
    a.update(kw)
    return nat.load().spec_commit_kv(a["k"], a["v"], a["path"], a["acc"], a["new_len"], a["B"],
                                     a["T"], a["Hkv"], a["D"], a["ctx"], a["dtype"], a["stream"])


def stree(**kw):
    a = dict(t=FAKE, d=FAKE, x=FAKE, par=FAKE, ua=FAKE, ud=FAKE, tau=1.0, al=FAKE, path=FAKE,
             out=FAKE, B=4, T=8, V=1000, ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return nat.load().spec_accept_tree_sampled(a["t"], a["d"], a["x"], a["par"], a["ua"],
                                               a["ud"], a["tau"], a["al"], a["path"],
                                               a["out"], a["B"], a["T"], a["V"], a["ws"],
                                               a["ws_bytes"], a["stream"])


def test_sampled_tree_validation():
    assert stree(t=None) == NULL
    assert stree(d=None) == NULL
    assert stree(ua=None) == NULL
    assert stree(ud=None) == NULL
    assert stree(path=None) == NULL
    assert stree(tau=0.0) == SHAPE
    assert stree(tau=float("inf")) == SHAPE
    assert stree(B=-1) == SHAPE
    assert stree(V=0) == SHAPE
    assert stree(T=65) == UNSUP
    assert stree(V=(1 << 24) + 1) == UNSUP
    assert stree(ws=None) == NULL
    assert stree(ws_bytes=8) == WS
    assert stree(B=1 << 27, T=16) == UNSUP
    assert stree(B=(1 << 27) - 1, T=16, t=None) == NULL
    assert stree(B=0, t=None) == OK
    assert stree(T=0, t=None) == OK
    f = nat.spec_accept_tree_sampled_workspace
    assert f(8, 64, 32000) >= 2 * 8 * 64 * 4 * 12 and f(8, 64, 32000) % 256 == 0
    assert f(0, 64, 32000) == 0 and f(8, 65, 32000) == 0


def ngram(**kw):
    a = dict(c=FAKE, lens=None, num=FAKE, d=FAKE, B=4, L=1000, N=8, n_min=1, n_max=4, ws=FAKE,
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return nat.load().spec_ngram_propose(a["c"], a["lens"], a["num"], a["d"], a["B"], a["L"],
                                         a["N"], a["n_min"], a["n_max"], a["ws"],
                                         a["ws_bytes"], a["stream"])


def test_ngram_validation():
    assert ngram(c=None) == NULL
    assert ngram(num=None) == NULL
    assert ngram(d=None) == NULL
    assert ngram(ws=None) == NULL
    assert ngram(B=-1) == SHAPE
    assert ngram(L=-1) == SHAPE
    assert ngram(N=-1) == SHAPE
    assert ngram(n_min=0) == SHAPE
    assert ngram(n_min=3, n_max=2) == SHAPE
    assert ngram(N=64) == UNSUP
    assert ngram(n_max=17) == UNSUP
    assert ngram(ws_bytes=8) == WS
    assert ngram(B=0, c=None) == OK
    f = nat.spec_ngram_propose_workspace
    assert f(64, 32768) >= 64 * 8 * 8 and f(64, 32768) % 256 == 0
    assert f(0, 100) == 0


def test_commit_validation():
    assert commit(acc=None) == NULL
    assert commit(new_len=None) == NULL
    assert commit(k=None) == NULL              # a tree commit moves rows
    assert commit(T=0) == SHAPE
    assert commit(Hkv=0) == SHAPE
    assert commit(ctx=-1) == SHAPE
    assert commit(T=65) == UNSUP
    assert commit(D=32) == UNSUP
    assert commit(ctx=(1 << 31) - 2) == UNSUP      # ctx + T past int32, no overflow
    assert commit(dtype=3) == UNSUP
    assert commit(v=FAKE + 8) == UNSUP         # 16-byte vectors
    assert commit(B=1 << 29, Hkv=8) == UNSUP   # B*Hkv past int32 block ids
    assert commit(B=(1 << 28) - 1, Hkv=8, acc=None) == NULL
    assert commit(B=0, acc=None) == OK         # empty problem: nothing launched
