"""ctypes binding of libspecverify.so (the C ABI in include/spec_verify.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their device pointers and the current HIP stream are passed to the
library, and a non-OK status raises.  Every step of the computation runs in
the library's HIP kernels; there is no fallback.  Workspaces (and outputs the
caller does not pass) are allocated with torch on the current stream; when
the call runs on another stream (``stream=``), that stream is recorded on
them, so the caching allocator does not reuse their memory before the
kernels are done.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspecverify.so")

SPEC_OK, SPEC_ERR_NULL, SPEC_ERR_SHAPE, SPEC_ERR_UNSUPPORTED, SPEC_ERR_WORKSPACE, SPEC_ERR_HIP = range(6)
SPEC_F32, SPEC_BF16 = 0, 1
SPEC_PAGES_HND, SPEC_PAGES_NHD = 0, 1
_LAYOUTS = {"hnd": SPEC_PAGES_HND, "nhd": SPEC_PAGES_NHD}

#: Every function the header declares, with its ctypes signature.
_c = ctypes
_SIGNATURES = {
    "spec_status_string": (_c.c_char_p, [_c.c_int]),
    "spec_verify_attention_workspace": (_c.c_size_t, [_c.c_int] * 6 + [_c.c_int]),
    "spec_verify_attention": (_c.c_int, [_c.c_void_p] * 5 + [_c.c_int] * 6 + [_c.c_int, _c.c_float,
                                        _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "spec_verify_attention_paged_workspace": (_c.c_size_t, [_c.c_int] * 6 + [_c.c_int]),
    "spec_verify_attention_paged": (_c.c_int, [_c.c_void_p] * 7 + [_c.c_int] * 9
                                    + [_c.c_int, _c.c_int, _c.c_float,
                                       _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "spec_accept_chain_workspace": (_c.c_size_t, [_c.c_int] * 3),
    "spec_accept_chain": (_c.c_int, [_c.c_void_p] * 5 + [_c.c_float] + [_c.c_void_p] * 2
                          + [_c.c_int] * 3 + [_c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "spec_accept_chain_noalloc": (_c.c_int, [_c.c_void_p] * 5 + [_c.c_float] + [_c.c_void_p] * 2
                                  + [_c.c_int] * 3 + [_c.c_void_p]),
    "spec_accept_tree_workspace": (_c.c_size_t, [_c.c_int] * 3),
    "spec_accept_tree": (_c.c_int, [_c.c_void_p] * 6 + [_c.c_int] * 3
                         + [_c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "spec_accept_tree_sampled_workspace": (_c.c_size_t, [_c.c_int] * 3),
    "spec_accept_tree_sampled": (_c.c_int, [_c.c_void_p] * 6 + [_c.c_float] + [_c.c_void_p] * 3
                                 + [_c.c_int] * 3 + [_c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "spec_ngram_propose_workspace": (_c.c_size_t, [_c.c_int] * 2),
    "spec_ngram_propose": (_c.c_int, [_c.c_void_p] * 4 + [_c.c_int] * 5
                           + [_c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "spec_commit_kv": (_c.c_int, [_c.c_void_p] * 5 + [_c.c_int] * 5 + [_c.c_int, _c.c_void_p]),
}

_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({status_string(status)})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(there is no fallback path)")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def exported_symbols() -> list[str]:
    return list(_SIGNATURES)


def status_string(status: int) -> str:
    return load().spec_status_string(status).decode()


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _keep_for_stream(stream, *tensors):
    """Tensors the binding allocated (workspaces, outputs) come from torch's
    caching allocator on the current stream.  When the kernels run on another
    stream, that stream is recorded on each tensor, so that its memory is not
    handed to another tensor before the kernels that use it have finished."""
    if stream is None:
        return
    s = torch.cuda.ExternalStream(stream) if isinstance(stream, int) else stream
    if s.cuda_stream == torch.cuda.current_stream().cuda_stream:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(s)


def _check(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _raise(status, what):
    if status != SPEC_OK:
        raise SpecVerifyError(status, what)


def _workspace(nbytes, device, workspace):
    if workspace is not None:
        return workspace
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------- attention
def spec_verify_attention_workspace(B, T, Hq, Hkv, D, ctx, dtype=SPEC_BF16) -> int:
    return int(load().spec_verify_attention_workspace(B, T, Hq, Hkv, D, ctx, dtype))


def spec_verify_attention(q, k, v, ctx, parents=None, out=None, scale=None,
                          workspace=None, stream=None):
    """out [B,T,Hq,D] fp32 = masked verify attention of q against k/v (see the header)."""
    B, T, Hq, D = q.shape
    Hkv = k.shape[1]
    dev = q.device
    dt = {torch.float32: SPEC_F32, torch.bfloat16: SPEC_BF16}[q.dtype]
    _check(k, "k", (B, Hkv, ctx + T, D), q.dtype, dev)
    _check(v, "v", (B, Hkv, ctx + T, D), q.dtype, dev)
    _check(q, "q", (B, T, Hq, D), q.dtype, dev)
    if parents is not None:
        _check(parents, "parents", (B, T), torch.int32, dev)
    made_out = out is None
    if out is None:
        out = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
    _check(out, "out", (B, T, Hq, D), torch.float32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = spec_verify_attention_workspace(B, T, Hq, Hkv, D, ctx, dt)
    ws = _workspace(need, dev, workspace)
    st = load().spec_verify_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(parents), _ptr(out),
                                      B, T, Hq, Hkv, D, ctx, dt, float(scale),
                                      _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _raise(st, "spec_verify_attention")
    _keep_for_stream(stream, ws if workspace is None else None, out if made_out else None)
    return out


def spec_verify_attention_paged_workspace(B, T, Hq, Hkv, D, max_ctx, dtype=SPEC_BF16) -> int:
    return int(load().spec_verify_attention_paged_workspace(B, T, Hq, Hkv, D, max_ctx, dtype))


def spec_verify_attention_paged(q, k_pages, v_pages, block_table, max_ctx, ctx_lens=None,
                                parents=None, layout="hnd", out=None, scale=None,
                                workspace=None, stream=None):
    """out [B,T,Hq,D] fp32 = verify attention over a paged KV cache (see the header).

    k_pages, v_pages: [P, Hkv, page_size, D] ("hnd") or [P, page_size, Hkv, D]
    ("nhd"); block_table [B, max_blocks] int32; ctx_lens [B] int32 or None.
    """
    B, T, Hq, D = q.shape
    dev = q.device
    dt = {torch.float32: SPEC_F32, torch.bfloat16: SPEC_BF16}[q.dtype]
    if layout not in _LAYOUTS:
        raise ValueError(f"layout must be 'hnd' or 'nhd', not {layout!r}")
    if k_pages.dim() != 4:
        raise ValueError("k_pages must be 4-D")
    P = k_pages.shape[0]
    if layout == "hnd":
        Hkv, ps = k_pages.shape[1], k_pages.shape[2]
        pshape = (P, Hkv, ps, D)
    else:
        ps, Hkv = k_pages.shape[1], k_pages.shape[2]
        pshape = (P, ps, Hkv, D)
    _check(q, "q", (B, T, Hq, D), q.dtype, dev)
    _check(k_pages, "k_pages", pshape, q.dtype, dev)
    _check(v_pages, "v_pages", pshape, q.dtype, dev)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [B, max_blocks]")
    _check(block_table, "block_table", (B, block_table.shape[1]), torch.int32, dev)
    if ctx_lens is not None:
        _check(ctx_lens, "ctx_lens", (B,), torch.int32, dev)
    if parents is not None:
        _check(parents, "parents", (B, T), torch.int32, dev)
    made_out = out is None
    if out is None:
        out = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
    _check(out, "out", (B, T, Hq, D), torch.float32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = spec_verify_attention_paged_workspace(B, T, Hq, Hkv, D, max_ctx, dt)
    ws = _workspace(need, dev, workspace)
    st = load().spec_verify_attention_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(ctx_lens), _ptr(parents),
        _ptr(out), B, T, Hq, Hkv, D, max_ctx, ps, P, block_table.shape[1], _LAYOUTS[layout], dt,
        float(scale), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _raise(st, "spec_verify_attention_paged")
    _keep_for_stream(stream, ws if workspace is None else None, out if made_out else None)
    return out


# --------------------------------------------------------------------------- chain
def spec_accept_chain_workspace(B, N, V) -> int:
    return int(load().spec_accept_chain_workspace(B, N, V))


def spec_accept_chain(target_logits, draft_logits, draft_tokens, u_accept, u_draw,
                      temperature=1.0, num_accepted=None, out_tokens=None,
                      workspace=None, stream=None):
    """Rejection-sampling acceptance of N drafts; returns (num_accepted [B], out_tokens [B,N+1])."""
    B, N1, V = target_logits.shape
    N = N1 - 1
    dev = target_logits.device
    _check(target_logits, "target_logits", (B, N + 1, V), torch.float32, dev)
    _check(draft_logits, "draft_logits", (B, N, V), torch.float32, dev)
    _check(draft_tokens, "draft_tokens", (B, N), torch.int32, dev)
    _check(u_accept, "u_accept", (B, N), torch.float32, dev)
    _check(u_draw, "u_draw", (B, N + 1), torch.float32, dev)
    made = [num_accepted is None, out_tokens is None]
    if num_accepted is None:
        num_accepted = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, N + 1), dtype=torch.int32, device=dev)
    _check(num_accepted, "num_accepted", (B,), torch.int32, dev)
    _check(out_tokens, "out_tokens", (B, N + 1), torch.int32, dev)
    ws = _workspace(spec_accept_chain_workspace(B, N, V), dev, workspace)
    st = load().spec_accept_chain(_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens),
                                  _ptr(u_accept), _ptr(u_draw), float(temperature),
                                  _ptr(num_accepted), _ptr(out_tokens), B, N, V,
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _raise(st, "spec_accept_chain")
    _keep_for_stream(stream, ws if workspace is None else None,
                     num_accepted if made[0] else None, out_tokens if made[1] else None)
    return num_accepted, out_tokens


#: Scratch of spec_accept_chain_noalloc per GPU (SPEC_CHAIN_NOALLOC_SCRATCH_BYTES).
CHAIN_NOALLOC_SCRATCH_BYTES = 4 << 20


def spec_accept_chain_noalloc(target_logits, draft_logits, draft_tokens, u_accept, u_draw,
                              num_accepted, out_tokens, temperature=1.0, stream=None):
    """spec_accept_chain with the library's static scratch instead of a
    workspace: the caller passes the outputs and nothing is allocated."""
    B, N1, V = target_logits.shape
    N = N1 - 1
    dev = target_logits.device
    _check(target_logits, "target_logits", (B, N + 1, V), torch.float32, dev)
    _check(draft_logits, "draft_logits", (B, N, V), torch.float32, dev)
    _check(draft_tokens, "draft_tokens", (B, N), torch.int32, dev)
    _check(u_accept, "u_accept", (B, N), torch.float32, dev)
    _check(u_draw, "u_draw", (B, N + 1), torch.float32, dev)
    _check(num_accepted, "num_accepted", (B,), torch.int32, dev)
    _check(out_tokens, "out_tokens", (B, N + 1), torch.int32, dev)
    st = load().spec_accept_chain_noalloc(_ptr(target_logits), _ptr(draft_logits),
                                          _ptr(draft_tokens), _ptr(u_accept), _ptr(u_draw),
                                          float(temperature), _ptr(num_accepted),
                                          _ptr(out_tokens), B, N, V, _stream(stream))
    _raise(st, "spec_accept_chain_noalloc")
    return num_accepted, out_tokens


# --------------------------------------------------------------------------- tree
def spec_accept_tree_workspace(B, T, V) -> int:
    return int(load().spec_accept_tree_workspace(B, T, V))


def spec_accept_tree(target_logits, tokens, parents, accept_len=None, path=None,
                     out_tokens=None, workspace=None, stream=None):
    """Greedy tree acceptance; returns (accept_len [B], path [B,T], out_tokens [B,T])."""
    B, T, V = target_logits.shape
    dev = target_logits.device
    _check(target_logits, "target_logits", (B, T, V), torch.float32, dev)
    _check(tokens, "tokens", (B, T), torch.int32, dev)
    _check(parents, "parents", (B, T), torch.int32, dev)
    made = [accept_len is None, path is None, out_tokens is None]
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if path is None:
        path = torch.empty((B, T), dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, T), dtype=torch.int32, device=dev)
    ws = _workspace(spec_accept_tree_workspace(B, T, V), dev, workspace)
    st = load().spec_accept_tree(_ptr(target_logits), _ptr(tokens), _ptr(parents),
                                 _ptr(accept_len), _ptr(path), _ptr(out_tokens), B, T, V,
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _raise(st, "spec_accept_tree")
    _keep_for_stream(stream, ws if workspace is None else None,
                     *(t for t, m in zip((accept_len, path, out_tokens), made) if m))
    return accept_len, path, out_tokens


def spec_accept_tree_sampled_workspace(B, T, V) -> int:
    return int(load().spec_accept_tree_sampled_workspace(B, T, V))


def spec_accept_tree_sampled(target_logits, draft_logits, tokens, parents, u_accept, u_draw,
                             temperature=1.0, accept_len=None, path=None, out_tokens=None,
                             workspace=None, stream=None):
    """Sampled tree acceptance; returns (accept_len [B], path [B,T], out_tokens [B,T])."""
    B, T, V = target_logits.shape
    dev = target_logits.device
    _check(target_logits, "target_logits", (B, T, V), torch.float32, dev)
    _check(draft_logits, "draft_logits", (B, T, V), torch.float32, dev)
    _check(tokens, "tokens", (B, T), torch.int32, dev)
    _check(parents, "parents", (B, T), torch.int32, dev)
    _check(u_accept, "u_accept", (B, T), torch.float32, dev)
    _check(u_draw, "u_draw", (B, T), torch.float32, dev)
    made = [accept_len is None, path is None, out_tokens is None]
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if path is None:
        path = torch.empty((B, T), dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, T), dtype=torch.int32, device=dev)
    ws = _workspace(spec_accept_tree_sampled_workspace(B, T, V), dev, workspace)
    st = load().spec_accept_tree_sampled(
        _ptr(target_logits), _ptr(draft_logits), _ptr(tokens), _ptr(parents), _ptr(u_accept),
        _ptr(u_draw), float(temperature), _ptr(accept_len), _ptr(path), _ptr(out_tokens),
        B, T, V, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _raise(st, "spec_accept_tree_sampled")
    _keep_for_stream(stream, ws if workspace is None else None,
                     *(t for t, m in zip((accept_len, path, out_tokens), made) if m))
    return accept_len, path, out_tokens


def spec_ngram_propose_workspace(B, L) -> int:
    return int(load().spec_ngram_propose_workspace(B, L))


def spec_ngram_propose(context, N, n_min=1, n_max=4, context_lens=None, num_drafts=None,
                       drafts=None, workspace=None, stream=None):
    """n-gram draft proposal; returns (num_drafts [B], drafts [B, N]) int32."""
    B, L = context.shape
    dev = context.device
    _check(context, "context", (B, L), torch.int32, dev)
    if context_lens is not None:
        _check(context_lens, "context_lens", (B,), torch.int32, dev)
    made = [num_drafts is None, drafts is None]
    if num_drafts is None:
        num_drafts = torch.empty(B, dtype=torch.int32, device=dev)
    if drafts is None:
        drafts = torch.empty((B, N), dtype=torch.int32, device=dev)
    _check(drafts, "drafts", (B, N), torch.int32, dev)
    ws = _workspace(spec_ngram_propose_workspace(B, L), dev, workspace)
    st = load().spec_ngram_propose(_ptr(context), _ptr(context_lens), _ptr(num_drafts),
                                   _ptr(drafts), B, L, N, n_min, n_max, _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream))
    _raise(st, "spec_ngram_propose")
    _keep_for_stream(stream, ws if workspace is None else None,
                     num_drafts if made[0] else None, drafts if made[1] else None)
    return num_drafts, drafts


def spec_commit_kv(k, v, ctx, accept_len, path=None, new_len=None, stream=None):
    """Commit the accepted path's K/V in place; returns new_len [B] (int32)."""
    B, Hkv, L, D = k.shape
    T = L - ctx
    dev = k.device
    dt = {torch.float32: SPEC_F32, torch.bfloat16: SPEC_BF16}[k.dtype]
    _check(k, "k", (B, Hkv, L, D), k.dtype, dev)
    _check(v, "v", (B, Hkv, L, D), k.dtype, dev)
    _check(accept_len, "accept_len", (B,), torch.int32, dev)
    if path is not None:
        _check(path, "path", (B, T), torch.int32, dev)
    made = new_len is None
    if new_len is None:
        new_len = torch.empty(B, dtype=torch.int32, device=dev)
    st = load().spec_commit_kv(_ptr(k), _ptr(v), _ptr(path), _ptr(accept_len), _ptr(new_len),
                               B, T, Hkv, D, ctx, dt, _stream(stream))
    _raise(st, "spec_commit_kv")
    _keep_for_stream(stream, new_len if made else None)
    return new_len
