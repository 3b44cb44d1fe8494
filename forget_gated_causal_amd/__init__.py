"""Causal Forgetting-Transformer (FoX) attention on MI355X: Python binding of libfox.

Every function here only marshals torch tensors (device memory) and the current
HIP stream into the C ABI of include/fox.h; all arithmetic runs in the HIP
kernels of libfox.so.  Outputs are allocated with torch when not supplied.

    c            = logf_cumsum(logf)                          # [..., N] fp32
    o, lse, c    = attn_fwd(q, k, v, logf, scale=None)        # q,k,v [B,H,N,d]
    o, lse, c    = attn_fwd_noncausal(q, k, v, logf)          # every key, no mask
    o, lse, c    = attn_fwd_ex(q, k, v, logf, causal, layout)  # layout "head" [B,H,N,d] / "token" [B,N,H,d]
    dq, dk, dv, dlogf = attn_bwd(q, k, v, o, dout, lse, logf)  # gradients (bf16 or fp32); layout="token" too
    o, lse       = attn_decode(q, k_cache, v_cache, c_cache, logf_new, scale=None)
    o, lse       = attn_decode_noalloc(q, k_cache, v_cache, c_cache, logf_new)   # no workspace: library scratch
    o, lse       = attn_decode_ragged(q, k_cache, v_cache, c_cache, logf_new, cache_lens)
    o, lse       = attn_decode_paged(q, k_pages, v_pages, c_pages, block_table, cache_lens, logf_new)
"""

from __future__ import annotations

import torch

from ._lib import FOX_BF16, FOX_F32, FOX_HEAD_MAJOR, FOX_TOKEN_MAJOR, FoxError, check, lib, status_string  # noqa: F401

__all__ = ["logf_cumsum", "attn_fwd", "attn_fwd_noncausal", "attn_fwd_ex", "attn_fwd_pruned", "attn_fwd_pruned_workspace_bytes",
           "attn_bwd", "attn_bwd_workspace_bytes", "attn_decode", "attn_decode_noalloc", "attn_decode_ragged",
           "attn_decode_paged",
           "decode_workspace_bytes", "FoxError", "status_string"]

_DTYPES = {torch.float32: FOX_F32, torch.bfloat16: FOX_BF16}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype=None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _out(t, name: str, shape, dtype, device):
    """A caller-supplied output buffer: same device, dtype and shape as the result, contiguous."""
    _need(t, name, dtype)
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} shape {tuple(t.shape)} != {tuple(shape)}")
    return t


def _alloc_or_check(t, name, shape, dtype, device):
    if t is None:
        return torch.empty(shape, device=device, dtype=dtype)
    return _out(t, name, shape, dtype, device)


def _default_scale(d: int) -> float:
    return float(torch.tensor(d ** -0.5, dtype=torch.float32))


def logf_cumsum(logf: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Inclusive prefix sum of log forget gates along the last axis (fp32 in/out)."""
    _need(logf, "logf", torch.float32)
    n = logf.shape[-1]
    rows = logf.numel() // max(n, 1)
    c = torch.empty_like(logf) if out is None else _out(out, "out", logf.shape, torch.float32, logf.device)
    check("fox_logf_cumsum", lib().fox_logf_cumsum(_ptr(logf), _ptr(c), rows, n, _stream()))
    return c


def _fwd_outputs(q, k, v, logf, out, lse, c, want_lse, want_c):
    """Checks the forward inputs and returns (dtype code, o, lse, c), allocating missing outputs."""
    B, H, N, d = q.shape
    dt = _DTYPES.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype)
        if tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{name} shape {tuple(t.shape)} != {(B, H, N, d)}")
    _need(logf, "logf", torch.float32)
    if tuple(logf.shape) != (B, H, N):
        raise ValueError(f"logf shape {tuple(logf.shape)} != {(B, H, N)}")
    o = _alloc_or_check(out, "out", (B, H, N, d), q.dtype, q.device)
    lse = _alloc_or_check(lse, "lse", (B, H, N), torch.float32, q.device) if want_lse else None
    c = _alloc_or_check(c, "c", (B, H, N), torch.float32, q.device) if want_c else None
    return dt, o, lse, c


def attn_fwd(q, k, v, logf, scale: float | None = None, out=None, lse=None, c=None,
             want_lse: bool = True, want_c: bool = True):
    """Causal FoX attention forward. q, k, v: [B,H,N,d] (fp32 or bf16); logf: [B,H,N] fp32.

    Returns (o, lse, c); lse / c are None when not wanted.
    """
    B, H, N, d = q.shape
    dt, o, lse, c = _fwd_outputs(q, k, v, logf, out, lse, c, want_lse, want_c)
    scale = _default_scale(d) if scale is None else float(scale)
    st = lib().fox_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(logf), _ptr(o), _ptr(lse), _ptr(c), B, H, N, d, scale,
                            dt, _stream())
    check("fox_attn_fwd", st)
    return o, lse, c


def attn_fwd_noncausal(q, k, v, logf, scale: float | None = None, out=None, lse=None, c=None,
                       want_lse: bool = True, want_c: bool = True):
    """FoX attention forward over every key (no causal mask); arguments and results as attn_fwd."""
    B, H, N, d = q.shape
    dt, o, lse, c = _fwd_outputs(q, k, v, logf, out, lse, c, want_lse, want_c)
    scale = _default_scale(d) if scale is None else float(scale)
    st = lib().fox_attn_fwd_noncausal(_ptr(q), _ptr(k), _ptr(v), _ptr(logf), _ptr(o), _ptr(lse), _ptr(c), B, H, N, d,
                                      scale, dt, _stream())
    check("fox_attn_fwd_noncausal", st)
    return o, lse, c


def attn_fwd_ex(q, k, v, logf, causal: bool = True, layout: str = "head", scale: float | None = None, out=None,
                lse=None, c=None, want_lse: bool = True, want_c: bool = True):
    """fox_attn_fwd_ex: the forward in either mode and layout.

    layout "head": q, k, v [B,H,N,d], logf / lse / c [B,H,N] (as attn_fwd);
    layout "token": q, k, v [B,N,H,d], logf / lse / c [B,N,H] (the projections' layout before
    the head permute).  Outputs are written in the inputs' layout.
    """
    if layout not in ("head", "token"):
        raise ValueError(f"layout must be 'head' or 'token', got {layout!r}")
    if layout == "token":
        B, N, H, d = q.shape
        dt = _DTYPES.get(q.dtype)
        if dt is None:
            raise ValueError(f"unsupported dtype {q.dtype}")
        for name, t in (("q", q), ("k", k), ("v", v)):
            _need(t, name, q.dtype)
            if tuple(t.shape) != (B, N, H, d):
                raise ValueError(f"{name} shape {tuple(t.shape)} != {(B, N, H, d)}")
        _need(logf, "logf", torch.float32)
        if tuple(logf.shape) != (B, N, H):
            raise ValueError(f"logf shape {tuple(logf.shape)} != {(B, N, H)}")
        o = _alloc_or_check(out, "out", (B, N, H, d), q.dtype, q.device)
        lse = _alloc_or_check(lse, "lse", (B, N, H), torch.float32, q.device) if want_lse else None
        c = _alloc_or_check(c, "c", (B, N, H), torch.float32, q.device) if want_c else None
        code = FOX_TOKEN_MAJOR
    else:
        B, H, N, d = q.shape
        dt, o, lse, c = _fwd_outputs(q, k, v, logf, out, lse, c, want_lse, want_c)
        code = FOX_HEAD_MAJOR
    scale = _default_scale(d) if scale is None else float(scale)
    st = lib().fox_attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(logf), _ptr(o), _ptr(lse), _ptr(c), B, H, N, d, scale,
                               dt, 1 if causal else 0, code, _stream())
    check("fox_attn_fwd_ex", st)
    return o, lse, c


def attn_fwd_pruned_workspace_bytes(b: int, h: int, n: int, d: int) -> int:
    return int(lib().fox_attn_fwd_pruned_workspace_bytes(b, h, n, d))


def attn_fwd_pruned(q, k, v, logf, scale: float | None = None, out=None, lse=None, c=None, workspace=None,
                    want_lse: bool = True, want_c: bool = True):
    """fox_attn_fwd_pruned: attn_fwd with gate-aware tile skipping (equal to fp32 rounding).

    ``workspace``: uint8 device tensor of at least attn_fwd_pruned_workspace_bytes(B, H, N, d)
    bytes (allocated here when None).
    """
    B, H, N, d = q.shape
    dt, o, lse, c = _fwd_outputs(q, k, v, logf, out, lse, c, want_lse, want_c)
    wb = attn_fwd_pruned_workspace_bytes(B, H, N, d)
    workspace = _workspace(workspace, wb, q.device)
    scale = _default_scale(d) if scale is None else float(scale)
    st = lib().fox_attn_fwd_pruned(_ptr(q), _ptr(k), _ptr(v), _ptr(logf), _ptr(o), _ptr(lse), _ptr(c),
                                   _ptr(workspace), _nbytes(workspace), B, H, N, d, scale, dt, _stream())
    check("fox_attn_fwd_pruned", st)
    return o, lse, c


def attn_bwd_workspace_bytes(b: int, h: int, n: int, d: int) -> int:
    return int(lib().fox_attn_bwd_workspace_bytes(b, h, n, d))


def attn_bwd(q, k, v, o, dout, lse, logf, causal: bool = True, scale: float | None = None, dq=None, dk=None,
             dv=None, dlogf=None, workspace=None, layout: str = "head"):
    """Gradients of FoX attention. q, k, v, o, dout: [B,H,N,d], all bf16 or all fp32 (o and lse [B,H,N]
    as attn_fwd / attn_fwd_noncausal returned them); logf [B,H,N] the log gates the forward was
    given.  Returns (dq, dk, dv, dlogf).

    layout "token" (fox_attn_bwd_ex): every tensor [B,N,H,d] and lse / logf / dlogf [B,N,H], as
    attn_fwd_ex(..., layout="token") reads and writes them."""
    if layout not in ("head", "token"):
        raise ValueError(f"layout must be 'head' or 'token', got {layout!r}")
    if layout == "token":
        B, N, H, d = q.shape
        tshape, vshape = (B, N, H, d), (B, N, H)
    else:
        B, H, N, d = q.shape
        tshape, vshape = (B, H, N, d), (B, H, N)
    dt = _DTYPES.get(q.dtype)
    if dt is None:
        raise ValueError(f"attn_bwd takes bf16 or fp32 tensors, got {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _need(t, name, q.dtype)
        if tuple(t.shape) != tshape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != {tshape}")
    for name, t in (("lse", lse), ("logf", logf)):
        _need(t, name, torch.float32)
        if tuple(t.shape) != vshape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != {vshape}")
    dq = _alloc_or_check(dq, "dq", tshape, q.dtype, q.device)
    dk = _alloc_or_check(dk, "dk", tshape, q.dtype, q.device)
    dv = _alloc_or_check(dv, "dv", tshape, q.dtype, q.device)
    dlogf = _alloc_or_check(dlogf, "dlogf", vshape, torch.float32, q.device)
    workspace = _workspace(workspace, attn_bwd_workspace_bytes(B, H, N, d), q.device)
    scale = _default_scale(d) if scale is None else float(scale)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(logf), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(dlogf), _ptr(workspace), _nbytes(workspace), B, H, N, d, scale, dt, 1 if causal else 0)
    if layout == "token":
        check("fox_attn_bwd_ex", lib().fox_attn_bwd_ex(*args, FOX_TOKEN_MAJOR, _stream()))
    else:
        check("fox_attn_bwd", lib().fox_attn_bwd(*args, _stream()))
    return dq, dk, dv, dlogf


def attn_bwd_staged_workspace_bytes(b: int, h: int, n: int, d: int) -> int:
    return int(lib().fox_attn_bwd_staged_workspace_bytes(b, h, n, d))


def attn_bwd_staged(q, k, v, o, dout, lse, logf, scale: float | None = None, dq=None, dk=None, dv=None,
                    dlogf=None, workspace=None, layout: str = "head"):
    """attn_bwd in decoder mode for bf16 tensors with d = 128 through fox_attn_bwd_staged: the
    key-side kernel stores dS (about N*N bytes per head of workspace) and dQ is contracted from it.
    layout as attn_bwd.  Returns (dq, dk, dv, dlogf)."""
    if layout not in ("head", "token"):
        raise ValueError(f"layout must be 'head' or 'token', got {layout!r}")
    if layout == "token":
        B, N, H, d = q.shape
        tshape, vshape = (B, N, H, d), (B, N, H)
    else:
        B, H, N, d = q.shape
        tshape, vshape = (B, H, N, d), (B, H, N)
    if q.dtype != torch.bfloat16:
        raise ValueError(f"attn_bwd_staged takes bf16 tensors, got {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _need(t, name, q.dtype)
        if tuple(t.shape) != tshape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != {tshape}")
    for name, t in (("lse", lse), ("logf", logf)):
        _need(t, name, torch.float32)
        if tuple(t.shape) != vshape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != {vshape}")
    dq = _alloc_or_check(dq, "dq", tshape, q.dtype, q.device)
    dk = _alloc_or_check(dk, "dk", tshape, q.dtype, q.device)
    dv = _alloc_or_check(dv, "dv", tshape, q.dtype, q.device)
    dlogf = _alloc_or_check(dlogf, "dlogf", vshape, torch.float32, q.device)
    workspace = _workspace(workspace, attn_bwd_staged_workspace_bytes(B, H, N, d), q.device)
    scale = _default_scale(d) if scale is None else float(scale)
    check("fox_attn_bwd_staged", lib().fox_attn_bwd_staged(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(logf), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(dlogf), _ptr(workspace), _nbytes(workspace), B, H, N, d, scale, FOX_BF16,
        FOX_TOKEN_MAJOR if layout == "token" else FOX_HEAD_MAJOR, _stream()))
    return dq, dk, dv, dlogf


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _workspace(ws, nbytes: int, device):
    """The caller's workspace (a contiguous device tensor; its size is checked by the library) or a new one."""
    if ws is None:
        return torch.empty(max(nbytes, 16), device=device, dtype=torch.uint8)
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    if ws.device != device:
        raise ValueError(f"workspace is on {ws.device}, the inputs on {device}")
    return ws


def decode_workspace_bytes(s: int, h: int, l: int, d: int) -> int:
    return int(lib().fox_attn_decode_workspace_bytes(s, h, l, d))


def _decode_prep(q, k_cache, v_cache, c_cache, logf_new, out, lse, workspace, want_lse):
    S, H, d = q.shape
    L = k_cache.shape[2]
    dt = _DTYPES.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    _need(q, "q", q.dtype)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, name, q.dtype)
        if tuple(t.shape) != (S, H, L, d):
            raise ValueError(f"{name} shape {tuple(t.shape)} != {(S, H, L, d)}")
    _need(c_cache, "c_cache", torch.float32)
    _need(logf_new, "logf_new", torch.float32)
    if tuple(c_cache.shape) != (S, H, L) or tuple(logf_new.shape) != (S, H):
        raise ValueError("c_cache must be [S,H,L] and logf_new [S,H]")
    o = _alloc_or_check(out, "out", (S, H, d), q.dtype, q.device)
    lse = _alloc_or_check(lse, "lse", (S, H), torch.float32, q.device) if want_lse else None
    if workspace is not False:  # False: no workspace at all (the no-allocation entry point)
        workspace = _workspace(workspace, decode_workspace_bytes(S, H, L, d), q.device)
    return S, H, L, d, dt, o, lse, workspace


def attn_decode(q, k_cache, v_cache, c_cache, logf_new, scale: float | None = None, out=None, lse=None,
                workspace=None, want_lse: bool = True):
    """One decode step. q: [S,H,d]; caches [S,H,L,d] with the new token at slot L-1;
    c_cache [S,H,L] fp32 (slot L-1 is written); logf_new [S,H] fp32.  Returns (o, lse)."""
    S, H, L, d, dt, o, lse, ws = _decode_prep(q, k_cache, v_cache, c_cache, logf_new, out, lse, workspace, want_lse)
    st = lib().fox_attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(c_cache), _ptr(logf_new), _ptr(o),
                               _ptr(lse), _ptr(ws), _nbytes(ws), S, H, L, d,
                               float(_default_scale(d) if scale is None else scale), dt, _stream())
    check("fox_attn_decode", st)
    return o, lse


def attn_decode_noalloc(q, k_cache, v_cache, c_cache, logf_new, scale: float | None = None, out=None, lse=None,
                        want_lse: bool = True):
    """fox_attn_decode_noalloc: attn_decode whose split records live in the library's fixed device
    scratch (no workspace).  Pass ``out`` (and ``lse``) to make the call allocate nothing at all."""
    S, H, L, d, dt, o, lse, _ = _decode_prep(q, k_cache, v_cache, c_cache, logf_new, out, lse, False, want_lse)
    st = lib().fox_attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(c_cache), _ptr(logf_new),
                                       _ptr(o), _ptr(lse), S, H, L, d,
                                       float(_default_scale(d) if scale is None else scale), dt, _stream())
    check("fox_attn_decode_noalloc", st)
    return o, lse


def attn_decode_ragged(q, k_cache, v_cache, c_cache, logf_new, cache_lens, scale: float | None = None, out=None,
                       lse=None, workspace=None, want_lse: bool = True):
    """attn_decode where sequence s uses the first cache_lens[s] slots (int32 device tensor [S])
    of caches allocated for L slots; its new token sits at slot cache_lens[s]-1."""
    S, H, L, d, dt, o, lse, ws = _decode_prep(q, k_cache, v_cache, c_cache, logf_new, out, lse, workspace, want_lse)
    _need(cache_lens, "cache_lens", torch.int32)
    if tuple(cache_lens.shape) != (S,):
        raise ValueError(f"cache_lens shape {tuple(cache_lens.shape)} != {(S,)}")
    st = lib().fox_attn_decode_ragged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(c_cache), _ptr(logf_new),
                                      _ptr(cache_lens), _ptr(o), _ptr(lse), _ptr(ws), _nbytes(ws),
                                      S, H, L, d, float(_default_scale(d) if scale is None else scale), dt, _stream())
    check("fox_attn_decode_ragged", st)
    return o, lse


def attn_decode_paged(q, k_pages, v_pages, c_pages, block_table, cache_lens, logf_new, scale: float | None = None,
                      out=None, lse=None, workspace=None, want_lse: bool = True):
    """attn_decode_ragged with the caches in pages: k_pages, v_pages [num_pages, H, P, d],
    c_pages [num_pages, H, P] fp32, block_table [S, max_pages] int32 (logical slot j of sequence s
    is row j % P of page block_table[s, j // P]), cache_lens [S] int32.  Returns (o, lse)."""
    S, H, d = q.shape
    NP, H2, P, d2 = k_pages.shape
    dt = _DTYPES.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if (H2, d2) != (H, d):
        raise ValueError(f"k_pages shape {tuple(k_pages.shape)} does not match q {tuple(q.shape)}")
    _need(q, "q", q.dtype)
    for name, t in (("k_pages", k_pages), ("v_pages", v_pages)):
        _need(t, name, q.dtype)
        if tuple(t.shape) != (NP, H, P, d):
            raise ValueError(f"{name} shape {tuple(t.shape)} != {(NP, H, P, d)}")
    _need(c_pages, "c_pages", torch.float32)
    _need(logf_new, "logf_new", torch.float32)
    _need(block_table, "block_table", torch.int32)
    _need(cache_lens, "cache_lens", torch.int32)
    if tuple(c_pages.shape) != (NP, H, P) or tuple(logf_new.shape) != (S, H):
        raise ValueError("c_pages must be [num_pages,H,P] and logf_new [S,H]")
    if block_table.dim() != 2 or block_table.shape[0] != S or tuple(cache_lens.shape) != (S,):
        raise ValueError("block_table must be [S, max_pages] and cache_lens [S]")
    maxp = block_table.shape[1]
    o = _alloc_or_check(out, "out", (S, H, d), q.dtype, q.device)
    lse = _alloc_or_check(lse, "lse", (S, H), torch.float32, q.device) if want_lse else None
    ws = _workspace(workspace, decode_workspace_bytes(S, H, maxp * P, d), q.device)
    st = lib().fox_attn_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(c_pages), _ptr(block_table),
                                     _ptr(cache_lens), _ptr(logf_new), _ptr(o), _ptr(lse),
                                     _ptr(ws), _nbytes(ws), S, H, NP, P, maxp, d,
                                     float(_default_scale(d) if scale is None else scale), dt, _stream())
    check("fox_attn_decode_paged", st)
    return o, lse
