"""Host-side checks of the C ABI: the library loads, exports every declared entry
point, and rejects bad arguments with the documented status before launching
anything (no GPU needed: every call here fails validation)."""

from __future__ import annotations

import functools

import ctypes
import os
import re
import subprocess

import pytest

from forget_gated_causal_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fox.h")

# fake, never dereferenced device addresses (16-byte aligned, far apart)
A, B, C, D, E, F, G, H = (0x10_0000_0000 * (i + 1) for i in range(8))
OK, INVALID, UNSUP, WS = _lib.FOX_OK, _lib.FOX_ERR_INVALID_ARG, _lib.FOX_ERR_UNSUPPORTED, _lib.FOX_ERR_WORKSPACE


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fox_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_are_exported(L):
    names = declared_functions()
    assert names == sorted(_lib.SIGNATURES), names
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fox_[a-z0-9_]+)", out))
    for n in names:
        assert n in exported, f"{n} not exported"
        assert getattr(L, n) is not None


def test_status_strings(L):
    for s in range(5):
        assert len(_lib.status_string(s)) > 0
    assert _lib.status_string(99) == "unknown status"


def test_decode_workspace_bytes(L):
    f = L.fox_attn_decode_workspace_bytes
    assert f(64, 32, 8192, 128) > 0
    assert f(64, 32, 8192, 128) % (4 * 130) == 0
    assert f(0, 32, 8192, 128) == 0 and f(1, 1, 0, 128) == 0 and f(1, 1, 10, 48) == 0
    assert f(1, 1, 1, 32) == 1 * 34 * 4  # one split for a single key


def _fwd(L, q=A, k=B, v=C, logf=D, o=E, lse=F, c=G, b=1, h=2, n=128, d=32, scale=0.17, dt=_lib.FOX_F32,
         fn="fox_attn_fwd"):
    return getattr(L, fn)(q, k, v, logf, o, lse, c, b, h, n, d, scale, dt, None)


@pytest.mark.parametrize("fn", ["fox_attn_fwd", "fox_attn_fwd_noncausal"])
def test_fwd_rejects_bad_arguments(L, fn):
    _fwd = functools.partial(globals()["_fwd"], fn=fn)
    assert _fwd(L, q=None) == INVALID
    assert _fwd(L, o=None) == INVALID
    assert _fwd(L, logf=None) == INVALID
    assert _fwd(L, n=0) == INVALID
    assert _fwd(L, b=-1) == INVALID
    assert _fwd(L, n=(1 << 22) + 1) == INVALID
    assert _fwd(L, d=48) == UNSUP
    assert _fwd(L, d=256) == UNSUP
    assert _fwd(L, dt=7) == UNSUP
    assert _fwd(L, scale=0.0) == INVALID
    assert _fwd(L, scale=float("nan")) == INVALID
    assert _fwd(L, scale=float("inf")) == INVALID
    assert _fwd(L, q=A + 8) == INVALID  # not 16-byte aligned
    assert _fwd(L, lse=F + 2) == INVALID  # not 4-byte aligned
    assert _fwd(L, o=A) == INVALID  # output aliases q
    assert _fwd(L, c=D) == INVALID  # c aliases logf
    assert _fwd(L, lse=G) == INVALID  # lse aliases c


def _fwdp(L, q=A, k=B, v=C, logf=D, o=E, lse=F, c=G, ws=H, wsb=1 << 20, b=1, h=2, n=128, d=64, scale=0.17,
          dt=_lib.FOX_BF16):
    return L.fox_attn_fwd_pruned(q, k, v, logf, o, lse, c, ws, wsb, b, h, n, d, scale, dt, None)


def test_fwd_pruned_workspace_bytes(L):
    f = L.fox_attn_fwd_pruned_workspace_bytes
    assert f(2, 16, 4096, 128) == 2 * 16 * 64 * 4  # one float per (batch, head, 64-key tile)
    assert f(1, 1, 65, 64) == 2 * 4
    assert f(0, 1, 10, 64) == 0 and f(1, 1, 10, 48) == 0 and f(1, 1, 0, 64) == 0


def test_bwd_workspace_bytes(L):
    f = L.fox_attn_bwd_workspace_bytes
    # per head: row vectors a_i, D_i, cl_i padded to a multiple of 64, the row and column sums and
    # an lse correction (fp32), plus one fp64 gate-sum start per 32 positions of n rounded up to 128
    assert f(2, 16, 4096, 128) == 32 * ((3 * 4096 + 3 * 4096) * 4 + 128 * 8)
    assert f(1, 3, 65, 64) == 3 * ((3 * 128 + 3 * 65) * 4 + 4 * 8)
    assert f(1, 1, 1, 32) == (3 * 64 + 3) * 4 + 4 * 8
    assert f(1, 1, 129, 32) == (3 * 192 + 3 * 129) * 4 + 8 * 8
    assert f(0, 1, 10, 64) == 0 and f(1, 1, 10, 48) == 0 and f(1, 1, 0, 64) == 0


def test_fwd_pruned_rejects_bad_arguments(L):
    # the forward's own checks apply unchanged
    assert _fwdp(L, q=None) == INVALID
    assert _fwdp(L, n=0) == INVALID
    assert _fwdp(L, d=48) == UNSUP
    assert _fwdp(L, scale=0.0) == INVALID
    assert _fwdp(L, o=A) == INVALID
    # workspace: present, 16-byte aligned, large enough, disjoint from the tensors
    assert _fwdp(L, ws=None) == _lib.FOX_ERR_WORKSPACE
    assert _fwdp(L, ws=H + 4) == _lib.FOX_ERR_WORKSPACE
    assert _fwdp(L, wsb=3) == _lib.FOX_ERR_WORKSPACE
    assert _fwdp(L, ws=D) == INVALID  # overlaps logf


def test_cumsum_rejects_bad_arguments(L):
    f = L.fox_logf_cumsum
    assert f(None, A, 1, 10, None) == INVALID
    assert f(A, None, 1, 10, None) == INVALID
    assert f(A, B, 0, 10, None) == INVALID
    assert f(A, B, 1, 0, None) == INVALID
    assert f(A, A + 4, 1, 10, None) == INVALID  # overlapping
    assert f(A + 1, B, 1, 10, None) == INVALID


def _dec(L, q=A, k=B, v=C, cc=D, ln=E, o=F, lse=G, ws=H, wsb=1 << 30, s=2, h=2, l=100, d=64, scale=0.1,
         dt=_lib.FOX_BF16):
    return L.fox_attn_decode(q, k, v, cc, ln, o, lse, ws, wsb, s, h, l, d, scale, dt, None)


def test_decode_rejects_bad_arguments(L):
    assert _dec(L, q=None) == INVALID
    assert _dec(L, cc=None) == INVALID
    assert _dec(L, l=0) == INVALID
    assert _dec(L, d=96) == UNSUP
    assert _dec(L, dt=3) == UNSUP
    assert _dec(L, scale=-1.0) == INVALID
    assert _dec(L, k=B + 4) == INVALID
    assert _dec(L, ws=None) == WS
    assert _dec(L, wsb=16) == WS
    assert _dec(L, ws=H + 8) == WS
    assert _dec(L, o=B) == INVALID  # output inside the K cache
    assert _dec(L, ws=C) == INVALID  # workspace inside the V cache


# Decode buffers for the alias checks: argument -> (address, bytes) at s=2, h=2, l=100, d=64, bf16
# (the workspace extent is the size the library checks: what it needs for these sizes).
def _dec_bufs(L):
    return {"q": (A, 2 * 2 * 64 * 2), "k": (B, 2 * 2 * 100 * 64 * 2), "v": (C, 2 * 2 * 100 * 64 * 2),
            "cc": (D, 2 * 2 * 100 * 4), "ln": (E, 2 * 2 * 4), "o": (F, 2 * 2 * 64 * 2), "lse": (G, 2 * 2 * 4),
            "ws": (H, L.fox_attn_decode_workspace_bytes(2, 2, 100, 64))}


@pytest.mark.parametrize("out", ["o", "lse", "cc", "ws"])
def test_decode_rejects_every_written_alias(L, out):
    """Each buffer the decode step writes (o, lse, the c slot, the workspace) may overlap no other
    argument: placed at the start, and at the last 16-byte-aligned word, of every other buffer."""
    bufs = _dec_bufs(L)
    assert bufs["ws"][1] > 0
    for other, (addr, nbytes) in bufs.items():
        if other == out:
            continue
        for at in (addr, addr + ((nbytes - 4) & ~15)):
            assert _dec(L, **{out: at}) == INVALID, (out, other, hex(at))


def test_decode_ragged_rejects_aliased_lengths(L):
    """The ragged step's length array may overlap no written buffer."""
    bufs = _dec_bufs(L)
    for out in ("o", "lse", "cc", "ws"):
        assert _decr(L, lens=bufs[out][0], s=2, h=2) == INVALID, out


def test_decode_noalloc_rejects_bad_arguments(L):
    """The no-allocation decode validates like fox_attn_decode (no workspace to check) and refuses
    sizes whose split records exceed the fixed scratch before it touches any device."""
    def na(q=A, k=B, v=C, cc=D, ln=E, o=F, lse=G, s=2, h=2, l=100, d=64, scale=0.1, dt=_lib.FOX_BF16):
        return L.fox_attn_decode_noalloc(q, k, v, cc, ln, o, lse, s, h, l, d, scale, dt, None)
    assert na(q=None) == INVALID
    assert na(l=0) == INVALID
    assert na(d=96) == UNSUP
    assert na(scale=float("inf")) == INVALID
    assert na(o=B) == INVALID  # output inside the K cache
    assert na(lse=E) == INVALID  # lse over the new gates
    # 65536 (sequence, head) pairs at d = 128: 34 MB of split records > FOX_DECODE_SCRATCH_BYTES
    assert L.fox_attn_decode_workspace_bytes(1024, 64, 1, 128) > _lib.FOX_DECODE_SCRATCH_BYTES
    assert na(s=1024, h=64, l=1, d=128) == _lib.FOX_ERR_SCRATCH
    assert L.fox_status_string(_lib.FOX_ERR_SCRATCH).decode().startswith("sizes need more")


def _decr(L, lens=0x90_0000_0000, **kw):
    args = dict(q=A, k=B, v=C, cc=D, lnew=E, o=F, lse=G, ws=H, wsb=1 << 24, s=2, h=3, l=100, d=64, scale=0.125,
                dt=_lib.FOX_BF16)
    args.update(kw)
    a = args
    return L.fox_attn_decode_ragged(a["q"], a["k"], a["v"], a["cc"], a["lnew"], lens, a["o"], a["lse"], a["ws"],
                                    a["wsb"], a["s"], a["h"], a["l"], a["d"], a["scale"], a["dt"], None)


def test_decode_ragged_rejects_bad_arguments(L):
    assert _decr(L, lens=None) == INVALID
    assert _decr(L, lens=0x90_0000_0002) == INVALID  # not 4-byte aligned
    assert _decr(L, lens=D) == INVALID  # lengths inside the prefix-sum cache
    assert _decr(L, q=None) == INVALID
    assert _decr(L, l=0) == INVALID
    assert _decr(L, d=96) == UNSUP
    assert _decr(L, ws=None) == WS
    assert _decr(L, o=B) == INVALID


def _decp(L, **kw):
    args = dict(q=A, k=B, v=C, cc=D, table=0x90_0000_0000, lens=0x91_0000_0000, lnew=E, o=F, lse=G, ws=H,
                wsb=1 << 24, s=2, h=3, npages=40, page=64, maxp=8, d=64, scale=0.125, dt=_lib.FOX_BF16)
    args.update(kw)
    a = args
    return L.fox_attn_decode_paged(a["q"], a["k"], a["v"], a["cc"], a["table"], a["lens"], a["lnew"], a["o"],
                                   a["lse"], a["ws"], a["wsb"], a["s"], a["h"], a["npages"], a["page"], a["maxp"],
                                   a["d"], a["scale"], a["dt"], None)


def test_decode_paged_rejects_bad_arguments(L):
    assert _decp(L, table=None) == INVALID
    assert _decp(L, lens=None) == INVALID
    assert _decp(L, table=0x90_0000_0002) == INVALID  # not 4-byte aligned
    for page in (0, 8, 48, 8192):  # a power of two in [16, 4096]
        assert _decp(L, page=page) == INVALID
    assert _decp(L, npages=0) == INVALID
    assert _decp(L, maxp=0) == INVALID
    assert _decp(L, maxp=(1 << 22) // 64 + 1) == INVALID  # capacity above FOX_MAX_SEQ
    assert _decp(L, d=96) == UNSUP
    assert _decp(L, scale=0.0) == INVALID
    assert _decp(L, ws=None) == WS
    assert _decp(L, wsb=16) == WS
    assert _decp(L, o=B) == INVALID  # output inside the K pages
    assert _decp(L, cc=C) == INVALID  # written c pages inside the V pages
    assert _decp(L, ws=0x90_0000_0000) == INVALID  # workspace over the page table


def _bwd(L, layout=None, **kw):
    I, J, K, M = (0x10_0000_0000 * (i + 9) for i in range(4))
    args = dict(q=A, k=B, v=C, o=D, dout=E, lse=F, logf=G, dq=H, dk=I, dv=J, dl=K, ws=M, wsb=1 << 30, b=1, h=2, n=300,
                d=64, scale=0.125, dt=_lib.FOX_BF16, causal=1)
    args.update(kw)
    a = args
    pos = (a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["logf"], a["dq"], a["dk"], a["dv"], a["dl"], a["ws"],
           a["wsb"], a["b"], a["h"], a["n"], a["d"], a["scale"], a["dt"], a["causal"])
    if layout is None:
        return L.fox_attn_bwd(*pos, None)
    return L.fox_attn_bwd_ex(*pos, layout, None)


def test_bwd_rejects_bad_arguments(L):
    assert _bwd(L, dout=None) == INVALID
    assert _bwd(L, dl=None) == INVALID
    assert _bwd(L, n=0) == INVALID
    assert _bwd(L, d=96) == UNSUP
    assert _bwd(L, dt=7) == UNSUP  # unknown dtype
    assert _bwd(L, dt=_lib.FOX_F32, n=65535 * 64 + 1, h=1) == INVALID  # fp32: 64-row blocks along grid y
    assert _bwd(L, scale=float("nan")) == INVALID
    assert _bwd(L, q=A + 8) == INVALID  # 16-byte alignment
    assert _bwd(L, ws=None) == WS
    assert _bwd(L, wsb=64) == WS
    # outputs may not alias an input or each other, also when the pointers are equal
    assert _bwd(L, dq=A) == INVALID
    assert _bwd(L, dv=0x10_0000_0000 * 9) == INVALID  # dv == dk
    assert _bwd(L, dl=F) == INVALID  # dlogf == lse
    assert _bwd(L, dl=G) == INVALID  # dlogf == logf
    assert _bwd(L, logf=None) == INVALID
    assert _bwd(L, logf=G + 2) == INVALID  # 4-byte alignment
    assert _bwd(L, ws=H) == INVALID  # workspace == dq


def _staged_tiles(n):
    nqt, nkb = -(-n // 32), -(-n // 128)
    return nkb * nqt - 2 * nkb * (nkb - 1)


def test_bwd_staged_workspace_bytes(L):
    f = L.fox_attn_bwd_staged_workspace_bytes
    # the staged tiles: (128-key block, 32-query tile) pairs at or below the diagonal, counted by brute force
    for n in (1, 31, 32, 127, 128, 129, 1000, 4096):
        assert _staged_tiles(n) == sum(1 for kb in range(-(-n // 128)) for t in range(-(-n // 32)) if t >= 4 * kb)
    # fox_attn_bwd's workspace rounded up to 256 bytes, then 8 KiB (128 x 32 bf16) per staged tile
    for b, h, n in ((2, 16, 4096), (1, 1, 1), (1, 3, 1000), (1, 32, 16384)):
        base = -(-L.fox_attn_bwd_workspace_bytes(b, h, n, 128) // 256) * 256
        assert f(b, h, n, 128) == base + b * h * _staged_tiles(n) * 8192
    assert f(1, 1, 4096, 64) == 0 and f(1, 1, 0, 128) == 0 and f(0, 1, 10, 128) == 0
    # one head's staged tiles are addressed with 32-bit byte offsets
    assert _staged_tiles(46272) * 8192 <= 2**31 - 1 < _staged_tiles(46273) * 8192
    assert f(1, 1, 46272, 128) > 0 and f(1, 1, 46273, 128) == 0


def _bwds(L, **kw):
    I, J, K, M = (0x10_0000_0000 * (i + 9) for i in range(4))
    a = dict(q=A, k=B, v=C, o=D, dout=E, lse=F, logf=G, dq=H, dk=I, dv=J, dl=K, ws=M, wsb=1 << 30, b=1, h=2, n=300,
             d=128, scale=0.125, dt=_lib.FOX_BF16)
    a.update(kw)
    return L.fox_attn_bwd_staged(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["logf"], a["dq"], a["dk"],
                                 a["dv"], a["dl"], a["ws"], a["wsb"], a["b"], a["h"], a["n"], a["d"], a["scale"],
                                 a["dt"], a.get("layout", _lib.FOX_HEAD_MAJOR), None)


def test_bwd_staged_rejects_bad_arguments(L):
    # fox_attn_bwd's checks, with the staged workspace
    assert _bwds(L, dout=None) == INVALID
    assert _bwds(L, n=0) == INVALID
    assert _bwds(L, scale=float("nan")) == INVALID
    assert _bwds(L, q=A + 8) == INVALID
    assert _bwds(L, ws=None) == WS
    assert _bwds(L, wsb=L.fox_attn_bwd_staged_workspace_bytes(1, 2, 300, 128) - 1) == WS
    assert _bwds(L, ws=0x10_0000_0000 * 8) == INVALID  # workspace == dq
    assert _bwds(L, dv=0x10_0000_0000 * 9) == INVALID  # dv == dk
    # then its own: bf16, d = 128, and n whose staged tiles fit 32-bit offsets
    assert _bwds(L, d=64) == UNSUP
    assert _bwds(L, d=96) == UNSUP
    assert _bwds(L, dt=_lib.FOX_F32) == UNSUP
    assert _bwds(L, n=46273, h=1) == UNSUP
    # the layout as fox_attn_bwd_ex: unknown values, and token-major spans past 32-bit offsets
    assert _bwds(L, layout=2) == UNSUP
    assert _bwds(L, layout=_lib.FOX_TOKEN_MAJOR, n=40000, h=512) == UNSUP
    assert _bwds(L, layout=_lib.FOX_TOKEN_MAJOR, dout=None) == INVALID


def test_bwd_ex_layout_checks(L):
    # the same argument checks as fox_attn_bwd, then the layout's own
    assert _bwd(L, layout=_lib.FOX_TOKEN_MAJOR, dout=None) == INVALID
    assert _bwd(L, layout=_lib.FOX_HEAD_MAJOR, wsb=64) == WS
    assert _bwd(L, layout=2) == UNSUP
    assert _bwd(L, layout=-1) == UNSUP
    # token-major rows are h*d apart: one head's span must fit 32-bit byte offsets
    assert _bwd(L, layout=_lib.FOX_TOKEN_MAJOR, n=1 << 20, h=64, d=128) == UNSUP
    # fp32 elements are 4 bytes: the same span limit is reached at half the tokens
    assert _bwd(L, layout=_lib.FOX_TOKEN_MAJOR, dt=_lib.FOX_F32, n=65536, h=64, d=128) == UNSUP


def test_fwd_ex_layout_checks(L):
    def ex(layout, n=128, h=2, d=32, causal=1):
        return L.fox_attn_fwd_ex(A, B, C, D, E, F, G, 1, h, n, d, 0.17, _lib.FOX_F32, causal, layout, None)
    assert ex(7) == UNSUP
    assert ex(-1) == UNSUP
    # token-major rows are h*d apart: one head's span must fit 32-bit byte offsets
    assert ex(_lib.FOX_TOKEN_MAJOR, n=1 << 20, h=64, d=128) == UNSUP
    assert ex(_lib.FOX_HEAD_MAJOR, n=0) == INVALID
