"""fox_attn_decode_noalloc (the decode step with its split records in the library's fixed device
scratch, for callers that cannot allocate) against fox_attn_decode with a caller workspace: the
same kernels, so the results must be equal bit for bit.  Two calls in a row, the second smaller,
so the second runs on scratch that still holds the first call's records; then a call whose sizes
need more than the scratch holds is rejected without a launch."""

from __future__ import annotations

import ctypes

import pytest
import torch

import forget_gated_causal_amd as fox
import fox_inputs as fi
from forget_gated_causal_amd import _lib

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(tag, S, H, L, d):
    cfg = fi.DecodeConfig(tag, S, H, L, d, "bf16", 4.0, 2.0)
    inp = fi.decode_inputs(cfg)
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    c0 = fox.logf_cumsum(inp["logf_all"].to(DEV))
    c0[..., L - 1] = float("nan")
    lnew = inp["logf_all"][..., L - 1].contiguous().to(DEV)
    return cfg, inp, q, k, v, c0, lnew


def test_noalloc_decode_equals_workspace_decode():
    for tag, S, H, L, d in (("noalloc_a", 8, 32, 3000, 128), ("noalloc_b", 3, 4, 500, 64)):
        cfg, inp, q, k, v, c0, lnew = _case(tag, S, H, L, d)
        assert fox.decode_workspace_bytes(S, H, L, d) <= _lib.FOX_DECODE_SCRATCH_BYTES
        print(f"  {cfg.desc}: workspace {fox.decode_workspace_bytes(S, H, L, d)} bytes", flush=True)
        c_ref = c0.clone()
        o_ref, lse_ref = fox.attn_decode(q, k, v, c_ref, lnew, scale=inp["scale"])
        c_na = c0.clone()
        o_na = torch.full_like(q, float("nan"))
        lse_na = torch.full((S, H), float("nan"), device=DEV)
        st = _lib.lib().fox_attn_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), c_na.data_ptr(),
                                                lnew.data_ptr(), o_na.data_ptr(), lse_na.data_ptr(), S, H, L, d,
                                                ctypes.c_float(inp["scale"]), _lib.FOX_BF16,
                                                torch.cuda.current_stream().cuda_stream)
        assert st == _lib.FOX_OK, _lib.status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ref) and torch.equal(lse_na, lse_ref) and torch.equal(c_na, c_ref), tag
        # the binding's wrapper gives the same
        o_b, lse_b = fox.attn_decode_noalloc(q, k, v, c0.clone(), lnew, scale=inp["scale"])
        torch.cuda.synchronize()
        assert torch.equal(o_b, o_ref) and torch.equal(lse_b, lse_ref), tag


def test_noalloc_decode_rejects_sizes_beyond_scratch():
    """65536 (sequence, head) pairs of d = 128 need 34 MB of split records: FOX_ERR_SCRATCH, and the
    outputs stay untouched (real, in-bounds buffers of a one-slot cache)."""
    S, H, L, d = 1024, 64, 1, 128
    assert fox.decode_workspace_bytes(S, H, L, d) > _lib.FOX_DECODE_SCRATCH_BYTES
    q = torch.zeros(S, H, d, device=DEV, dtype=torch.bfloat16)
    k = torch.zeros(S, H, L, d, device=DEV, dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    cc = torch.zeros(S, H, L, device=DEV)
    ln = torch.zeros(S, H, device=DEV)
    o = torch.full_like(q, 7.0)
    lse = torch.full((S, H), 7.0, device=DEV)
    st = _lib.lib().fox_attn_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), cc.data_ptr(), ln.data_ptr(),
                                            o.data_ptr(), lse.data_ptr(), S, H, L, d, ctypes.c_float(0.088),
                                            _lib.FOX_BF16, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == _lib.FOX_ERR_SCRATCH
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
