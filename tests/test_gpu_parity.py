"""Parity of the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (max-abs over every compared element): 1e-5 for fp32 inputs and 2e-2
for bf16 inputs with fp32 accumulation, on O and lse; the gate prefix sums c
within one fp32 ulp of max|c| (they are accumulated in fp64 and rounded once).
For fp32 lse the bound is 1e-5 wherever an fp32 value can hold lse that closely
(|lse| < 256); above, where half an fp32 ulp is already 1.5e-5 or more, lse must
be the correctly rounded value up to 1e-6 (``_lse_bound``).
The oracle sees exactly the values the GPU sees (bf16 widened exactly, the fp32
scale widened).  Output buffers are pre-filled with NaN so an unwritten element
fails.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import forget_gated_causal_amd as fox
import fox_inputs as fi
import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
DEV = "cuda"


def _np(t):
    return t.detach().cpu().double().numpy()


def _ulp(x):
    return float(np.spacing(np.float32(np.max(np.abs(x)) if np.size(x) else 1.0)))


def _lse_bound(ref, dtype):
    """Per-element bound on lse: the tolerance, or for fp32 where the output format itself is
    coarser than 1e-5 (|lse| >= 256), half an fp32 ulp of the exact value plus 1e-6."""
    if dtype != "f32":
        return TOL[dtype]
    half_ulp = 0.5 * np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    return np.maximum(TOL["f32"], half_ulp + 1e-6)


def _lse_excess(got, ref, dtype):
    """max over elements of |got - ref| - bound (<= 0 when every element is within its bound)."""
    return float(np.max(np.abs(got - ref) - _lse_bound(ref, dtype))) if np.size(ref) else 0.0


def _run_fwd(inp):
    q, k, v, logf = (inp[n].to(DEV) for n in ("q", "k", "v", "logf"))
    nan = float("nan")
    o = torch.full_like(q, nan)
    lse = torch.full_like(logf, nan)
    c = torch.full_like(logf, nan)
    fox.attn_fwd(q, k, v, logf, scale=inp["scale"], out=o, lse=lse, c=c)
    torch.cuda.synchronize()
    return o, lse, c


def _check_fwd_full(inp, tol):
    o, lse, c = _run_fwd(inp)
    o_ref, lse_ref, c_ref = oracle.attn_fwd(_np(inp["q"]), _np(inp["k"]), _np(inp["v"]), _np(inp["logf"]),
                                            inp["scale"])
    eo, el, ec = np.abs(_np(o) - o_ref).max(), np.abs(_np(lse) - lse_ref).max(), np.abs(_np(c) - c_ref).max()
    print(f"  max|dO|={eo:.3e} max|dlse|={el:.3e} max|dc|={ec:.3e} (ulp {_ulp(c_ref):.1e})", flush=True)
    dt = "f32" if inp["q"].dtype == torch.float32 else "bf16"
    assert eo <= tol and _lse_excess(_np(lse), lse_ref, dt) <= 0 and ec <= _ulp(c_ref)
    return o, lse, c


# ---------------------------------------------------------------------------------- gate scan

@pytest.mark.parametrize("rows,n", [(1, 1), (3, 1000), (2, 1025), (5, 4097), (2048, 8192)])
def test_logf_cumsum_parity(rows, n):
    g = torch.Generator().manual_seed(rows * 7919 + n)
    logf = torch.nn.functional.logsigmoid((torch.randn(rows, n, generator=g) * 2 + 4).double()).float()
    c = fox.logf_cumsum(logf.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.logf_cumsum(logf.double().numpy())
    err = np.abs(_np(c) - ref).max()
    assert err <= _ulp(ref), err


# ---------------------------------------------------------------------------------- forward

@pytest.mark.parametrize("tag", ["c1", "c2", "c2_f1", "c2_alibi"])
def test_fwd_config_full_parity(tag):
    cfg = fi.FWD[tag]
    inp = fi.fwd_inputs(cfg)
    print(f"  {cfg.desc} inputs {fi.digest(inp['q'], inp['k'], inp['v'], inp['logf'])}", flush=True)
    _check_fwd_full(inp, TOL[cfg.dtype])


RAGGED = [(dt, d, n) for dt in ("f32", "bf16") for d in (32, 64, 128) for n in (1, 33, 64, 65, 129, 300)]


@pytest.mark.parametrize("dtype,d,n", RAGGED)
def test_fwd_ragged_parity(dtype, d, n):
    cfg = fi.FwdConfig(f"ragged_{dtype}_{d}_{n}", 2, 2, n, d, dtype, 1.0, 2.0)
    _check_fwd_full(fi.fwd_inputs(cfg), TOL[dtype])


# Grids with >= 2 blocks of 256 rows per CU select the 8-wave (256-row) forward; ragged tails included.
WIDE = [("bf16", 64, 4, 64, 777), ("bf16", 128, 4, 64, 777), ("bf16", 128, 2, 128, 1000), ("bf16", 64, 1, 512, 300)]


@pytest.mark.parametrize("dtype,d,B,H,n", WIDE)
def test_fwd_wide_grid_parity(dtype, d, B, H, n):
    cfg = fi.FwdConfig(f"wide_{d}_{B}_{H}_{n}", B, H, n, d, dtype, 2.0, 2.0)
    inp = fi.fwd_inputs(cfg)
    o, lse, c = _run_fwd(inp)
    rows = _sampled_rows(n)
    o_ref, lse_ref = oracle.attn_fwd_rows(_np(inp["q"]), _np(inp["k"]), _np(inp["v"]), _np(inp["logf"]),
                                          inp["scale"], rows)
    c_ref = oracle.logf_cumsum(_np(inp["logf"]))
    eo = np.abs(_np(o[:, :, rows]) - o_ref).max()
    el = np.abs(_np(lse[:, :, rows]) - lse_ref).max()
    ec = np.abs(_np(c) - c_ref).max()
    print(f"  {cfg.desc}: max|dO|={eo:.3e} max|dlse|={el:.3e} max|dc|={ec:.3e}", flush=True)
    assert eo <= TOL[dtype] and el <= TOL[dtype] and ec <= _ulp(c_ref)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def _sampled_rows(n):
    rows = {0, 1, 2, 31, 32, 63, 64, 65, 127, 128, 129, n // 2 - 1, n // 2, n - 129, n - 128, n - 65, n - 64,
            n - 2, n - 1}
    return np.array(sorted(r for r in rows if 0 <= r < n))


@pytest.mark.parametrize("tag", ["c3", "c4"])
def test_fwd_full_size_sampled_parity(tag):
    cfg = fi.FWD[tag]
    inp = fi.fwd_inputs(cfg)
    o, lse, c = _run_fwd(inp)
    rows = _sampled_rows(cfg.N)
    o_ref, lse_ref = oracle.attn_fwd_rows(_np(inp["q"]), _np(inp["k"]), _np(inp["v"]), _np(inp["logf"]),
                                          inp["scale"], rows)
    eo = np.abs(_np(o[:, :, rows]) - o_ref).max()
    el = np.abs(_np(lse[:, :, rows]) - lse_ref).max()
    c_ref = oracle.logf_cumsum(_np(inp["logf"]))
    ec = np.abs(_np(c) - c_ref).max()
    print(f"  {cfg.desc}: rows {len(rows)}/head max|dO|={eo:.3e} max|dlse|={el:.3e} max|dc|={ec:.3e}", flush=True)
    assert eo <= TOL[cfg.dtype] and el <= TOL[cfg.dtype] and ec <= _ulp(c_ref)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def _check_whole_heads(inp, o, lse, heads, causal=True, label=""):
    """Every row of the given (batch, head) pairs against the oracle's definition."""
    n = inp["q"].shape[2]
    for b, h in heads:
        o_ref, lse_ref = oracle.fwd_head_rows(_np(inp["q"][b, h]), _np(inp["k"][b, h]), _np(inp["v"][b, h]),
                                              _np(inp["logf"][b, h]), inp["scale"], np.arange(n), causal=causal)
        eo = np.abs(_np(o[b, h]) - o_ref).max()
        el = np.abs(_np(lse[b, h]) - lse_ref).max()
        print(f"  {label} head ({b},{h}) all {n} rows: max|dO|={eo:.3e} max|dlse|={el:.3e}", flush=True)
        assert eo <= TOL["bf16"] and el <= TOL["bf16"], (b, h, eo, el)


def test_fwd_c3_whole_heads():
    """c3 (B=2 H=16 N=4096 d=128) in the launch configuration the bench times (256-row blocks of 8
    waves): every row of the first and the last head against the oracle."""
    cfg = fi.FWD["c3"]
    inp = fi.fwd_inputs(cfg)
    o, lse, _ = _run_fwd(inp)
    _check_whole_heads(inp, o, lse, [(0, 0), (cfg.B - 1, cfg.H - 1)], label=cfg.desc)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def test_fwd_c4_whole_head():
    """c4 (B=1 H=32 N=16384 d=128): every one of the 16384 rows of the last head against the oracle."""
    cfg = fi.FWD["c4"]
    inp = fi.fwd_inputs(cfg)
    o, lse, _ = _run_fwd(inp)
    _check_whole_heads(inp, o, lse, [(0, cfg.H - 1)], label=cfg.desc)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def test_fwd_noncausal_wide_grid_whole_heads():
    """The unmasked mode on a grid that selects the 8-wave kernel (B=2 H=128 N=1000 d=128): two whole
    heads against the oracle."""
    cfg = fi.FwdConfig("ncwide_whole", 2, 128, 1000, 128, "bf16", 2.0, 2.0)
    inp = fi.fwd_inputs(cfg)
    o, lse, _ = _run_fwd_nc(inp)
    _check_whole_heads(inp, o, lse, [(0, 0), (1, 127)], causal=False, label=cfg.desc + " unmasked")


# Tile counts around the staging depths: the lead wave scans a tile's gates two tiles ahead of its
# MFMAs and loads them three ahead, so splits of 1..6 tiles (and their key-split halves) each take a
# different path through the prologue and the last steps.  Small grids (the key-split kernel at
# d = 64, 4-wave blocks at d = 128) and the 8-wave kernel, both modes, every row.
EDGES = [(d, B, H, n) for d in (64, 128) for (B, H) in ((1, 2), (2, 128)) for n in (128, 192, 193, 257, 320, 383)]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "unmasked"])
@pytest.mark.parametrize("d,B,H,n", EDGES)
def test_fwd_tile_count_edges(d, B, H, n, causal):
    cfg = fi.FwdConfig(f"edges_{d}_{B}_{H}_{n}", B, H, n, d, "bf16", 1.0, 2.0)
    inp = fi.fwd_inputs(cfg)
    o, lse, c = _run_fwd(inp) if causal else _run_fwd_nc(inp)
    heads = [(0, 0), (B - 1, H - 1)]
    _check_whole_heads(inp, o, lse, heads, causal=causal, label=cfg.desc + ("" if causal else " unmasked"))
    c_ref = oracle.logf_cumsum(_np(inp["logf"]))
    assert np.abs(_np(c) - c_ref).max() <= _ulp(c_ref)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


# Gates far from 1 (log f about -3 per step, and a constant -20): the gate biases of a 256-row block
# reach hundreds to thousands of nats, and the bf16 forward carries them in its fp32 S accumulators
# (as R_j / scale) through every k-step.  Both the 4-wave and the 8-wave kernels, both modes.
STRONG = [(64, 2, 2, 1000, "lsig", -3.0), (128, 2, 2, 1000, "lsig", -3.0), (128, 2, 2, 1000, "const", 20.0),
          (128, 2, 128, 1000, "lsig", -3.0), (128, 2, 128, 1000, "const", 20.0)]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "unmasked"])
@pytest.mark.parametrize("d,B,H,n,gate,g", STRONG)
def test_fwd_strong_gates(d, B, H, n, gate, g, causal):
    if gate == "const":
        cfg = fi.FwdConfig(f"strong_{d}_{B}_{H}_{n}_c{g}", B, H, n, d, "bf16", gate="const", m=g)
    else:
        cfg = fi.FwdConfig(f"strong_{d}_{B}_{H}_{n}_{g}", B, H, n, d, "bf16", g, 1.0)
    inp = fi.fwd_inputs(cfg)
    o, lse, _ = _run_fwd(inp) if causal else _run_fwd_nc(inp)
    heads = [(0, 0), (B - 1, H - 1)]
    _check_whole_heads(inp, o, lse, heads, causal=causal, label=cfg.desc + ("" if causal else " unmasked"))
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


# ---------------------------------------------------------------- forward without the causal mask

def _run_fwd_nc(inp):
    q, k, v, logf = (inp[n].to(DEV) for n in ("q", "k", "v", "logf"))
    nan = float("nan")
    o = torch.full_like(q, nan)
    lse = torch.full_like(logf, nan)
    c = torch.full_like(logf, nan)
    fox.attn_fwd_noncausal(q, k, v, logf, scale=inp["scale"], out=o, lse=lse, c=c)
    torch.cuda.synchronize()
    return o, lse, c


def _check_fwd_nc(inp, tol, rows=None):
    o, lse, c = _run_fwd_nc(inp)
    n = inp["q"].shape[2]
    rows = np.arange(n) if rows is None else rows
    o_ref, lse_ref = oracle.attn_fwd_rows(_np(inp["q"]), _np(inp["k"]), _np(inp["v"]), _np(inp["logf"]),
                                          inp["scale"], rows, causal=False)
    c_ref = oracle.logf_cumsum(_np(inp["logf"]))
    eo = np.abs(_np(o[:, :, rows]) - o_ref).max()
    el = np.abs(_np(lse[:, :, rows]) - lse_ref).max()
    ec = np.abs(_np(c) - c_ref).max()
    print(f"  unmasked: max|dO|={eo:.3e} max|dlse|={el:.3e} max|dc|={ec:.3e}", flush=True)
    dt = "f32" if inp["q"].dtype == torch.float32 else "bf16"
    assert eo <= tol and _lse_excess(_np(lse[:, :, rows]), lse_ref, dt) <= 0 and ec <= _ulp(c_ref)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("tag", ["c1", "c2", "c2_f1", "c2_alibi"])
def test_fwd_noncausal_config_parity(tag):
    cfg = fi.FWD[tag]
    _check_fwd_nc(fi.fwd_inputs(cfg), TOL[cfg.dtype])


@pytest.mark.parametrize("dtype,d,n", [(dt, d, n) for dt in ("f32", "bf16") for d in (32, 64, 128)
                                       for n in (1, 33, 65, 129, 300)])
def test_fwd_noncausal_ragged_parity(dtype, d, n):
    cfg = fi.FwdConfig(f"nc_{dtype}_{d}_{n}", 2, 2, n, d, dtype, 1.0, 2.0)
    _check_fwd_nc(fi.fwd_inputs(cfg), TOL[dtype])


@pytest.mark.parametrize("dtype,d,B,H,n", WIDE)
def test_fwd_noncausal_wide_grid_parity(dtype, d, B, H, n):
    cfg = fi.FwdConfig(f"ncwide_{d}_{B}_{H}_{n}", B, H, n, d, dtype, 2.0, 2.0)
    _check_fwd_nc(fi.fwd_inputs(cfg), TOL[dtype], rows=_sampled_rows(n))


def test_fwd_noncausal_last_row_equals_causal():
    """The last row sees every key in both modes."""
    inp = fi.fwd_inputs(fi.FwdConfig("nc_last", 2, 3, 777, 64, "bf16", 3.0, 1.5))
    o_nc, l_nc, c_nc = _run_fwd_nc(inp)
    o_c, l_c, c_c = _run_fwd(inp)
    assert (o_nc[:, :, -1].float() - o_c[:, :, -1].float()).abs().max().item() <= 2.0 ** -7
    assert (l_nc[:, :, -1] - l_c[:, :, -1]).abs().max().item() <= 2.0 ** -9 + 1e-5
    assert torch.equal(c_nc, c_c)


# ---------------------------------------------------------------- token-major layout

TOKEN_MAJOR = [("f32", 32, 1, 2, 128), ("bf16", 64, 4, 12, 1024), ("bf16", 128, 2, 3, 300), ("bf16", 32, 2, 2, 65),
               ("bf16", 64, 4, 64, 777), ("bf16", 128, 2, 128, 1000)]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dtype,d,B,H,n", TOKEN_MAJOR)
def test_fwd_token_major_equals_head_major(dtype, d, B, H, n, causal):
    """[B,N,H,d] tensors (the projections' layout before the head permute) give the head-major
    results bit for bit: the same arithmetic with other addresses.  The head-major results are
    checked against the oracle on sampled rows."""
    cfg = fi.FwdConfig(f"tm_{dtype}_{d}_{B}_{H}_{n}", B, H, n, d, dtype, 2.0, 2.0)
    inp = fi.fwd_inputs(cfg)
    q, k, v, logf = (inp[x].to(DEV) for x in ("q", "k", "v", "logf"))
    o_h, l_h, c_h = fox.attn_fwd_ex(q, k, v, logf, causal=causal, layout="head", scale=inp["scale"])
    tm = lambda t: t.permute(0, 2, 1, 3).contiguous()  # noqa: E731
    o_t, l_t, c_t = fox.attn_fwd_ex(tm(q), tm(k), tm(v), logf.permute(0, 2, 1).contiguous(), causal=causal,
                                    layout="token", scale=inp["scale"])
    torch.cuda.synchronize()
    assert torch.equal(o_t.permute(0, 2, 1, 3), o_h)
    assert torch.equal(l_t.permute(0, 2, 1), l_h) and torch.equal(c_t.permute(0, 2, 1), c_h)
    rows = _sampled_rows(n)
    o_ref, lse_ref = oracle.attn_fwd_rows(_np(inp["q"]), _np(inp["k"]), _np(inp["v"]), _np(inp["logf"]),
                                          inp["scale"], rows, causal=causal)
    eo = np.abs(_np(o_h[:, :, rows]) - o_ref).max()
    el = np.abs(_np(l_h[:, :, rows]) - lse_ref).max()
    print(f"  {cfg.desc} causal={causal}: max|dO|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= TOL[dtype] and el <= TOL[dtype]


# ---------------------------------------------------------------- forward with tile skipping

def _run_fwd_pruned(inp):
    q, k, v, logf = (inp[n].to(DEV) for n in ("q", "k", "v", "logf"))
    nan = float("nan")
    o = torch.full_like(q, nan)
    lse = torch.full_like(logf, nan)
    c = torch.full_like(logf, nan)
    fox.attn_fwd_pruned(q, k, v, logf, scale=inp["scale"], out=o, lse=lse, c=c)
    torch.cuda.synchronize()
    return o, lse, c


# (d, B, H, n, gate-logit mean, sd): low means forget fast, so most key tiles are skippable;
# mean 8 keeps every tile.  Small grids run the 4-wave kernel, the 256-head ones the 8-wave kernel.
PRUNED = [(64, 2, 2, 777, 0.0, 1.0), (128, 1, 2, 1000, 1.0, 2.0), (32, 2, 2, 300, -1.0, 1.0), (64, 2, 2, 65, 0.0, 1.0),
          (128, 2, 2, 129, 0.0, 1.0), (64, 2, 2, 512, 8.0, 0.5), (128, 2, 128, 1000, 1.0, 1.0),
          (64, 4, 64, 777, 0.0, 1.0)]


@pytest.mark.parametrize("d,B,H,n,mu,sigma", PRUNED)
def test_fwd_pruned_parity(d, B, H, n, mu, sigma):
    """The pruned forward against the oracle (the bf16 bound) and against the unpruned kernel:
    skipped keys weigh < 2^-24 of each row sum, so the two GPU results agree to output rounding."""
    cfg = fi.FwdConfig(f"pruned_{d}_{B}_{H}_{n}_{mu}", B, H, n, d, "bf16", mu, sigma)
    inp = fi.fwd_inputs(cfg)
    o, lse, c = _run_fwd_pruned(inp)
    o_full, lse_full, _ = _run_fwd(inp)
    rows = np.arange(n) if B * H <= 4 else _sampled_rows(n)
    o_ref, lse_ref = oracle.attn_fwd_rows(_np(inp["q"]), _np(inp["k"]), _np(inp["v"]), _np(inp["logf"]),
                                          inp["scale"], rows)
    c_ref = oracle.logf_cumsum(_np(inp["logf"]))
    eo = np.abs(_np(o[:, :, rows]) - o_ref).max()
    el = np.abs(_np(lse[:, :, rows]) - lse_ref).max()
    ec = np.abs(_np(c) - c_ref).max()
    do = (o.float() - o_full.float()).abs().max().item()
    dl = (lse - lse_full).abs().max().item()
    print(f"  {cfg.desc}: max|dO|={eo:.3e} max|dlse|={el:.3e} max|dc|={ec:.3e}; vs unpruned dO={do:.2e} "
          f"dlse={dl:.2e}", flush=True)
    assert eo <= TOL["bf16"] and el <= TOL["bf16"] and ec <= _ulp(c_ref)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    # Both sum the bf16-rounded weights, and for d <= 64 small grids the unpruned path runs the
    # key-split kernel (another summation order and max reference): they may differ at the level
    # of that rounding (a couple of bf16 ulps of O, ~2^-9 of a row sum), not more.
    assert do <= 2.0 ** -6 and dl <= 4e-3


def test_fwd_pruned_full_size_c3():
    cfg = fi.FWD["c3"]
    inp = fi.fwd_inputs(cfg)
    o, lse, c = _run_fwd_pruned(inp)
    rows = _sampled_rows(cfg.N)
    o_ref, lse_ref = oracle.attn_fwd_rows(_np(inp["q"]), _np(inp["k"]), _np(inp["v"]), _np(inp["logf"]),
                                          inp["scale"], rows)
    eo = np.abs(_np(o[:, :, rows]) - o_ref).max()
    el = np.abs(_np(lse[:, :, rows]) - lse_ref).max()
    print(f"  {cfg.desc} pruned: rows {len(rows)}/head max|dO|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= TOL["bf16"] and el <= TOL["bf16"]
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def test_fwd_pruned_c3_whole_heads():
    """The pruned forward at c3's full size (8-wave kernel with tile skipping): every row of the first
    and the last head against the oracle."""
    cfg = fi.FWD["c3"]
    inp = fi.fwd_inputs(cfg)
    o, lse, _ = _run_fwd_pruned(inp)
    _check_whole_heads(inp, o, lse, [(0, 0), (cfg.B - 1, cfg.H - 1)], label=cfg.desc + " pruned")


def test_fwd_pruned_f32_is_full():
    inp = fi.fwd_inputs(fi.FWD["c1"])
    o, lse, _ = _run_fwd_pruned(inp)
    o_ref, lse_ref, _ = oracle.attn_fwd(_np(inp["q"]), _np(inp["k"]), _np(inp["v"]), _np(inp["logf"]), inp["scale"])
    assert np.abs(_np(o) - o_ref).max() <= TOL["f32"] and np.abs(_np(lse) - lse_ref).max() <= TOL["f32"]


def test_fwd_deterministic():
    inp = fi.fwd_inputs(fi.FWD["c2"])
    a = _run_fwd(inp)
    b = _run_fwd(inp)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x, y.view(torch.uint8)
                           if y.dtype == torch.bfloat16 else y)


# ---------------------------------------------------------------------------------- decode

def _decode_caches(logf_all):
    """GPU cache from the library's scan; oracle cache from the oracle's scan (fp32-rounded like a real cache)."""
    L = logf_all.shape[-1]
    c_gpu = fox.logf_cumsum(logf_all.to(DEV))
    c_gpu[..., L - 1] = float("nan")
    c_ora = oracle.logf_cumsum(logf_all.double().numpy()).astype(np.float32).astype(np.float64)
    c_ora[..., L - 1] = np.nan
    return c_gpu, c_ora


def _run_decode(inp):
    L = inp["cfg"].L
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    c_gpu, c_ora = _decode_caches(inp["logf_all"])
    lnew = inp["logf_all"][..., L - 1].contiguous()
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), device=DEV)
    fox.attn_decode(q, k, v, c_gpu, lnew.to(DEV), scale=inp["scale"], out=o, lse=lse)
    torch.cuda.synchronize()
    return o, lse, c_gpu, c_ora, lnew


def _check_decode(inp, tol):
    L = inp["cfg"].L
    o, lse, c_gpu, c_ora, lnew = _run_decode(inp)
    o_ref, lse_ref, cnew_ref = oracle.attn_decode(_np(inp["q"]), _np(inp["k"]), _np(inp["v"]), c_ora,
                                                  lnew.double().numpy(), inp["scale"])
    eo, el = np.abs(_np(o) - o_ref).max(), np.abs(_np(lse) - lse_ref).max()
    ec = np.abs(_np(c_gpu[..., L - 1]) - cnew_ref).max()
    print(f"  max|dO|={eo:.3e} max|dlse|={el:.3e} max|dc_new|={ec:.3e}", flush=True)
    assert eo <= tol and el <= tol and ec <= _ulp(cnew_ref)


DECODE_SMALL = [(dt, d, L) for dt in ("f32", "bf16") for d in (32, 64, 128) for L in (1, 2, 77, 1000, 4097)]


@pytest.mark.parametrize("dtype,d,L", DECODE_SMALL)
def test_decode_small_parity(dtype, d, L):
    cfg = fi.DecodeConfig(f"dec_{dtype}_{d}_{L}", 2, 3, L, d, dtype, 4.0, 2.0)
    _check_decode(fi.decode_inputs(cfg), TOL[dtype])


def test_decode_full_size_sampled_parity():
    cfg = fi.DECODE["c5"]
    full = fi.decode_inputs(cfg)
    o, lse, c_gpu, _, lnew = _run_decode(full)
    seqs = [0, 9, 18, 27, 36, 45, 54, 63]
    sub = fi.decode_inputs(cfg, seqs=seqs)  # regenerated independently from the per-sequence seeds
    assert torch.equal(sub["k"][len(seqs) - 1], full["k"][63])
    c_ora = oracle.logf_cumsum(sub["logf_all"].double().numpy()).astype(np.float32).astype(np.float64)
    c_ora[..., cfg.L - 1] = np.nan
    o_ref, lse_ref, cnew_ref = oracle.attn_decode(_np(sub["q"]), _np(sub["k"]), _np(sub["v"]), c_ora,
                                                  sub["logf_all"][..., cfg.L - 1].double().numpy(), sub["scale"])
    eo = np.abs(_np(o[seqs]) - o_ref).max()
    el = np.abs(_np(lse[seqs]) - lse_ref).max()
    ec = np.abs(_np(c_gpu[seqs, :, cfg.L - 1]) - cnew_ref).max()
    print(f"  {cfg.desc}: seqs {seqs} max|dO|={eo:.3e} max|dlse|={el:.3e} max|dc_new|={ec:.3e}", flush=True)
    assert eo <= TOL["bf16"] and el <= TOL["bf16"] and ec <= _ulp(cnew_ref)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all() and torch.isfinite(c_gpu).all()


def test_decode_ignores_poisoned_workspace():
    """Every split writes its record before the combine reads it: a workspace filled with NaN (and
    one filled with large finite values) gives the same results as a fresh one, bit for bit, for
    the full and the ragged step."""
    cfg = fi.DecodeConfig("dec_poison", 3, 4, 3000, 128, "bf16", 4.0, 2.0)
    inp = fi.decode_inputs(cfg)
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    c0 = fox.logf_cumsum(inp["logf_all"].to(DEV))
    lnew = inp["logf_all"][..., cfg.L - 1].contiguous().to(DEV)
    lens = torch.tensor([3000, 1, 1777], dtype=torch.int32, device=DEV)
    nbytes = fox.decode_workspace_bytes(cfg.S, cfg.H, cfg.L, cfg.d)
    results = []
    for fill in (0.0, float("nan"), 3.0e38):
        ws = torch.full((max(nbytes, 16) // 4,), fill, device=DEV, dtype=torch.float32)
        cc = c0.clone()
        o, lse = fox.attn_decode(q, k, v, cc, lnew, scale=inp["scale"], workspace=ws)
        ws.fill_(fill)
        ccr = c0.clone()
        o_r, lse_r = fox.attn_decode_ragged(q, k, v, ccr, lnew, lens, scale=inp["scale"], workspace=ws)
        torch.cuda.synchronize()
        results.append((o, lse, cc, o_r, lse_r, ccr))
    for name, a, b, c in zip(("o", "lse", "c", "o_ragged", "lse_ragged", "c_ragged"), *results):
        assert torch.isfinite(a.float()).all(), name
        assert torch.equal(a, b) and torch.equal(a, c), name


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_equals_prefill_last_row(dtype):
    """Decode of token L-1 against a cache built by the forward (its c output) equals row L-1 of the forward."""
    B, H, N, d = 2, 4, 777, 128
    inp = fi.fwd_inputs(fi.FwdConfig(f"consist_{dtype}", B, H, N, d, dtype, 3.0, 1.5))
    q, k, v, logf = (inp[n].to(DEV) for n in ("q", "k", "v", "logf"))
    o, lse, c = fox.attn_fwd(q, k, v, logf, scale=inp["scale"])
    cache_c = c.clone()
    cache_c[..., N - 1] = float("nan")
    od, lsed = fox.attn_decode(q[:, :, N - 1].contiguous(), k, v, cache_c, logf[..., N - 1].contiguous(),
                               scale=inp["scale"])
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert (od.double() - o[:, :, N - 1].double()).abs().max().item() <= tol
    # The bf16 forward sums the bf16-rounded weights (those its P.V product uses), each within
    # 2^-9 of the fp32 weight the decode sums, so the two row sums differ by at most 2^-9
    # relative and the two lse by at most about 2^-9 (natural log); fp32 paths agree closely.
    assert (lsed - lse[..., N - 1]).abs().max().item() <= (2.0 ** -9 + 1e-5 if dtype == "bf16" else 1e-4)
    assert (cache_c[..., N - 1] - c[..., N - 1]).abs().max().item() <= _ulp(_np(c))


# ---------------------------------------------------------------------------------- ragged decode

def _ragged_lens(S, L, seed):
    g = torch.Generator().manual_seed(seed)
    lens = torch.randint(1, L + 1, (S,), generator=g, dtype=torch.int32)
    lens[0] = 1
    lens[-1] = L
    return lens


def _check_decode_ragged(inp, lens, tol, seqs=None):
    L = inp["cfg"].L
    S = inp["q"].shape[0]
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    la = inp["logf_all"]
    c_gpu = fox.logf_cumsum(la.to(DEV))
    c_ora = oracle.logf_cumsum(la.double().numpy()).astype(np.float32).astype(np.float64)
    lnew = torch.empty(S, la.shape[1])
    for s in range(S):
        Ls = int(lens[s])
        lnew[s] = la[s, :, Ls - 1]
        c_gpu[s, :, Ls - 1:] = float("nan")  # the slot the step writes, and the unused tail
        c_ora[s, :, Ls - 1:] = np.nan
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), device=DEV)
    fox.attn_decode_ragged(q, k, v, c_gpu, lnew.to(DEV), lens.to(DEV), scale=inp["scale"], out=o, lse=lse)
    torch.cuda.synchronize()
    seqs = list(range(S)) if seqs is None else seqs
    o_ref, lse_ref, cnew_ref = oracle.attn_decode_ragged(_np(inp["q"])[seqs], _np(inp["k"])[seqs],
                                                         _np(inp["v"])[seqs], c_ora[seqs],
                                                         lnew.double().numpy()[seqs], lens.numpy()[seqs],
                                                         inp["scale"])
    eo = np.abs(_np(o)[seqs] - o_ref).max()
    el = np.abs(_np(lse)[seqs] - lse_ref).max()
    cg = _np(c_gpu)
    ec = max(abs(cg[s, :, int(lens[s]) - 1] - cnew_ref[i]).max() for i, s in enumerate(seqs))
    tails_untouched = all(np.isnan(cg[s, :, int(lens[s]):]).all() for s in seqs)
    print(f"  ragged lens {lens.tolist()[:8]}...: max|dO|={eo:.3e} max|dlse|={el:.3e} max|dc_new|={ec:.3e}",
          flush=True)
    assert eo <= tol and el <= tol and ec <= _ulp(cnew_ref)
    assert tails_untouched


@pytest.mark.parametrize("dtype,d,L", [(dt, d, L) for dt in ("f32", "bf16") for d in (32, 64, 128)
                                       for L in (1, 77, 1000, 4097)])
def test_decode_ragged_parity(dtype, d, L):
    cfg = fi.DecodeConfig(f"ragged_dec_{dtype}_{d}_{L}", 5, 3, L, d, dtype, 4.0, 2.0)
    _check_decode_ragged(fi.decode_inputs(cfg), _ragged_lens(5, L, L + d), TOL[dtype])


@pytest.mark.parametrize("S", [1024, 1025])
def test_decode_ragged_many_sequences(S):
    """The split workgroups take the sequences longest first when there are at most 1024 of them
    (ranked on the device), in index order beyond that: both sides of the limit."""
    cfg = fi.DecodeConfig(f"ragged_many_{S}", S, 1, 40, 32, "bf16", 4.0, 2.0)
    _check_decode_ragged(fi.decode_inputs(cfg), _ragged_lens(S, cfg.L, 11), TOL["bf16"])


def test_decode_ragged_full_size_sampled():
    cfg = fi.DECODE["c5"]
    inp = fi.decode_inputs(cfg)
    lens = _ragged_lens(cfg.S, cfg.L, 5)
    _check_decode_ragged(inp, lens, TOL["bf16"], seqs=[0, 1, 17, 40, 63])


def test_decode_ragged_full_length_equals_decode():
    """With every length equal to the capacity the ragged step is the plain step, bit for bit."""
    cfg = fi.DecodeConfig("ragged_eq", 3, 4, 1500, 128, "bf16", 4.0, 2.0)
    inp = fi.decode_inputs(cfg)
    o1, lse1, c1, _, lnew = _run_decode(inp)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    c2, _ = _decode_caches(inp["logf_all"])
    lens = torch.full((cfg.S,), cfg.L, dtype=torch.int32, device=DEV)
    o2, lse2 = fox.attn_decode_ragged(q, k, v, c2, lnew.to(DEV), lens, scale=inp["scale"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(lse1, lse2) and torch.equal(c1, c2)


# ------------------------------------------------------------------------------ paged decode

def _paged_case(inp, lens, P, seed):
    """Ragged caches of capacity L (a multiple of P) scattered over shuffled pages of P slots, with
    3 spare pages; unused slots hold NaN.  Returns GPU and oracle views plus the ragged GPU caches."""
    S, H, L, d = inp["k"].shape
    maxp = L // P
    npages = S * maxp + 3
    g = torch.Generator().manual_seed(seed)
    table = torch.randperm(npages, generator=g)[: S * maxp].reshape(S, maxp).to(torch.int32)
    la = inp["logf_all"]
    c_dense = fox.logf_cumsum(la.to(DEV)).cpu()
    lnew = torch.empty(S, H)
    kp = torch.full((npages, H, P, d), float("nan"), dtype=inp["k"].dtype)
    vp = torch.full((npages, H, P, d), float("nan"), dtype=inp["v"].dtype)
    cp = torch.full((npages, H, P), float("nan"))
    for s in range(S):
        Ls = int(lens[s])
        lnew[s] = la[s, :, Ls - 1]
        c_dense[s, :, Ls - 1:] = float("nan")  # the slot the step writes, and the unused tail
        for i in range((Ls + P - 1) // P):
            pg, n0 = int(table[s, i]), i * P
            cnt = min(P, Ls - n0)
            kp[pg, :, :cnt] = inp["k"][s, :, n0:n0 + cnt]
            vp[pg, :, :cnt] = inp["v"][s, :, n0:n0 + cnt]
            cp[pg, :, :cnt] = c_dense[s, :, n0:n0 + cnt]
    return table, kp, vp, cp, c_dense, lnew


PAGED = [("bf16", 128, 64, 1024), ("bf16", 64, 16, 512), ("f32", 32, 256, 1024), ("bf16", 32, 4096, 8192)]


@pytest.mark.parametrize("dtype,d,P,L", PAGED)
def test_decode_paged_parity_and_equals_ragged(dtype, d, P, L):
    """Paged caches against the oracle's page gather, and bit-equal to the ragged step on the
    same logical caches (the same arithmetic with other addresses); unused page slots (NaN) are
    never read and the written c lands in the right page slot."""
    cfg = fi.DecodeConfig(f"paged_{dtype}_{d}_{P}_{L}", 5, 3, L, d, dtype, 4.0, 2.0)
    inp = fi.decode_inputs(cfg)
    lens = _ragged_lens(5, L, P + d)
    table, kp, vp, cp, c_dense, lnew = _paged_case(inp, lens, P, P + L)
    q = inp["q"].to(DEV)
    cp_gpu = cp.to(DEV)
    o, lse = fox.attn_decode_paged(q, kp.to(DEV), vp.to(DEV), cp_gpu, table.to(DEV), lens.to(DEV), lnew.to(DEV),
                                   scale=inp["scale"])
    c_r = c_dense.to(DEV)
    o_r, lse_r = fox.attn_decode_ragged(q, inp["k"].to(DEV), inp["v"].to(DEV), c_r, lnew.to(DEV), lens.to(DEV),
                                        scale=inp["scale"])
    torch.cuda.synchronize()
    assert torch.equal(o, o_r) and torch.equal(lse, lse_r)
    cpg, crg = cp_gpu.cpu(), c_r.cpu()
    for s in range(cfg.S):
        j = int(lens[s]) - 1
        assert torch.equal(cpg[int(table[s, j // P]), :, j % P], crg[s, :, j])
    o_ref, lse_ref, cnew_ref = oracle.attn_decode_paged(_np(inp["q"]), _np(kp), _np(vp), _np(cp), table.numpy(),
                                                        lens.numpy(), lnew.double().numpy(), inp["scale"])
    eo, el = np.abs(_np(o) - o_ref).max(), np.abs(_np(lse) - lse_ref).max()
    print(f"  paged P={P} lens {lens.tolist()}: max|dO|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= TOL[dtype] and el <= TOL[dtype]
    assert np.isfinite(_np(o)).all()


def test_decode_paged_full_size_equals_ragged():
    """c5's shape (S=64 H=32 L=8192 d=128) with 256-slot pages in a shuffled pool: bit-equal to the
    ragged step, which the full-size ragged test checks against the oracle."""
    cfg = fi.DECODE["c5"]
    inp = fi.decode_inputs(cfg)
    lens = _ragged_lens(cfg.S, cfg.L, 11)
    table, kp, vp, cp, c_dense, lnew = _paged_case(inp, lens, 256, 12)
    q = inp["q"].to(DEV)
    o, lse = fox.attn_decode_paged(q, kp.to(DEV), vp.to(DEV), cp.to(DEV), table.to(DEV), lens.to(DEV),
                                   lnew.to(DEV), scale=inp["scale"])
    del kp, vp
    o_r, lse_r = fox.attn_decode_ragged(q, inp["k"].to(DEV), inp["v"].to(DEV), c_dense.to(DEV), lnew.to(DEV),
                                        lens.to(DEV), scale=inp["scale"])
    torch.cuda.synchronize()
    assert torch.equal(o, o_r) and torch.equal(lse, lse_r)


# ---------------------------------------------------------------------------------- backward

# (d, B, H, n, causal, gate-logit mean, sd)
BWD = [(32, 1, 2, 65, True, 2.0, 1.0), (64, 2, 2, 300, True, 2.0, 2.0), (128, 1, 2, 257, True, 3.0, 1.5),
       (64, 2, 3, 129, False, 2.0, 1.0), (128, 2, 2, 200, False, 1.0, 2.0), (32, 3, 2, 1000, True, 4.0, 2.0),
       (64, 4, 12, 1024, True, 3.0, 1.5),
       # edges: one row; less than, exactly and one past a 32-query tile; exactly one 128-key block
       (64, 1, 1, 1, True, 2.0, 1.0), (128, 1, 1, 1, False, 2.0, 1.0), (128, 1, 2, 31, True, 2.0, 1.0),
       (32, 1, 1, 32, True, 2.0, 1.0), (64, 1, 1, 33, False, 2.0, 1.0), (64, 1, 2, 128, True, 2.0, 1.0),
       (128, 1, 1, 129, True, 2.0, 1.0),
       # grids above the single-launch limit (2 * heads * 128-blocks > 1024): the two-kernel path
       (32, 2, 16, 2100, False, 2.0, 1.0), (128, 2, 16, 2100, True, 3.0, 1.5)]


@pytest.mark.parametrize("d,B,H,n,causal,mu,sigma", BWD)
def test_bwd_parity(d, B, H, n, causal, mu, sigma):
    """fox_attn_bwd against the fp64 oracle's chain-rule gradients on the same bf16 inputs.

    Bound: bf16 rounds P and dS before the products (2^-9 relative each), the forward's O and
    lse enter through D_i and P, and the outputs are rounded to bf16; every gradient element
    is a sum of such terms, so the error is a small multiple of 2^-9 of the tensor's scale.
    Checked as max|gpu - ref| <= 2e-2 * max(1, max|ref|) per gradient tensor."""
    cfg = fi.FwdConfig(f"bwd_{d}_{B}_{H}_{n}_{causal}", B, H, n, d, "bf16", mu, sigma)
    inp = fi.fwd_inputs(cfg)
    q, k, v, logf = (inp[x].to(DEV) for x in ("q", "k", "v", "logf"))
    g = torch.Generator().manual_seed(n * 31 + d)
    dout = torch.randn(B, H, n, d, generator=g).to(torch.bfloat16)
    fwd = fox.attn_fwd if causal else fox.attn_fwd_noncausal
    o, lse, c = fwd(q, k, v, logf, scale=inp["scale"])
    dq, dk, dv, dl = fox.attn_bwd(q, k, v, o, dout.to(DEV), lse, logf, causal=causal, scale=inp["scale"])
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(_np(inp["q"]), _np(inp["k"]), _np(inp["v"]), _np(inp["logf"]), inp["scale"], _np(dout),
                          causal=causal)
    msg = []
    for name, got, r in zip(("dq", "dk", "dv", "dlogf"), (dq, dk, dv, dl), ref):
        err = np.abs(_np(got) - r).max()
        bound = 2e-2 * max(1.0, np.abs(r).max())
        msg.append(f"{name} {err:.2e} (max|ref| {np.abs(r).max():.2e})")
        assert torch.isfinite(got).all(), name
        assert err <= bound, (name, err, bound)
    print("  " + cfg.desc + ": " + ", ".join(msg), flush=True)


def test_bwd_c3_full_size_sampled_heads():
    """The backward at c3's full size (B=2 H=16 N=4096 d=128) in the bench's launch configuration;
    two whole heads (first and last) against the fp64 oracle, the rest checked finite."""
    cfg = fi.FWD["c3"]
    inp = fi.fwd_inputs(cfg)
    q, k, v, logf = (inp[x].to(DEV) for x in ("q", "k", "v", "logf"))
    g = torch.Generator().manual_seed(1)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    o, lse, c = fox.attn_fwd(q, k, v, logf, scale=inp["scale"])
    dq, dk, dv, dl = fox.attn_bwd(q, k, v, o, dout.to(DEV), lse, logf, scale=inp["scale"])
    torch.cuda.synchronize()
    for t in (dq, dk, dv, dl):
        assert torch.isfinite(t).all()
    for b, h in ((0, 0), (cfg.B - 1, cfg.H - 1)):
        ref = oracle.fwd_bwd_head(_np(inp["q"][b, h]), _np(inp["k"][b, h]), _np(inp["v"][b, h]),
                                  _np(inp["logf"][b, h]), inp["scale"], _np(dout[b, h]))
        msg = []
        for name, got, r in zip(("dq", "dk", "dv", "dlogf"), (dq, dk, dv, dl), ref):
            err = np.abs(_np(got[b, h]) - r).max()
            bound = 2e-2 * max(1.0, np.abs(r).max())
            msg.append(f"{name} {err:.2e} (max|ref| {np.abs(r).max():.2e})")
            assert err <= bound, (b, h, name, err, bound)
        print(f"  c3 head ({b},{h}): " + ", ".join(msg), flush=True)


# (B, H, n, gate-logit mean, sd): d = 128, decoder mode.  n covers one row, a partial tile, a
# partial and exactly one 128-key block, several blocks with a ragged tail, and a query block whose
# last waves lie past n (n not a multiple of 128).
BWD_STAGED = [(1, 1, 1, 2.0, 1.0), (1, 2, 31, 2.0, 1.0), (1, 1, 128, 2.0, 1.0), (2, 2, 257, 3.0, 1.5),
              (1, 3, 1000, 4.0, 2.0), (2, 3, 1500, -1.0, 1.0), (1, 2, 2049, 6.0, 1.0)]


def _bwd_case(cfg, seed):
    inp = fi.fwd_inputs(cfg)
    g = torch.Generator().manual_seed(seed)
    dout = torch.randn(cfg.B, cfg.H, cfg.N, cfg.d, generator=g).to(torch.bfloat16)
    return inp, dout


@pytest.mark.parametrize("B,H,n,mu,sigma", BWD_STAGED)
def test_bwd_staged_parity(B, H, n, mu, sigma):
    """fox_attn_bwd_staged against the fp64 oracle (bound as test_bwd_parity), and against
    fox_attn_bwd: dk and dv come from the same key-side arithmetic (bit-equal); dq and dlogf take
    the staged dS and agree with the default path to bf16 rounding."""
    cfg = fi.FwdConfig(f"bwd_staged_{B}_{H}_{n}", B, H, n, 128, "bf16", mu, sigma)
    inp, dout = _bwd_case(cfg, n * 7 + 3)
    q, k, v, logf = (inp[x].to(DEV) for x in ("q", "k", "v", "logf"))
    o, lse, c = fox.attn_fwd(q, k, v, logf, scale=inp["scale"])
    ws = torch.full((fox.attn_bwd_staged_workspace_bytes(B, H, n, 128),), 0xFF, dtype=torch.uint8, device=DEV)
    got = fox.attn_bwd_staged(q, k, v, o, dout.to(DEV), lse, logf, scale=inp["scale"], workspace=ws)
    base = fox.attn_bwd(q, k, v, o, dout.to(DEV), lse, logf, scale=inp["scale"])
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(_np(inp["q"]), _np(inp["k"]), _np(inp["v"]), _np(inp["logf"]), inp["scale"], _np(dout))
    msg = []
    for name, a, r in zip(("dq", "dk", "dv", "dlogf"), got, ref):
        err = np.abs(_np(a) - r).max()
        bound = 2e-2 * max(1.0, np.abs(r).max())
        msg.append(f"{name} {err:.2e} (max|ref| {np.abs(r).max():.2e})")
        assert torch.isfinite(a).all(), name
        assert err <= bound, (name, err, bound)
    assert torch.equal(got[1], base[1]) and torch.equal(got[2], base[2])
    for name, a, b in (("dq", got[0], base[0]), ("dlogf", got[3], base[3])):
        scale_ = max(1.0, b.float().abs().max().item())
        assert (a.float() - b.float()).abs().max().item() <= 8e-3 * scale_, name
    print("  " + cfg.desc + " staged: " + ", ".join(msg), flush=True)


@pytest.mark.parametrize("B,H,n", [(1, 2, 65), (2, 3, 300), (1, 16, 2100)])
def test_bwd_staged_token_major_equals_head_major(B, H, n):
    """fox_attn_bwd_staged on [B,N,H,d] tensors gives the head-major call's gradients bit for bit
    (only addresses differ), which test_bwd_staged_parity checks against the oracle."""
    cfg = fi.FwdConfig(f"bwd_staged_tm_{B}_{H}_{n}", B, H, n, 128, "bf16", 3.0, 1.5)
    inp, dout = _bwd_case(cfg, n + 17)
    q, k, v, logf = (inp[x].to(DEV) for x in ("q", "k", "v", "logf"))
    dout = dout.to(DEV)
    o, lse, c = fox.attn_fwd(q, k, v, logf, scale=inp["scale"])
    head = fox.attn_bwd_staged(q, k, v, o, dout, lse, logf, scale=inp["scale"])
    tm = lambda t: t.transpose(1, 2).contiguous()  # noqa: E731
    tok = fox.attn_bwd_staged(tm(q), tm(k), tm(v), tm(o), tm(dout), tm(lse), tm(logf), scale=inp["scale"],
                              layout="token")
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "dlogf"), head, tok):
        assert torch.equal(a, b.transpose(1, 2)), name


def test_bwd_staged_c3_full_size_sampled_heads():
    """The staged backward at c3's full size, in the bench's launch configuration: two whole heads
    against the fp64 oracle, every head's dk, dv bit-equal to fox_attn_bwd, and a second call
    (the workspace keeping the first call's dS) bit-equal to the first."""
    cfg = fi.FWD["c3"]
    inp = fi.fwd_inputs(cfg)
    q, k, v, logf = (inp[x].to(DEV) for x in ("q", "k", "v", "logf"))
    g = torch.Generator().manual_seed(1)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    o, lse, c = fox.attn_fwd(q, k, v, logf, scale=inp["scale"])
    ws = torch.empty(fox.attn_bwd_staged_workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.d), dtype=torch.uint8, device=DEV)
    got = fox.attn_bwd_staged(q, k, v, o, dout.to(DEV), lse, logf, scale=inp["scale"], workspace=ws)
    again = fox.attn_bwd_staged(q, k, v, o, dout.to(DEV), lse, logf, scale=inp["scale"], workspace=ws)
    base = fox.attn_bwd(q, k, v, o, dout.to(DEV), lse, logf, scale=inp["scale"])
    torch.cuda.synchronize()
    for x, y in zip(got, again):
        assert torch.equal(x, y)
    assert torch.equal(got[1], base[1]) and torch.equal(got[2], base[2])
    for t in got:
        assert torch.isfinite(t).all()
    for b, h in ((0, 0), (cfg.B - 1, cfg.H - 1)):
        ref = oracle.fwd_bwd_head(_np(inp["q"][b, h]), _np(inp["k"][b, h]), _np(inp["v"][b, h]),
                                  _np(inp["logf"][b, h]), inp["scale"], _np(dout[b, h]))
        msg = []
        for name, a, r in zip(("dq", "dk", "dv", "dlogf"), got, ref):
            err = np.abs(_np(a[b, h]) - r).max()
            bound = 2e-2 * max(1.0, np.abs(r).max())
            msg.append(f"{name} {err:.2e} (max|ref| {np.abs(r).max():.2e})")
            assert err <= bound, (b, h, name, err, bound)
        print(f"  c3 staged head ({b},{h}): " + ", ".join(msg), flush=True)


def test_bwd_repeatable():
    """Every backward output has one writer: two calls give bit-identical gradients."""
    cfg = fi.FwdConfig("bwd_rep", 2, 3, 700, 64, "bf16", 2.0, 1.0)
    inp = fi.fwd_inputs(cfg)
    q, k, v, logf = (inp[x].to(DEV) for x in ("q", "k", "v", "logf"))
    g = torch.Generator().manual_seed(5)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16).to(DEV)
    o, lse, c = fox.attn_fwd(q, k, v, logf, scale=inp["scale"])
    a = fox.attn_bwd(q, k, v, o, dout, lse, logf, scale=inp["scale"])
    b = fox.attn_bwd(q, k, v, o, dout, lse, logf, scale=inp["scale"])
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# (d, B, H, n, causal); the last two launch the two-kernel path (2 * heads * 128-blocks > 1024)
BWD_TOKEN = [(32, 1, 2, 65, True), (64, 2, 3, 300, True), (128, 2, 2, 257, False), (64, 1, 64, 333, True),
             (128, 2, 16, 2100, True), (64, 2, 16, 2100, False)]


@pytest.mark.parametrize("d,B,H,n,causal", BWD_TOKEN)
def test_bwd_token_major_equals_head_major(d, B, H, n, causal):
    """fox_attn_bwd_ex on [B,N,H,d] tensors ([B,N,H] lse / c / dlogf) gives the head-major
    gradients bit for bit: the same arithmetic with other addresses.  Below 1024 tokens the
    head-major gradients are also checked against the fp64 oracle (bound as in the parity test)."""
    cfg = fi.FwdConfig(f"bwd_tm_{d}_{B}_{H}_{n}_{causal}", B, H, n, d, "bf16", 2.0, 1.5)
    inp = fi.fwd_inputs(cfg)
    q, k, v, logf = (inp[x].to(DEV) for x in ("q", "k", "v", "logf"))
    g = torch.Generator().manual_seed(n * 7 + H)
    dout = torch.randn(B, H, n, d, generator=g).to(torch.bfloat16)
    o, lse, c = fox.attn_fwd_ex(q, k, v, logf, causal=causal, scale=inp["scale"])
    head = fox.attn_bwd(q, k, v, o, dout.to(DEV), lse, logf, causal=causal, scale=inp["scale"])
    tm = lambda t: t.permute(0, 2, 1, 3).contiguous()  # noqa: E731
    tv = lambda t: t.permute(0, 2, 1).contiguous()  # noqa: E731
    tok = fox.attn_bwd(tm(q), tm(k), tm(v), tm(o), tm(dout.to(DEV)), tv(lse), tv(logf), causal=causal,
                       scale=inp["scale"], layout="token")
    torch.cuda.synchronize()
    for name, h_, t_ in zip(("dq", "dk", "dv", "dlogf"), head, tok):
        back = t_.permute(0, 2, 1, 3) if t_.dim() == 4 else t_.permute(0, 2, 1)
        assert torch.equal(back, h_), name
    if n < 1024:
        ref = oracle.attn_bwd(_np(inp["q"]), _np(inp["k"]), _np(inp["v"]), _np(inp["logf"]), inp["scale"],
                              _np(dout), causal=causal)
        for name, got, r in zip(("dq", "dk", "dv", "dlogf"), head, ref):
            err = np.abs(_np(got) - r).max()
            assert err <= 2e-2 * max(1.0, np.abs(r).max()), (name, err)
    print(f"  {cfg.desc}: token-major == head-major", flush=True)


# (d, B, H, n, causal, gate-logit mean, sd): c1's shape in both modes, ragged n, edges; then small
# gates (logit means near 0: log f near -0.7, |c| in the hundreds to thousands) over long rows
BWD_F32 = [(32, 1, 2, 128, True, 2.0, 1.0), (32, 1, 2, 128, False, 2.0, 1.0), (64, 2, 3, 300, True, 2.0, 1.0),
           (128, 1, 2, 257, False, 2.0, 1.0), (64, 1, 1, 1, True, 2.0, 1.0), (32, 2, 2, 65, True, 2.0, 1.0),
           (128, 2, 2, 1000, True, 2.0, 1.0), (64, 1, 1, 63, False, 2.0, 1.0),
           (128, 1, 2, 1074, True, 0.86, 2.07), (128, 1, 2, 1862, True, 0.34, 1.47), (64, 1, 2, 4096, True, 0.2, 1.0),
           (32, 1, 2, 4096, False, 0.5, 2.0)]


@pytest.mark.parametrize("d,B,H,n,causal,mu,sigma", BWD_F32)
def test_bwd_f32_parity(d, B, H, n, causal, mu, sigma):
    """fp32 backward (fp32 forward's O and lse) against the fp64 oracle, and token-major equal to
    head-major bit for bit.  Bound: every score's bias is formed from fp64 gate sums (block starts)
    and an in-block part, so it carries rounding of the size of the bias, not of |c|; the fp32
    products, exponentials and sums then leave a relative error of a few 1e-6 (sums over thousands of
    terms of fp32 roundoff 6e-8).  Checked as max|gpu - ref| <= 2e-5 * max(1, max|ref|) per gradient
    tensor."""
    cfg = fi.FwdConfig(f"bwd32_{d}_{B}_{H}_{n}_{causal}_{mu}", B, H, n, d, "f32", mu, sigma)
    inp = fi.fwd_inputs(cfg)
    q, k, v, logf = (inp[x].to(DEV) for x in ("q", "k", "v", "logf"))
    g = torch.Generator().manual_seed(n * 13 + d)
    dout = torch.randn(B, H, n, d, generator=g)
    o, lse, c = fox.attn_fwd_ex(q, k, v, logf, causal=causal, scale=inp["scale"])
    head = fox.attn_bwd(q, k, v, o, dout.to(DEV), lse, logf, causal=causal, scale=inp["scale"])
    tm = lambda t: t.permute(0, 2, 1, 3).contiguous()  # noqa: E731
    tv = lambda t: t.permute(0, 2, 1).contiguous()  # noqa: E731
    tok = fox.attn_bwd(tm(q), tm(k), tm(v), tm(o), tm(dout.to(DEV)), tv(lse), tv(logf), causal=causal,
                       scale=inp["scale"], layout="token")
    torch.cuda.synchronize()
    for name, h_, t_ in zip(("dq", "dk", "dv", "dlogf"), head, tok):
        back = t_.permute(0, 2, 1, 3) if t_.dim() == 4 else t_.permute(0, 2, 1)
        assert torch.equal(back, h_), name
    ref = oracle.attn_bwd(_np(inp["q"]), _np(inp["k"]), _np(inp["v"]), _np(inp["logf"]), inp["scale"], _np(dout),
                          causal=causal)
    msg = []
    for name, got, r in zip(("dq", "dk", "dv", "dlogf"), head, ref):
        err = np.abs(_np(got) - r).max()
        msg.append(f"{name} {err:.2e} (max|ref| {np.abs(r).max():.2e})")
        assert torch.isfinite(got).all(), name
        assert err <= 2e-5 * max(1.0, np.abs(r).max()), (name, err)
    print("  " + cfg.desc + ": " + ", ".join(msg), flush=True)


# ------------------------------------------------------------------------- the largest sequence

MAX_SEQ = 1 << 22  # FOX_MAX_SEQ in include/fox.h


def test_max_seq_forward_backward_tail():
    """One head of FOX_MAX_SEQ = 4,194,304 tokens (d = 64, bf16; gate logits N(6,1): long windows,
    |c| near 10^4 at the end): the gate prefix sums at every position against the oracle, the last
    32 rows' O and lse and the last 32 positions' dq, dk, dv and dlogf against the oracle's tail
    computation (exact for the causal mask), every output finite.  Byte offsets inside one head
    reach 512 MB here."""
    n, d, T = MAX_SEQ, 64, 32
    cfg = fi.FwdConfig("maxseq", 1, 1, n, d, "bf16", 6.0, 1.0)
    inp = fi.fwd_inputs(cfg)
    g = torch.Generator().manual_seed(11)
    dout = torch.randn(1, 1, n, d, generator=g).to(torch.bfloat16)
    print(f"  {cfg.desc}: inputs ready", flush=True)
    q, k, v, logf = (inp[x].to(DEV) for x in ("q", "k", "v", "logf"))
    o, lse, c = fox.attn_fwd(q, k, v, logf, scale=inp["scale"])
    dq, dk, dv, dl = fox.attn_bwd(q, k, v, o, dout.to(DEV), lse, logf, scale=inp["scale"])
    torch.cuda.synchronize()
    print("  forward and backward done", flush=True)
    for name, t in (("o", o), ("lse", lse), ("c", c), ("dq", dq), ("dk", dk), ("dv", dv), ("dlogf", dl)):
        assert torch.isfinite(t).all(), name
    c_ref = oracle.logf_cumsum(_np(inp["logf"]))
    ec = np.abs(_np(c) - c_ref).max()
    assert ec <= _ulp(c_ref), ec
    ref = oracle.fwd_bwd_tail(_np(inp["q"][0, 0]), _np(inp["k"][0, 0]), _np(inp["v"][0, 0]), _np(inp["logf"][0, 0]),
                              inp["scale"], _np(dout[0, 0]), n - T)
    msg = [f"max|dc|={ec:.2e}"]
    for name, got, r in zip(("o", "lse", "dq", "dk", "dv", "dlogf"), (o, lse, dq, dk, dv, dl), ref):
        err = np.abs(_np(got[0, 0, n - T:]) - r).max()
        bound = TOL["bf16"] if name in ("o", "lse") else 2e-2 * max(1.0, np.abs(r).max())
        msg.append(f"{name} {err:.2e}")
        assert err <= bound, (name, err, bound)
    print("  last 32 positions: " + ", ".join(msg), flush=True)


def test_bwd_large_prefix_sums_tail():
    """One head of 2^20 tokens with gate logits N(3,1.5) (log f near -0.12 on average): |c| reaches
    about 1.2e5 at the end, where an fp32 c is only good to ~0.008, far coarser than the biases of
    nearby keys.  The backward builds its biases from fp64 block sums instead; the last 32
    positions' O, lse, dq, dk, dv and dlogf are checked against the oracle's tail computation."""
    n, d, T = 1 << 20, 64, 32
    cfg = fi.FwdConfig("bigc", 1, 1, n, d, "bf16", 3.0, 1.5)
    inp = fi.fwd_inputs(cfg)
    g = torch.Generator().manual_seed(13)
    dout = torch.randn(1, 1, n, d, generator=g).to(torch.bfloat16)
    print(f"  {cfg.desc}: inputs ready", flush=True)
    q, k, v, logf = (inp[x].to(DEV) for x in ("q", "k", "v", "logf"))
    o, lse, c = fox.attn_fwd(q, k, v, logf, scale=inp["scale"])
    dq, dk, dv, dl = fox.attn_bwd(q, k, v, o, dout.to(DEV), lse, logf, scale=inp["scale"])
    torch.cuda.synchronize()
    print(f"  forward and backward done; |c| at the end {abs(float(c[0, 0, -1])):.3e}", flush=True)
    for name, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv), ("dlogf", dl)):
        assert torch.isfinite(t).all(), name
    ref = oracle.fwd_bwd_tail(_np(inp["q"][0, 0]), _np(inp["k"][0, 0]), _np(inp["v"][0, 0]), _np(inp["logf"][0, 0]),
                              inp["scale"], _np(dout[0, 0]), n - T)
    msg = []
    for name, got, r in zip(("o", "lse", "dq", "dk", "dv", "dlogf"), (o, lse, dq, dk, dv, dl), ref):
        err = np.abs(_np(got[0, 0, n - T:]) - r).max()
        bound = TOL["bf16"] if name in ("o", "lse") else 2e-2 * max(1.0, np.abs(r).max())
        msg.append(f"{name} {err:.2e}")
        assert err <= bound, (name, err, bound)
    print("  last 32 positions: " + ", ".join(msg), flush=True)


def test_max_seq_decode():
    """Decode of the last token of a FOX_MAX_SEQ-slot cache (one sequence, one head, d = 128)."""
    cfg = fi.DecodeConfig("maxdec", 1, 1, MAX_SEQ, 128, "bf16", 6.0, 1.0)
    _check_decode(fi.decode_inputs(cfg), TOL["bf16"])


# ------------------------------------------------------------------------------ graph capture

def test_graph_replays_match_eager():
    """The entry points launch kernels only (no allocation, copy, memset or synchronisation), so a
    forward, backward and decode step captured in a HIP graph replay to the eager results; checked
    on several replays with eager work and synchronisations between them."""
    cfg = fi.FwdConfig("graph", 2, 3, 300, 64, "bf16", 2.0, 1.0)
    inp = fi.fwd_inputs(cfg)
    q, k, v, logf = (inp[x].to(DEV) for x in ("q", "k", "v", "logf"))
    g = torch.Generator().manual_seed(9)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16).to(DEV)
    dcfg = fi.DecodeConfig("graph_dec", 2, 3, 500, 64, "bf16", 4.0, 2.0)
    dinp = fi.decode_inputs(dcfg)
    qd, kd, vd = (dinp[x].to(DEV) for x in ("q", "k", "v"))
    c0 = fox.logf_cumsum(dinp["logf_all"].to(DEV))
    lnew = dinp["logf_all"][..., dcfg.L - 1].contiguous().to(DEV)
    # preallocated outputs and workspaces, shared by the eager run and the graph
    o, lse, c = torch.empty_like(q), torch.empty_like(logf), torch.empty_like(logf)
    dq, dk, dv, dl = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q), torch.empty_like(logf)
    wsb = torch.empty(fox.attn_bwd_workspace_bytes(2, 3, 300, 64), device=DEV, dtype=torch.uint8)
    od, lsed = torch.empty_like(qd), torch.empty(2, 3, device=DEV)
    wsd = torch.empty(fox.decode_workspace_bytes(2, 3, dcfg.L, 64), device=DEV, dtype=torch.uint8)
    cd = c0.clone()

    def run():
        fox.attn_fwd(q, k, v, logf, scale=inp["scale"], out=o, lse=lse, c=c)
        fox.attn_bwd(q, k, v, o, dout, lse, logf, scale=inp["scale"], dq=dq, dk=dk, dv=dv, dlogf=dl, workspace=wsb)
        fox.attn_decode(qd, kd, vd, cd, lnew, scale=dinp["scale"], out=od, lse=lsed, workspace=wsd)

    outs = (o, lse, c, dq, dk, dv, dl, od, lsed, cd)
    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        cd.copy_(c0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t, e in zip(("o", "lse", "c", "dq", "dk", "dv", "dlogf", "o_dec", "lse_dec", "c_cache"), outs, eager):
            assert torch.equal(t, e), (rep, name)
        x = (q.float() @ k.float().transpose(-1, -2)).sum()  # eager work between replays
        assert torch.isfinite(x)


def test_graph_replays_staged_backward():
    """fox_attn_bwd_staged launches kernels only as well: captured in a HIP graph, every replay
    (outputs and staged dS NaN-filled before it, eager work between replays) equals the eager call."""
    cfg = fi.FwdConfig("graph_staged", 1, 2, 300, 128, "bf16", 3.0, 1.5)
    inp = fi.fwd_inputs(cfg)
    q, k, v, logf = (inp[x].to(DEV) for x in ("q", "k", "v", "logf"))
    g = torch.Generator().manual_seed(19)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16).to(DEV)
    o, lse, _ = fox.attn_fwd(q, k, v, logf, scale=inp["scale"])
    dq, dk, dv, dl = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q), torch.empty_like(logf)
    ws = torch.empty(fox.attn_bwd_staged_workspace_bytes(1, 2, 300, 128), device=DEV, dtype=torch.uint8)

    def run():
        fox.attn_bwd_staged(q, k, v, o, dout, lse, logf, scale=inp["scale"], dq=dq, dk=dk, dv=dv, dlogf=dl,
                            workspace=ws)

    outs = (dq, dk, dv, dl)
    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t, e in zip(("dq", "dk", "dv", "dlogf"), outs, eager):
            assert torch.equal(t, e), (rep, name)
        x = (q.float() @ k.float().transpose(-1, -2)).sum()  # eager work between replays
        assert torch.isfinite(x)


# ------------------------------------------------------------------ binding: caller-supplied outputs

def test_binding_rejects_bad_outputs():
    """Outputs the caller supplies are checked before any launch: wrong shape, dtype, device layout
    (non-contiguous) or a CPU tensor raise ValueError."""
    inp = fi.fwd_inputs(fi.FwdConfig("outs", 1, 2, 64, 32, "bf16", 2.0, 1.0))
    q, k, v, logf = (inp[x].to(DEV) for x in ("q", "k", "v", "logf"))
    bad_o = [torch.empty(1, 2, 63, 32, device=DEV, dtype=torch.bfloat16),  # shape
             torch.empty(1, 2, 64, 32, device=DEV, dtype=torch.float32),  # dtype
             torch.empty(1, 2, 32, 64, device=DEV, dtype=torch.bfloat16).transpose(2, 3),  # strided
             torch.empty(1, 2, 64, 32, dtype=torch.bfloat16)]  # host memory
    for o in bad_o:
        with pytest.raises(ValueError):
            fox.attn_fwd(q, k, v, logf, out=o)
    for kw in ({"lse": torch.empty(1, 2, 64, device=DEV, dtype=torch.bfloat16)},
               {"c": torch.empty(2, 1, 64, device=DEV)}, {"lse": torch.empty(1, 2, 65, device=DEV)}):
        with pytest.raises(ValueError):
            fox.attn_fwd(q, k, v, logf, **kw)
        with pytest.raises(ValueError):
            fox.attn_fwd_noncausal(q, k, v, logf, **kw)
    o, lse, _ = fox.attn_fwd(q, k, v, logf)
    dout = torch.zeros_like(q)
    for kw in ({"dq": torch.empty(1, 2, 64, 32, device=DEV)}, {"dk": torch.empty(1, 2, 64, 16, device=DEV,
                                                                                  dtype=torch.bfloat16)},
               {"dlogf": torch.empty(1, 2, 64, device=DEV, dtype=torch.float64)}):
        with pytest.raises(ValueError):
            fox.attn_bwd(q, k, v, o, dout, lse, logf, **kw)
    dinp = fi.decode_inputs(fi.DecodeConfig("outs_dec", 2, 2, 100, 64, "bf16", 4.0, 2.0))
    qd, kd, vd = (dinp[x].to(DEV) for x in ("q", "k", "v"))
    cc = fox.logf_cumsum(dinp["logf_all"].to(DEV))
    ln = dinp["logf_all"][..., 99].contiguous().to(DEV)
    for kw in ({"out": torch.empty(2, 2, 32, device=DEV, dtype=torch.bfloat16)},
               {"lse": torch.empty(2, 3, device=DEV)}, {"lse": torch.empty(2, 2, device=DEV, dtype=torch.bfloat16)},
               {"workspace": torch.empty(4096, dtype=torch.uint8)}):
        with pytest.raises(ValueError):
            fox.attn_decode(qd, kd, vd, cc, ln, **kw)
    torch.cuda.synchronize()
