"""Pins of the fp64 backward oracle (CPU only).

The pages derive no backward pass: the oracle differentiates the forward definition by the chain
rule (oracle.fwd_bwd_head).  Its pins check that derivation against routes that do not use it:
finite differences of the pinned forward oracle, PyTorch autograd through the decay-product form
of the weights (foxwindow README, opening paragraph: content term times D_ij, the product of the
gates between key and query), PyTorch's own attention backward when the gates are 1, and the
invariance of the result to the first gate.  Planted mistakes in copies of the derivation must each
fail a pin.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import attn_bwd, fwd_bwd_head, fwd_bwd_tail, fwd_head_rows

TOL = 1e-11


def _logsigmoid(x):
    return -np.logaddexp(0.0, -x)


def _case(seed, n, d, mu=1.0, sigma=1.5):
    r = np.random.default_rng(seed)
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    logf = _logsigmoid(r.normal(mu, sigma, n))
    return q, k, v, logf, do


def _loss(q, k, v, logf, scale, do, causal):
    o, _ = fwd_head_rows(q, k, v, logf, scale, np.arange(q.shape[0]), causal=causal)
    return float((o * do).sum())


def bpin_finite_differences(bwd):
    """Directional derivatives of L = sum(dO * O), central differences of the forward oracle."""
    for causal in (True, False):
        for seed, (n, d) in enumerate([(7, 3), (12, 5)]):
            q, k, v, logf, do = _case(300 + seed, n, d)
            scale = 0.6
            grads = bwd(q, k, v, logf, scale, do, causal)
            r = np.random.default_rng(400 + seed)
            h = 1e-5
            for idx, x in enumerate((q, k, v, logf)):
                delta = r.standard_normal(x.shape)
                args_p = [q, k, v, logf]
                args_m = [q, k, v, logf]
                args_p[idx] = x + h * delta
                args_m[idx] = x - h * delta
                fd = (_loss(*args_p, scale, do, causal) - _loss(*args_m, scale, do, causal)) / (2 * h)
                an = float((grads[idx] * delta).sum())
                assert abs(fd - an) < 1e-7 * max(1.0, abs(fd)), (causal, idx, fd, an)


def _torch_grads(q, k, v, logf, scale, do, causal):
    """Autograd (fp64) through the weights written as content times decay (foxwindow README,
    opening paragraph): w_ij = exp(scale q_i.k_j) * D_ij with D_ij the product of the gates f_t,
    j < t <= i, and o_i = sum_j w_ij v_j / sum_j w_ij.  Unmasked, a key j > i takes the reciprocal
    product over i < t <= j (the same c_i - c_j).  D is built from an explicit indicator of which
    gates lie between each query and key, not from prefix sums."""
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)  # noqa: E731
    tq, tk, tv, tl = t(q), t(k), t(v), t(logf)
    n = q.shape[0]
    ii = torch.arange(n)[:, None, None]
    jj = torch.arange(n)[None, :, None]
    tt = torch.arange(n)[None, None, :]
    between = ((jj < tt) & (tt <= ii)).double() - ((ii < tt) & (tt <= jj)).double()  # [query, key, gate]
    log_decay = between @ tl
    logw = scale * (tq @ tk.T) + log_decay
    if causal:
        keep = torch.arange(n)[None, :] <= torch.arange(n)[:, None]
        logw = torch.where(keep, logw, torch.full_like(logw, float("-inf")))
    w = torch.exp(logw - logw.max(dim=1, keepdim=True).values.detach())
    o = (w @ tv) / w.sum(dim=1, keepdim=True)
    (o * torch.tensor(do)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(), tl.grad.numpy()


def bpin_autograd(bwd):
    for causal in (True, False):
        q, k, v, logf, do = _case(310, 40, 8)
        ref = _torch_grads(q, k, v, logf, 0.35, do, causal)
        got = bwd(q, k, v, logf, 0.35, do, causal)
        for a, b in zip(got, ref):
            assert np.abs(a - b).max() < TOL


def bpin_unit_gate_matches_library_attention(bwd):
    """log f = 0: dq, dk, dv equal the gradients of PyTorch's causal attention (math path, fp64)."""
    q, k, v, _, do = _case(320, 33, 6)
    scale = 6 ** -0.5
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
        o = torch.nn.functional.scaled_dot_product_attention(tq[None, None], tk[None, None], tv[None, None],
                                                             is_causal=True, scale=scale)[0, 0]
    (o * torch.tensor(do)).sum().backward()
    dq, dk, dv, dl = bwd(q, k, v, np.zeros(33), scale, do, True)
    for a, b in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.abs(a - b.numpy()).max() < TOL


def bpin_first_gate_irrelevant(bwd):
    """Only differences c_i - c_j enter the forward, so the loss does not depend on log f_0."""
    for causal in (True, False):
        q, k, v, logf, do = _case(330, 25, 4)
        dl = bwd(q, k, v, logf, 0.5, do, causal)[3]
        assert abs(dl[0]) < 1e-12 * max(1.0, np.abs(dl).max())


BPINS = [bpin_finite_differences, bpin_autograd, bpin_unit_gate_matches_library_attention, bpin_first_gate_irrelevant]


def _oracle_bwd(q, k, v, logf, scale, do, causal):
    return fwd_bwd_head(q, k, v, logf, scale, do, causal=causal)


@pytest.mark.parametrize("pin", BPINS, ids=[p.__name__ for p in BPINS])
def test_backward_oracle_pin(pin):
    pin(_oracle_bwd)


def test_batched_backward_matches_heads():
    r = np.random.default_rng(340)
    B, H, N, d = 2, 2, 17, 4
    q, k, v, do = (r.standard_normal((B, H, N, d)) for _ in range(4))
    logf = _logsigmoid(r.normal(2, 1, (B, H, N)))
    got = attn_bwd(q, k, v, logf, 0.5, do)
    for b in range(B):
        for h in range(H):
            ref = fwd_bwd_head(q[b, h], k[b, h], v[b, h], logf[b, h], 0.5, do[b, h])
            for a, x in zip(got, ref):
                assert np.array_equal(a[b, h], x)


@pytest.mark.parametrize("n,t0", [(1, 0), (9, 0), (9, 4), (40, 39), (40, 17), (64, 0), (64, 63)])
def test_tail_oracle_equals_full_head(n, t0):
    """fwd_bwd_tail (the last rows of a sequence too long for N x N matrices) against the pinned
    full-head forward and backward oracles, position by position."""
    q, k, v, logf, do = _case(400 + n + t0, n, 5)
    o, lse, dq, dk, dv, dl = fwd_bwd_tail(q, k, v, logf, 0.4, do, t0)
    fo, flse = fwd_head_rows(q, k, v, logf, 0.4, np.arange(n))
    fq, fk, fv, fl = fwd_bwd_head(q, k, v, logf, 0.4, do)
    for got, ref in ((o, fo[t0:]), (lse, flse[t0:]), (dq, fq[t0:]), (dk, fk[t0:]), (dv, fv[t0:]), (dl, fl[t0:])):
        assert got.shape == ref.shape
        assert np.abs(got - ref).max() <= TOL * max(1.0, np.abs(ref).max())


def _mutant(kind):
    def bwd(q, k, v, logf, scale, do, causal):
        c = np.cumsum(logf)
        n = q.shape[0]
        s = scale * (q @ k.T) + (c[:, None] - c[None, :])
        if causal:
            s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        dv = p @ do if kind == "dv_untransposed" else p.T @ do
        dp = do @ v.T
        ds = p * dp if kind == "jacobian_without_row_term" else p * (dp - (dp * p).sum(axis=1, keepdims=True))
        dq = ds @ k if kind == "dq_unscaled" else scale * (ds @ k)
        dk = scale * (ds @ q) if kind == "dk_untransposed" else scale * (ds.T @ q)
        dc = ds.sum(axis=1) - ds.sum(axis=0)
        if kind == "dc_sign":
            dc = -dc
        if kind == "dc_query_side_only":
            dc = ds.sum(axis=1)
        dl = np.cumsum(dc[::-1])[::-1]
        if kind == "dlogf_forward_scan":
            dl = np.cumsum(dc)
        if kind == "dlogf_exclusive_scan":
            dl = dl - dc
        return dq, dk, dv, dl
    return bwd


MUTANTS = ["dv_untransposed", "jacobian_without_row_term", "dq_unscaled", "dk_untransposed", "dc_sign",
           "dc_query_side_only", "dlogf_forward_scan", "dlogf_exclusive_scan"]


def test_reference_mutant_passes():
    for pin in BPINS:
        pin(_mutant("none"))


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    failed = []
    with np.errstate(all="ignore"):
        for pin in BPINS:
            try:
                pin(_mutant(kind))
            except (AssertionError, ValueError, IndexError):
                failed.append(pin.__name__)
    assert failed, f"mutant {kind} passed every backward pin"
