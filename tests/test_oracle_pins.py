"""Pins of the fp64 oracle against facts fixed outside the oracle itself (CPU only).

Each pin is a function of the forward routine under test, so the last test can
plant plausible mistakes in copies of the oracle and show that some pin fails
for every one of them.

Sources of the pinned facts:
* FoX module page (frankenstein-transformer docs), ``ForgettingAttention.forward``:
  bias = cum[i] - cum[j] of the log gates, added after the scaled product;
  decoder mode masks the strict upper triangle (diagonal kept); softmax over keys.
* foxwindow README, opening paragraph: score = q.k + sum_{t=j+1..i} log g_t;
  "The window is a first-passage time": decay strictly decreasing in distance;
  "ALiBi is the zero-variance limit": constant gate exp(-m) is ALiBi with slope m,
  window 138.2 (m = 0.05) and 69.1 (m = 0.1).
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attn_decode, attn_decode_paged, attn_decode_ragged, attn_fwd, brute_decode_head, brute_fwd_head, fwd_head_rows, logf_cumsum

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _logsigmoid(x):
    return -np.logaddexp(0.0, -x)


def _rand_head(seed, n, d, mu=2.0, sigma=1.0):
    r = _rng(seed)
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    logf = _logsigmoid(r.normal(mu, sigma, n))
    return q, k, v, logf


def _all_rows(fwd, q, k, v, logf, scale):
    return fwd(q, k, v, logf, scale, np.arange(q.shape[0]))


def _sdpa(q, k, v, scale, mask=None, causal=False):
    """Independent library route: PyTorch's CPU flash-attention kernel in fp64, returning (O, lse)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]  # noqa: E731
    o, lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        t(q), t(k), t(v), 0.0, causal, attn_mask=None if mask is None else torch.from_numpy(mask), scale=scale)
    return o[0, 0].numpy(), lse[0, 0].numpy()


# ----------------------------------------------------------------------------------------------
# pins, each parameterised by the forward routine (signature of oracle.fwd_head_rows)
# ----------------------------------------------------------------------------------------------

def pin_unit_gate_is_causal_softmax(fwd):
    """log f = 0 (f = 1): no bias, so FoX is plain causal softmax attention."""
    q, k, v, _ = _rand_head(1, 96, 16)
    logf = np.zeros(96)
    scale = 16 ** -0.5
    o, lse = _all_rows(fwd, q, k, v, logf, scale)
    o_ref, lse_ref = _sdpa(q, k, v, scale, causal=True)
    assert np.abs(o - o_ref).max() < TOL and np.abs(lse - lse_ref).max() < TOL


def pin_constant_gate_is_alibi(fwd):
    """log f = -m: bias -m (i - j), ALiBi with slope m (unscaled by the dot-product scale)."""
    n, d = 80, 8
    q, k, v, _ = _rand_head(2, n, d)
    scale = 0.37
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    for m in (0.05, 0.3):
        mask = np.where(j > i, -np.inf, -m * (i - j).astype(np.float64))
        o, lse = _all_rows(fwd, q, k, v, np.full(n, -m), scale)
        o_ref, lse_ref = _sdpa(q, k, v, scale, mask=mask)
        assert np.abs(o - o_ref).max() < TOL and np.abs(lse - lse_ref).max() < TOL


def pin_general_bias_by_indicator_sum(fwd):
    """Random gates: bias built as sum_t [j < t <= i] log f_t (an explicit 3-index indicator, no prefix sums)."""
    n, d = 48, 12
    q, k, v, logf = _rand_head(3, n, d, mu=0.5, sigma=1.5)
    scale = d ** -0.5
    t = np.arange(n)
    ind = (t[None, None, :] > t[None, :, None]) & (t[None, None, :] <= t[:, None, None])  # [i, j, t]
    bias = np.where(t[None, :] > t[:, None], -np.inf, ind.astype(np.float64) @ logf)
    o, lse = _all_rows(fwd, q, k, v, logf, scale)
    o_ref, lse_ref = _sdpa(q, k, v, scale, mask=bias)
    assert np.abs(o - o_ref).max() < TOL and np.abs(lse - lse_ref).max() < TOL


def pin_row0_attends_to_itself(fwd):
    """Diagonal kept, D_00 = 0: O_0 = V_0 and lse_0 = scale q_0 . k_0 whatever the gates."""
    q, k, v, logf = _rand_head(4, 20, 8, mu=-1.0)
    scale = 0.5
    o, lse = fwd(q, k, v, logf, scale, np.array([0]))
    assert np.abs(o[0] - v[0]).max() < TOL
    assert abs(lse[0] - scale * float(q[0] @ k[0])) < TOL


def pin_rows_normalised(fwd):
    """Softmax rows sum to 1: with every value vector equal to 1 the output is exactly 1."""
    q, k, _, logf = _rand_head(5, 64, 8)
    v = np.ones((64, 3))
    o, _ = _all_rows(fwd, q, k, v, logf, 0.9)
    assert np.abs(o - 1.0).max() < TOL


def pin_zero_query_recurrence(fwd):
    """q = 0: weights are prod_{t=j+1..i} f_t, so O_i = S_i / Z_i with S_i = f_i S_{i-1} + v_i,
    Z_i = f_i Z_{i-1} + 1 and lse_i = ln Z_i (an O(N) route with no softmax)."""
    n, d = 120, 5
    _, k, v, logf = _rand_head(6, n, d, mu=1.0, sigma=2.0)
    q = np.zeros((n, d))
    f = np.exp(logf)
    S = np.zeros(d)
    Z = 0.0
    o_ref = np.empty((n, d))
    lse_ref = np.empty(n)
    for i in range(n):
        S = f[i] * S + v[i]
        Z = f[i] * Z + 1.0
        o_ref[i], lse_ref[i] = S / Z, math.log(Z)
    o, lse = _all_rows(fwd, q, k, v, logf, 1.0)
    assert np.abs(o - o_ref).max() < 1e-11 and np.abs(lse - lse_ref).max() < 1e-11


def pin_gate_spike(fwd):
    """One tiny gate at j*: keys before j* are cut off, key j* itself is not
    (bias runs over t = j+1..i), so O_i = mean(V_{j*..i}) for i >= j*."""
    n, d, js = 40, 4, 17
    _, k, v, _ = _rand_head(7, n, d)
    logf = np.zeros(n)
    logf[js] = -60.0
    o, _ = _all_rows(fwd, np.zeros((n, d)), k, v, logf, 1.0)
    for i in range(js, n):
        assert np.abs(o[i] - v[js:i + 1].mean(axis=0)).max() < 1e-12
    for i in range(js):
        assert np.abs(o[i] - v[: i + 1].mean(axis=0)).max() < 1e-12


def pin_alibi_window(fwd):
    """foxwindow README, 'ALiBi is the zero-variance limit': with q = 0 and gate exp(-m) the number of
    keys whose weight is >= eps times the diagonal weight is floor(ln(1/eps)/m) + 1."""
    with open(os.path.join(GOLDEN, "alibi_window.json")) as fh:
        gold = json.load(fh)
    eps = gold["eps"]
    for case in gold["cases"]:
        m = case["m"]
        assert round(math.log(1 / eps) / m, 1) == case["printed_L_over_m"]
        n = case["exact_count"] + 40
        v = np.eye(n)  # O_i is then row i of the weight matrix
        rows = np.arange(case["exact_count"], n)
        o, _ = fwd(np.zeros((n, 1)), np.zeros((n, 1)), v, np.full(n, np.float64(np.float32(-m))), 1.0, rows)
        for r, i in enumerate(rows):
            w = o[r]
            assert int((w >= eps * w[i]).sum()) == case["exact_count"]


def pin_gate_origin_irrelevant(fwd):
    """Only differences c_i - c_j enter: log f_0 never matters."""
    q, k, v, logf = _rand_head(8, 50, 6)
    o1, l1 = _all_rows(fwd, q, k, v, logf, 0.4)
    logf2 = logf.copy()
    logf2[0] = -7.5
    o2, l2 = _all_rows(fwd, q, k, v, logf2, 0.4)
    assert np.abs(o1 - o2).max() < 1e-13 and np.abs(l1 - l2).max() < 1e-13


def pin_brute_force(fwd):
    """Scalar enumeration (bias summed directly over t = j+1..i) on N <= 8."""
    for seed, (n, d) in enumerate([(1, 1), (2, 3), (5, 4), (8, 8), (7, 2)]):
        q, k, v, logf = _rand_head(100 + seed, n, d, mu=0.3, sigma=2.0)
        scale = d ** -0.5
        o_b, l_b = brute_fwd_head(q.tolist(), k.tolist(), v.tolist(), logf.tolist(), scale)
        o, lse = _all_rows(fwd, q, k, v, logf, scale)
        assert np.abs(o - np.array(o_b)).max() < TOL and np.abs(lse - np.array(l_b)).max() < TOL


PINS = [
    pin_unit_gate_is_causal_softmax,
    pin_constant_gate_is_alibi,
    pin_general_bias_by_indicator_sum,
    pin_row0_attends_to_itself,
    pin_rows_normalised,
    pin_zero_query_recurrence,
    pin_gate_spike,
    pin_alibi_window,
    pin_gate_origin_irrelevant,
    pin_brute_force,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(fwd_head_rows)


# ----------------------------------------------------------------------------------------------
# gate scan, batched wrapper, decode
# ----------------------------------------------------------------------------------------------

def test_cumsum_against_running_fsum_and_monotone():
    logf = _logsigmoid(_rng(9).normal(2.0, 1.0, (3, 200)))
    c = logf_cumsum(logf)
    for r in range(3):
        for i in (0, 1, 57, 199):
            assert abs(c[r, i] - math.fsum(logf[r, : i + 1])) < 1e-12
        # foxwindow README: every log g < 0, so c_i - c_j is strictly increasing in j (decreasing in distance)
        i = 150
        bias = c[r, i] - c[r, : i + 1]
        assert np.all(np.diff(bias) > 0)


def test_batched_wrapper_matches_heads_and_permutes():
    r = _rng(10)
    B, H, N, d = 2, 3, 33, 4
    q, k, v = (r.standard_normal((B, H, N, d)) for _ in range(3))
    logf = _logsigmoid(r.normal(2, 1, (B, H, N)))
    o, lse, c = attn_fwd(q, k, v, logf, 0.5)
    for b in range(B):
        for h in range(H):
            oh, lh = fwd_head_rows(q[b, h], k[b, h], v[b, h], logf[b, h], 0.5, np.arange(N))
            assert np.array_equal(oh, o[b, h]) and np.array_equal(lh, lse[b, h])
    perm = [2, 0, 1]
    o2, l2, _ = attn_fwd(q[:, perm], k[:, perm], v[:, perm], logf[:, perm], 0.5)
    assert np.array_equal(o2, o[:, perm]) and np.array_equal(l2, lse[:, perm])
    assert np.abs(c - np.cumsum(logf, -1)).max() == 0.0


def _decode_case(seed, S, H, L, d):
    r = _rng(seed)
    q = r.standard_normal((S, H, d))
    kc, vc = r.standard_normal((S, H, L, d)), r.standard_normal((S, H, L, d))
    logf_all = _logsigmoid(r.normal(2, 1.5, (S, H, L)))
    cc = np.cumsum(logf_all, -1)
    cc[..., L - 1] = np.nan  # the slot the decode step computes
    return q, kc, vc, logf_all, cc


@pytest.mark.parametrize("L", [1, 2, 7])
def test_decode_matches_brute_force(L):
    S, H, d = 2, 2, 3
    q, kc, vc, logf_all, cc = _decode_case(11 + L, S, H, L, d)
    scale = 0.6
    o, lse, c_new = attn_decode(q, kc, vc, cc, logf_all[..., L - 1], scale)
    for s in range(S):
        for h in range(H):
            ob, lb = brute_decode_head(q[s, h].tolist(), kc[s, h].tolist(), vc[s, h].tolist(),
                                       logf_all[s, h].tolist(), scale)
            assert np.abs(o[s, h] - np.array(ob)).max() < TOL and abs(lse[s, h] - lb) < TOL
            assert abs(c_new[s, h] - math.fsum(logf_all[s, h])) < 1e-12


def test_ragged_decode_matches_brute_force():
    """Per-sequence cache lengths: each sequence against the scalar enumeration of its own slots."""
    S, H, L, d = 4, 2, 9, 3
    q, kc, vc, logf_all, _ = _decode_case(30, S, H, L, d)
    lens = [1, 9, 4, 2]
    cc = np.cumsum(logf_all, -1)
    ln = np.empty((S, H))
    for s, Ls in enumerate(lens):
        ln[s] = logf_all[s, :, Ls - 1]
        cc[s, :, Ls - 1:] = np.nan  # the slot the step computes, and the unused tail
    o, lse, c_new = attn_decode_ragged(q, kc, vc, cc, ln, lens, 0.45)
    for s, Ls in enumerate(lens):
        for h in range(H):
            ob, lb = brute_decode_head(q[s, h].tolist(), kc[s, h, :Ls].tolist(), vc[s, h, :Ls].tolist(),
                                       logf_all[s, h, :Ls].tolist(), 0.45)
            assert np.abs(o[s, h] - np.array(ob)).max() < TOL and abs(lse[s, h] - lb) < TOL
            assert abs(c_new[s, h] - math.fsum(logf_all[s, h, :Ls])) < 1e-12


def test_paged_decode_matches_brute_force():
    """Paged caches: sequences of several lengths scattered over shuffled pages of 4 slots (the
    last page partly used, unused pages and slots NaN), each against the scalar enumeration of its
    own tokens."""
    S, H, L, d, P = 4, 2, 11, 3, 4
    q, kc, vc, logf_all, _ = _decode_case(31, S, H, L, d)
    lens = [1, 11, 5, 8]
    maxp = (L + P - 1) // P
    rng = np.random.default_rng(7)
    npages = S * maxp + 3
    perm = rng.permutation(npages)
    table = perm[: S * maxp].reshape(S, maxp)
    kp = np.full((npages, H, P, d), np.nan)
    vp = np.full((npages, H, P, d), np.nan)
    cp = np.full((npages, H, P), np.nan)
    cc = np.cumsum(logf_all, -1)
    ln = np.empty((S, H))
    for s, Ls in enumerate(lens):
        ln[s] = logf_all[s, :, Ls - 1]
        for j in range(Ls):
            pg, r = table[s, j // P], j % P
            kp[pg, :, r], vp[pg, :, r] = kc[s, :, j], vc[s, :, j]
            cp[pg, :, r] = cc[s, :, j] if j < Ls - 1 else np.nan  # the slot the step computes
    o, lse, c_new = attn_decode_paged(q, kp, vp, cp, table, lens, ln, 0.45)
    for s, Ls in enumerate(lens):
        for h in range(H):
            ob, lb = brute_decode_head(q[s, h].tolist(), kc[s, h, :Ls].tolist(), vc[s, h, :Ls].tolist(),
                                       logf_all[s, h, :Ls].tolist(), 0.45)
            assert np.abs(o[s, h] - np.array(ob)).max() < TOL and abs(lse[s, h] - lb) < TOL
            assert abs(c_new[s, h] - math.fsum(logf_all[s, h, :Ls])) < 1e-12


def test_decode_is_last_row_of_forward():
    S, H, L, d = 2, 3, 64, 8
    q, kc, vc, logf_all, cc = _decode_case(20, S, H, L, d)
    qs = kc.copy()
    qs[..., L - 1, :] = q  # the decode query sits at position L-1
    o_f, l_f, _ = attn_fwd(qs, kc, vc, logf_all, 0.3)
    o_d, l_d, _ = attn_decode(q, kc, vc, cc, logf_all[..., L - 1], 0.3)
    assert np.abs(o_d - o_f[..., L - 1, :]).max() < 1e-13 and np.abs(l_d - l_f[..., L - 1]).max() < 1e-13


# ----------------------------------------------------------------------------------------------
# planted mistakes: every plausible slip in the oracle must fail at least one pin
# ----------------------------------------------------------------------------------------------

def _mutant(kind):
    def fwd(q, k, v, logf, scale, rows):
        q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
        logf = np.asarray(logf, np.float64)
        c = np.cumsum(logf)
        if kind == "exclusive_scan":
            c = c - logf
        n = q.shape[0]
        rows = np.asarray(rows)
        keys = np.arange(n)
        qq, kk = (k, q) if kind == "swap_qk" else (q, k)
        bias = c[rows][:, None] - c[None, :]
        if kind == "bias_sign":
            bias = -bias
        if kind == "docstring_index":  # sum over t = j..i instead of j+1..i
            bias = bias + logf[None, :]
        if kind == "scaled_bias":
            s = scale * (qq[rows] @ kk.T + bias)
        else:
            s = scale * (qq[rows] @ kk.T) + bias
        if kind == "drop_bias":
            s = scale * (qq[rows] @ kk.T)
        cut = keys[None, :] >= rows[:, None] if kind == "mask_diagonal" else keys[None, :] > rows[:, None]
        if kind == "no_mask":
            cut = np.zeros_like(cut)
        s = np.where(cut, -np.inf, s)
        m = s.max(1)
        lse = m + np.log(np.exp(s - m[:, None]).sum(1))
        if kind == "lse_base2":
            lse = lse / math.log(2)
            p = np.exp((s - m[:, None])) / np.exp(s - m[:, None]).sum(1)[:, None]
        else:
            p = np.exp(s - lse[:, None])
        vv = v[::-1] if kind == "reversed_values" else v
        return p @ vv, lse
    return fwd


MUTANTS = ["exclusive_scan", "swap_qk", "bias_sign", "docstring_index", "scaled_bias", "drop_bias",
           "mask_diagonal", "no_mask", "lse_base2", "reversed_values"]


def test_reference_mutant_passes():
    # the mutant harness with no mutation is the oracle's definition and must pass every pin
    for pin in PINS:
        pin(_mutant("none"))


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    failed = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(_mutant(kind))
            except (AssertionError, ValueError, IndexError):
                failed.append(pin.__name__)
    assert failed, f"mutant {kind} passed every pin"


# ----------------------------------------------------------------------------------------------
# unmasked (default, non-decoder) mode: every key enters, bias c_i - c_j for all pairs
# ----------------------------------------------------------------------------------------------
# FoX module page, ForgettingAttention.forward: the triangle mask belongs to decoder mode only;
# without it the same scaled q k^T + (cum[i] - cum[j]) is softmaxed over all keys.

def _nc(fwd):
    """The routine under test in unmasked mode, with the fwd_head_rows signature."""
    return lambda q, k, v, logf, scale, rows: fwd(q, k, v, logf, scale, rows, causal=False)


def npin_unit_gate_is_softmax(fwd):
    """log f = 0: no bias and no mask, plain softmax attention."""
    q, k, v, _ = _rand_head(31, 96, 16)
    scale = 16 ** -0.5
    o, lse = _all_rows(fwd, q, k, v, np.zeros(96), scale)
    o_ref, lse_ref = _sdpa(q, k, v, scale, causal=False)
    assert np.abs(o - o_ref).max() < TOL and np.abs(lse - lse_ref).max() < TOL


def npin_constant_gate_is_two_sided_slope(fwd):
    """log f = -m: bias -m (i - j) for every pair, +m per step for keys after the query."""
    n, d = 72, 8
    q, k, v, _ = _rand_head(32, n, d)
    scale = 0.37
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    for m in (0.05, 0.3):
        o, lse = _all_rows(fwd, q, k, v, np.full(n, -m), scale)
        o_ref, lse_ref = _sdpa(q, k, v, scale, mask=-m * (i - j).astype(np.float64))
        assert np.abs(o - o_ref).max() < TOL and np.abs(lse - lse_ref).max() < TOL


def npin_general_bias_by_signed_indicator_sum(fwd):
    """Random gates: bias_ij = sum_t ([j < t <= i] - [i < t <= j]) log f_t, no prefix sums."""
    n, d = 40, 12
    q, k, v, logf = _rand_head(33, n, d, mu=0.5, sigma=1.5)
    scale = d ** -0.5
    t = np.arange(n)
    fwd_ind = (t[None, None, :] > t[None, :, None]) & (t[None, None, :] <= t[:, None, None])  # j < t <= i
    bwd_ind = (t[None, None, :] > t[:, None, None]) & (t[None, None, :] <= t[None, :, None])  # i < t <= j
    bias = (fwd_ind.astype(np.float64) - bwd_ind.astype(np.float64)) @ logf
    o, lse = _all_rows(fwd, q, k, v, logf, scale)
    o_ref, lse_ref = _sdpa(q, k, v, scale, mask=bias)
    assert np.abs(o - o_ref).max() < TOL and np.abs(lse - lse_ref).max() < TOL


def npin_zero_query_closed_form(fwd):
    """q = 0: the bias c_i - c_j is rank one, so every row has the same weights, proportional to
    exp(-c_j): O_i = sum_j e^{-c_j} v_j / sum_j e^{-c_j} and lse_i = c_i + ln sum_j e^{-c_j}."""
    n, d = 64, 5
    _, k, v, logf = _rand_head(34, n, d, mu=1.0, sigma=2.0)
    c = np.array([math.fsum(logf[: i + 1]) for i in range(n)])
    w = np.exp(-(c - c.max()))  # shifted for range; the shift cancels in the ratio
    o_ref = (w[:, None] * v).sum(0) / w.sum()
    lse_ref = c - c.max() + math.log(math.fsum(w))
    o, lse = _all_rows(fwd, np.zeros((n, d)), k, v, logf, 1.0)
    assert np.abs(o - o_ref[None, :]).max() < 1e-11 and np.abs(lse - lse_ref).max() < 1e-11


def npin_rows_normalised(fwd):
    q, k, _, logf = _rand_head(35, 50, 8)
    o, _ = _all_rows(fwd, q, k, np.ones((50, 3)), logf, 0.9)
    assert np.abs(o - 1.0).max() < TOL


def npin_gate_origin_irrelevant(fwd):
    q, k, v, logf = _rand_head(36, 45, 6)
    o1, l1 = _all_rows(fwd, q, k, v, logf, 0.4)
    logf2 = logf.copy()
    logf2[0] = -7.5
    o2, l2 = _all_rows(fwd, q, k, v, logf2, 0.4)
    assert np.abs(o1 - o2).max() < 1e-13 and np.abs(l1 - l2).max() < 1e-13


def npin_brute_force(fwd):
    """Scalar enumeration over every key, biases summed directly in both directions, N <= 8."""
    for seed, (n, d) in enumerate([(1, 1), (2, 3), (5, 4), (8, 8), (7, 2)]):
        q, k, v, logf = _rand_head(200 + seed, n, d, mu=0.3, sigma=2.0)
        scale = d ** -0.5
        o_b, l_b = brute_fwd_head(q.tolist(), k.tolist(), v.tolist(), logf.tolist(), scale, causal=False)
        o, lse = _all_rows(fwd, q, k, v, logf, scale)
        assert np.abs(o - np.array(o_b)).max() < TOL and np.abs(lse - np.array(l_b)).max() < TOL


NPINS = [
    npin_unit_gate_is_softmax,
    npin_constant_gate_is_two_sided_slope,
    npin_general_bias_by_signed_indicator_sum,
    npin_zero_query_closed_form,
    npin_rows_normalised,
    npin_gate_origin_irrelevant,
    npin_brute_force,
]


@pytest.mark.parametrize("pin", NPINS, ids=[p.__name__ for p in NPINS])
def test_oracle_pin_unmasked(pin):
    pin(_nc(fwd_head_rows))


def test_unmasked_wrapper_matches_heads():
    r = _rng(37)
    B, H, N, d = 2, 2, 19, 4
    q, k, v = (r.standard_normal((B, H, N, d)) for _ in range(3))
    logf = _logsigmoid(r.normal(2, 1, (B, H, N)))
    o, lse, _ = attn_fwd(q, k, v, logf, 0.5, causal=False)
    for b in range(B):
        for h in range(H):
            oh, lh = fwd_head_rows(q[b, h], k[b, h], v[b, h], logf[b, h], 0.5, np.arange(N), causal=False)
            assert np.array_equal(oh, o[b, h]) and np.array_equal(lh, lse[b, h])
    # the last row sees every key in both modes
    oc, lc, _ = attn_fwd(q, k, v, logf, 0.5)
    assert np.abs(oc[:, :, -1] - o[:, :, -1]).max() < 1e-13 and np.abs(lc[:, :, -1] - lse[:, :, -1]).max() < 1e-13


def _mutant_unmasked(kind):
    def fwd(q, k, v, logf, scale, rows):
        q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
        logf = np.asarray(logf, np.float64)
        c = np.cumsum(logf)
        if kind == "exclusive_scan":
            c = c - logf
        n = q.shape[0]
        rows = np.asarray(rows)
        keys = np.arange(n)
        qq, kk = (k, q) if kind == "swap_qk" else (q, k)
        bias = c[rows][:, None] - c[None, :]
        if kind == "bias_sign":
            bias = -bias
        if kind == "future_bias_dropped":  # bias applied below the diagonal only
            bias = np.where(keys[None, :] > rows[:, None], 0.0, bias)
        if kind == "future_bias_mirrored":  # |i - j| distance decay in both directions
            bias = np.where(keys[None, :] > rows[:, None], -bias, bias)
        s = scale * (qq[rows] @ kk.T + bias) if kind == "scaled_bias" else scale * (qq[rows] @ kk.T) + bias
        if kind == "drop_bias":
            s = scale * (qq[rows] @ kk.T)
        if kind == "causal_mask":
            s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
        m = s.max(1)
        lse = m + np.log(np.exp(s - m[:, None]).sum(1))
        if kind == "lse_base2":
            lse = lse / math.log(2)
            p = np.exp((s - m[:, None])) / np.exp(s - m[:, None]).sum(1)[:, None]
        else:
            p = np.exp(s - lse[:, None])
        vv = v[::-1] if kind == "reversed_values" else v
        return p @ vv, lse
    return fwd


MUTANTS_UNMASKED = ["exclusive_scan", "swap_qk", "bias_sign", "future_bias_dropped", "future_bias_mirrored",
                    "scaled_bias", "drop_bias", "causal_mask", "lse_base2", "reversed_values"]


def test_unmasked_reference_mutant_passes():
    for pin in NPINS:
        pin(_mutant_unmasked("none"))


@pytest.mark.parametrize("kind", MUTANTS_UNMASKED)
def test_unmasked_planted_mistake_is_caught(kind):
    failed = []
    with np.errstate(all="ignore"):
        for pin in NPINS:
            try:
                pin(_mutant_unmasked(kind))
            except (AssertionError, ValueError, IndexError):
                failed.append(pin.__name__)
    assert failed, f"mutant {kind} passed every unmasked-mode pin"
