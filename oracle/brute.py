"""Scalar brute-force enumeration of FoX attention for tiny inputs.

TEST INFRASTRUCTURE (same rule as the rest of ``oracle/``).

This is a second, deliberately different route to the same definition, used
to pin the vectorised oracle on N <= 8: pure-Python loops, ``math.fsum`` for
every sum, and the bias taken directly as the sum of ``log f_t`` over
t = j+1 .. i (foxwindow README, opening paragraph) instead of as a difference
of prefix sums.  No numpy arithmetic is used.
"""

from __future__ import annotations

import math


def brute_fwd_head(q, k, v, logf, scale, causal=True):
    """q, k, v: lists [N][d] of floats; logf: list [N]. Returns (O [N][d], lse [N]).

    causal=False (the module's unmasked mode) enumerates every key; a key after the
    query gets the bias -(sum of log f_t over t = i+1 .. j), summed directly.
    """
    n = len(q)
    d = len(v[0]) if n else 0
    out, lse = [], []
    for i in range(n):
        keys = range(i + 1) if causal else range(n)
        logits = []
        for j in keys:
            dot = math.fsum(q[i][e] * k[j][e] for e in range(len(q[i])))
            if j <= i:
                bias = math.fsum(logf[t] for t in range(j + 1, i + 1))
            else:
                bias = -math.fsum(logf[t] for t in range(i + 1, j + 1))
            logits.append(scale * dot + bias)
        top = max(logits)
        z = math.fsum(math.exp(s - top) for s in logits)
        row_lse = top + math.log(z)
        w = [math.exp(s - row_lse) for s in logits]
        out.append([math.fsum(w[a] * v[j][e] for a, j in enumerate(keys)) for e in range(d)])
        lse.append(row_lse)
    return out, lse


def brute_decode_head(q, k_cache, v_cache, logf_all, scale):
    """Decode for one (sequence, head) where the whole gate history is known.

    q: [d]; k_cache, v_cache: [L][d]; logf_all: [L] (logf_all[L-1] is the new
    token's gate).  The last row of ``brute_fwd_head`` is the decode result;
    the bias is again the direct sum over t = j+1 .. L-1.
    """
    L = len(k_cache)
    i = L - 1
    logits = []
    for j in range(L):
        dot = math.fsum(q[e] * k_cache[j][e] for e in range(len(q)))
        bias = math.fsum(logf_all[t] for t in range(j + 1, i + 1))
        logits.append(scale * dot + bias)
    top = max(logits)
    z = math.fsum(math.exp(s - top) for s in logits)
    row_lse = top + math.log(z)
    w = [math.exp(s - row_lse) for s in logits]
    out = [math.fsum(w[j] * v_cache[j][e] for j in range(L)) for e in range(len(v_cache[0]))]
    return out, row_lse
