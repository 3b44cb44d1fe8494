"""Plain fp64 CPU oracle for Forgetting-Transformer (FoX) attention.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this module. The product path (the HIP
library and its Python binding) never calls it, and this module imports
nothing from the product.

What is computed (the plain definition, written out; no tiling, no online
softmax, no split-K):

* Gate scan -- ``c_i = sum_{t<=i} log f_t`` along the sequence, per (batch,
  head).  Source: "Forgetting Transformer (FoX) Attention" module page
  (frankenstein-transformer docs), ``ForgettingAttention.forward``: the
  cumulative sum of the log forget gates over the sequence axis.
* Scores -- for key j <= query i,
  ``s_ij = scale * q_i . k_j + (c_i - c_j)``, i.e. the bias is the sum of
  ``log f_t`` for t = j+1 .. i and is *not* multiplied by ``scale``.
  Sources: the same ``forward`` (bias ``cum[i] - cum[j]`` added after the
  scaled product, scale = head_dim ** -0.5) and the "foxwindow" README,
  opening paragraph (score = q_i . k_j + sum over t = j+1..i of log g_t).
  Keys j > i get weight exactly 0: decoder-mode causal mask, which masks the
  strict upper triangle and keeps the diagonal.
* Softmax over keys and the weighted sum of values -- same ``forward``.
  ``lse_i`` is the natural-log log-sum-exp of the full logits row (scale and
  bias included); the pages do not define it, this is the plainest reading.
* Unmasked mode -- the module's default (not decoder) mode applies no mask: every
  key j = 0 .. N-1 enters the softmax with the same bias ``c_i - c_j``, which for a
  key after the query equals ``-(sum_{t=i+1..j} log f_t)`` (>= 0).  Source: the same
  ``forward``, whose triangle mask is applied in decoder mode only.
* Backward -- gradients of a loss through O with respect to q, k, v and the log
  gates, by the chain rule through the definition (``fwd_bwd_head``).
* Decode -- the single query row i = L-1 of a sequence whose key/value cache
  holds slots 0..L-1 (the new token's k, v already at slot L-1) and whose
  cached prefix sums hold slots 0..L-2; the new prefix sum is
  ``c_{L-1} = c_{L-2} + log f_new`` (``c_0 = log f_new`` when L = 1).
  The pages define no decode; this reading follows the attention definition
  above applied to the last row.

Every function takes and returns float64 numpy arrays; callers pass the exact
values the GPU sees (bf16 inputs widened exactly, fp32 gates widened, the
fp32 ``scale`` widened).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "logf_cumsum",
    "fwd_head_rows",
    "attn_fwd",
    "attn_fwd_rows",
    "attn_decode",
    "attn_decode_ragged",
    "fwd_bwd_head",
    "attn_bwd",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def logf_cumsum(logf) -> np.ndarray:
    """Inclusive prefix sum of the log forget gates along the last axis.

    FoX module page, ``ForgettingAttention.forward``: cumulative sum of
    ``log f`` over the sequence dimension.  ``c_i = sum_{t=0}^{i} logf_t``.
    """
    return np.cumsum(_f64(logf), axis=-1)


def fwd_head_rows(q, k, v, logf, scale, rows, chunk: int = 256, causal: bool = True):
    """Definition of FoX attention for one head, for selected rows.

    q, k, v: [N, d]; logf: [N]; rows: 1-D integer array of query indices.
    Returns (O[rows] [len(rows), d], lse[rows] [len(rows)]).

    FoX module page, ``ForgettingAttention.forward``:
    logits = scale * q k^T + (c_i - c_j); in decoder mode (``causal``) the
    strict upper triangle is set to -inf, in the default mode nothing is
    masked; softmax over keys, times v.  ``lse`` is log sum_j exp(logit_ij).
    Each row is computed from the definition independently; ``chunk`` only
    bounds how many rows are held in memory at once.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    c = logf_cumsum(logf)
    rows = np.asarray(rows, dtype=np.int64)
    n = q.shape[0]
    keys = np.arange(n)
    out = np.empty((rows.size, v.shape[1]), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    for lo in range(0, rows.size, chunk):
        r = rows[lo:lo + chunk]
        # causal: logits over keys 0..kmax-1 (keys beyond every selected row are masked anyway)
        kmax = (int(r.max()) + 1 if r.size else 0) if causal else n
        s = scale * (q[r] @ k[:kmax].T) + (c[r][:, None] - c[None, :kmax])
        if causal:
            s = np.where(keys[None, :kmax] > r[:, None], -np.inf, s)
        m = s.max(axis=1)
        z = np.exp(s - m[:, None]).sum(axis=1)
        row_lse = m + np.log(z)
        p = np.exp(s - row_lse[:, None])
        out[lo:lo + chunk] = p @ v[:kmax]
        lse[lo:lo + chunk] = row_lse
    return out, lse


def attn_fwd_rows(q, k, v, logf, scale, rows, causal: bool = True):
    """Rows ``rows`` of every (batch, head): q,k,v [B,H,N,d], logf [B,H,N].

    Returns (O [B,H,len(rows),d], lse [B,H,len(rows)]).
    """
    q = _f64(q)
    bsz, nh, _, d = q.shape
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((bsz, nh, rows.size, d), dtype=np.float64)
    lse = np.empty((bsz, nh, rows.size), dtype=np.float64)
    for b in range(bsz):
        for h in range(nh):
            out[b, h], lse[b, h] = fwd_head_rows(q[b, h], k[b, h], v[b, h], logf[b, h], scale, rows,
                                                 causal=causal)
    return out, lse


def attn_fwd(q, k, v, logf, scale, causal: bool = True):
    """Full FoX attention (causal, or unmasked with causal=False): q,k,v [B,H,N,d], logf [B,H,N].

    Returns (O [B,H,N,d], lse [B,H,N], c [B,H,N]) in float64.
    """
    n = np.asarray(q).shape[2]
    out, lse = attn_fwd_rows(q, k, v, logf, scale, np.arange(n), causal=causal)
    return out, lse, logf_cumsum(logf)


def attn_decode(q, k_cache, v_cache, c_cache, logf_new, scale):
    """One decode step of causal FoX attention against a cache.

    q: [S,H,d]; k_cache, v_cache: [S,H,L,d] with the new token at slot L-1;
    c_cache: [S,H,L] whose slots 0..L-2 hold the cached prefix sums (slot L-1
    is ignored); logf_new: [S,H].
    Returns (O [S,H,d], lse [S,H], c_new [S,H]) where
    ``c_new = c_cache[..., L-2] + logf_new`` (``logf_new`` when L = 1).

    This is the last row i = L-1 of the forward definition: logits
    ``scale * q . k_j + (c_new - c_j)`` for j = 0..L-1 with ``c_{L-1} = c_new``.
    """
    q, kc, vc, cc = _f64(q), _f64(k_cache), _f64(v_cache), _f64(c_cache)
    ln = _f64(logf_new)
    L = kc.shape[2]
    c_prev = cc[..., L - 2] if L >= 2 else np.zeros_like(ln)
    c_new = c_prev + ln
    c_all = np.concatenate([cc[..., : L - 1], c_new[..., None]], axis=-1)  # [S,H,L]
    s = scale * np.einsum("shd,shld->shl", q, kc) + (c_new[..., None] - c_all)
    m = s.max(axis=-1)
    z = np.exp(s - m[..., None]).sum(axis=-1)
    lse = m + np.log(z)
    p = np.exp(s - lse[..., None])
    out = np.einsum("shl,shld->shd", p, vc)
    return out, lse, c_new


def attn_decode_ragged(q, k_cache, v_cache, c_cache, logf_new, lens, scale):
    """Decode against caches of per-sequence length: sequence s uses slots 0..lens[s]-1 of
    caches with capacity L (k_cache, v_cache [S,H,L,d], c_cache [S,H,L]), its new token at
    slot lens[s]-1.  Each sequence is exactly ``attn_decode`` on its own first lens[s] slots.

    Returns (O [S,H,d], lse [S,H], c_new [S,H]).
    """
    q, kc, vc, cc = _f64(q), _f64(k_cache), _f64(v_cache), _f64(c_cache)
    ln = _f64(logf_new)
    S, H, d = q.shape
    out = np.empty((S, H, d))
    lse = np.empty((S, H))
    c_new = np.empty((S, H))
    for s in range(S):
        L = int(lens[s])
        o_s, l_s, c_s = attn_decode(q[s:s + 1], kc[s:s + 1, :, :L], vc[s:s + 1, :, :L], cc[s:s + 1, :, :L],
                                    ln[s:s + 1], scale)
        out[s], lse[s], c_new[s] = o_s[0], l_s[0], c_s[0]
    return out, lse, c_new


def attn_decode_paged(q, k_pages, v_pages, c_pages, block_table, lens, logf_new, scale):
    """Decode against caches held in pages: logical slot j of sequence s is row j % P of page
    block_table[s, j // P] (P = page size) in k_pages, v_pages [num_pages, H, P, d] and c_pages
    [num_pages, H, P].  Each sequence's first lens[s] slots are gathered into a plain cache and
    decoded as ``attn_decode`` (the new token at slot lens[s]-1).

    Returns (O [S,H,d], lse [S,H], c_new [S,H]).
    """
    q = _f64(q)
    kp, vp, cp = np.asarray(k_pages), np.asarray(v_pages), np.asarray(c_pages)
    ln = _f64(logf_new)
    S, H, d = q.shape
    P = kp.shape[2]
    out = np.empty((S, H, d))
    lse = np.empty((S, H))
    c_new = np.empty((S, H))
    for s in range(S):
        L = int(lens[s])
        pages = [int(block_table[s, j // P]) for j in range(L)]
        rows = [j % P for j in range(L)]
        kc = np.stack([kp[pg, :, r] for pg, r in zip(pages, rows)], axis=1)  # [H, L, d]
        vc = np.stack([vp[pg, :, r] for pg, r in zip(pages, rows)], axis=1)
        cc = np.stack([cp[pg, :, r] for pg, r in zip(pages, rows)], axis=1)  # [H, L]
        o_s, l_s, c_s = attn_decode(q[s:s + 1], kc[None], vc[None], cc[None], ln[s:s + 1], scale)
        out[s], lse[s], c_new[s] = o_s[0], l_s[0], c_s[0]
    return out, lse, c_new


def fwd_bwd_head(q, k, v, logf, scale, do, causal: bool = True):
    """Gradients of FoX attention for one head (fp64), from the definition by the chain rule.

    q, k, v: [N, d]; logf: [N]; do: [N, d] (the gradient of a loss with respect to O).
    Returns (dq, dk, dv, dlogf).  The pages derive no backward pass; this differentiates the
    forward above (FoX module page, ``ForgettingAttention.forward``) step by step:

      S = scale q k^T + (c_i - c_j) (masked),  P = softmax_rows(S),  O = P v
      dv = P^T do;   dP = do v^T;   dS = P * (dP - rowsum(dP * P))   (softmax Jacobian)
      dq = scale dS k;   dk = scale dS^T q
      dc_i = sum_j dS_ij - sum_i' dS_i'i   (S_ij depends on c_i with +1 and on c_j with -1)
      dlogf_t = sum_{i >= t} dc_i           (c_i = sum_{t <= i} logf_t)
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    c = logf_cumsum(logf)
    n = q.shape[0]
    s = scale * (q @ k.T) + (c[:, None] - c[None, :])
    if causal:
        s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    dc = ds.sum(axis=1) - ds.sum(axis=0)
    dlogf = np.cumsum(dc[::-1])[::-1]
    return dq, dk, dv, dlogf


def fwd_bwd_tail(q, k, v, logf, scale, do, t0: int):
    """Causal forward and gradients of one head at the positions t0..N-1 only (fp64).

    q, k, v, do: [N, d]; logf: [N].  Returns (O, lse, dq, dk, dv, dlogf), each restricted to
    positions t0..N-1 (rows for O, lse, dq; keys for dk, dv; gates for dlogf).  The same chain
    rule as ``fwd_bwd_head``, written for the last rows: with the causal mask a key j >= t0 is
    seen only by rows i >= j, so dk_j, dv_j and the column sums of dS at j need only the rows
    t0..N-1; dq_i needs the whole row i (every key j <= i); dlogf_t for t >= t0 is the suffix
    sum of dc_i over i >= t.  Lets a sequence too long for the full N x N matrices be checked
    at its end.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    c = logf_cumsum(logf)
    n = q.shape[0]
    r = np.arange(t0, n)
    s = scale * (q[r] @ k.T) + (c[r][:, None] - c[None, :])
    s = np.where(np.arange(n)[None, :] > r[:, None], -np.inf, s)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    p = e / z
    lse = (m + np.log(z))[:, 0]
    o = p @ v
    dp = do[r] @ v.T
    ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
    dq = scale * (ds @ k)
    dv = p[:, t0:].T @ do[r]
    dk = scale * (ds[:, t0:].T @ q[r])
    dc = ds.sum(axis=1) - ds[:, t0:].sum(axis=0)
    dlogf = np.cumsum(dc[::-1])[::-1]
    return o, lse, dq, dk, dv, dlogf


def attn_bwd(q, k, v, logf, scale, do, causal: bool = True):
    """Gradients for every (batch, head): q, k, v, do [B,H,N,d], logf [B,H,N].

    Returns (dq, dk, dv [B,H,N,d], dlogf [B,H,N]) in float64.
    """
    q = _f64(q)
    bsz, nh, n, d = q.shape
    dq, dk, dv = (np.empty((bsz, nh, n, d)) for _ in range(3))
    dl = np.empty((bsz, nh, n))
    for b in range(bsz):
        for h in range(nh):
            dq[b, h], dk[b, h], dv[b, h], dl[b, h] = fwd_bwd_head(q[b, h], k[b, h], v[b, h], logf[b, h], scale,
                                                                 do[b, h], causal=causal)
    return dq, dk, dv, dl
