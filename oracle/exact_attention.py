"""Exact attention in float64 (test infrastructure only).

``attention`` is the definition itself, written out: it materialises the
score matrix S for one (batch, head) at a time, exactly the standard
attention that [P3] "什么是注意力？" states and whose O(n^2) memory the method
removes.  The GPU path must reach this result up to rounding, because the
method is exact ([P2], introduction: speed without loss of accuracy).

Readings of the pages that this file relies on (the formulas themselves were
lost from the pages' text):
  * scores are S = scale * Q K^T with the caller's scale (1/sqrt(d) in every
    workload used here);
  * with ``causal`` set, key j is visible to query i iff j <= i (the mask is
    not on the pages; it belongs to the causal workload);
  * L is the natural-log logsumexp of the scaled, masked scores of each row,
    L_i = m_i + ln sum_j e^{S_ij - m_i} (also not on the pages; it is what a
    backward pass that recomputes S, [P3] "Flash Attention", needs);
  * a row whose every key is masked (impossible when queries and keys have
    the same length) is defined as O = 0, L = -inf.

Arrays are [B, H, N, d] (any float dtype, upcast exactly to float64);
O is [B, H, N, d] and L is [B, H, N], both float64.
"""

import math

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _causal_mask(n_q, kv_lo, kv_hi):
    """Boolean [n_q, kv_hi - kv_lo]: True where key j > query i (hidden)."""
    i = np.arange(n_q)[:, None]
    j = np.arange(kv_lo, kv_hi)[None, :]
    return j > i


def attention(q, k, v, scale, causal=False):
    """O = softmax(scale * Q K^T) V and L = logsumexp, by the definition.

    Per (b, h): S is materialised in full, masked, and passed through the safe
    (max-subtracted) softmax of [P1] "(Safe) Softmax"; the probabilities P are
    normalised rows, O = P V.  Returns (O, L).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, v.shape[-1]))
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            S = scale * (q[b, h] @ k[b, h].T)
            if causal:
                S[_causal_mask(N, 0, k.shape[2])] = -np.inf
            m = S.max(axis=1)
            dead = ~np.isfinite(m)
            m_safe = np.where(dead, 0.0, m)
            E = np.exp(S - m_safe[:, None])
            l = E.sum(axis=1)
            with np.errstate(invalid="ignore", divide="ignore"):
                P = np.where(dead[:, None], 0.0, E / np.where(dead, 1.0, l)[:, None])
                O[b, h] = P @ v[b, h]
                L[b, h] = np.where(dead, -np.inf, m_safe + np.log(np.where(dead, 1.0, l)))
    return O, L


def expand_block_mask(block_mask, n_q, block=64, n_k=None):
    """Boolean [n_q, n_k] element mask (True = visible) of a block mask.

    Query i and key j are in blocks i // block and j // block; the last block
    of each side may be partial.  n_k defaults to n_q.
    """
    n_k = n_q if n_k is None else n_k
    bm = np.asarray(block_mask) != 0
    return bm[np.ix_(np.arange(n_q) // block, np.arange(n_k) // block)]


def attention_block_sparse(q, k, v, scale, causal, block_mask, block=64):
    """The definition with a block mask: key j is visible to query i iff the
    block (i // block, j // block) is set (and, with ``causal``, j <= i).

    The Triton article's introduction ([P3]) extends the tiled kernel to
    block-sparse attention without stating it further; this is the plainest
    reading: hidden scores are -inf before the softmax, exactly as the causal
    mask, so a row with no visible key is O = 0, L = -inf.  ``block_mask`` is
    [nbq, nbk] (shared by every head), [H, nbq, nbk] (per head) or
    [B, H, nbq, nbk], with nbq = ceil(N_q / block), nbk = ceil(N_k / block).
    Returns (O, L) in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    bm = np.asarray(block_mask)
    nbq, nbk = -(-Nq // block), -(-Nk // block)
    if bm.shape[-2:] != (nbq, nbk):
        raise ValueError(f"block mask must end in ({nbq}, {nbk})")
    if bm.ndim == 2:
        bm = np.broadcast_to(bm, (B, H, nbq, nbk))
    elif bm.ndim == 3:
        bm = np.broadcast_to(bm[None], (B, H, nbq, nbk))
    O = np.zeros((B, H, Nq, v.shape[-1]))
    L = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            S = scale * (q[b, h] @ k[b, h].T)
            hidden = ~expand_block_mask(bm[b, h], Nq, block, Nk)
            if causal:
                hidden |= _causal_mask(Nq, 0, Nk)
            S[hidden] = -np.inf
            m = S.max(axis=1)
            dead = ~np.isfinite(m)
            m_safe = np.where(dead, 0.0, m)
            E = np.exp(S - m_safe[:, None])
            l = E.sum(axis=1)
            with np.errstate(invalid="ignore", divide="ignore"):
                P = np.where(dead[:, None], 0.0, E / np.where(dead, 1.0, l)[:, None])
                O[b, h] = P @ v[b, h]
                L[b, h] = np.where(dead, -np.inf, m_safe + np.log(np.where(dead, 1.0, l)))
    return O, L


def attention_block_sparse_rows(q, k, v, scale, causal, block_mask, rows, block=64):
    """``attention_block_sparse`` for selected rows (b, h, i) only, O(N d) each.

    ``block_mask`` as in ``attention_block_sparse``.  Returns (O_rows [R, d],
    L_rows [R]) in float64; a row with no visible key gives O = 0, L = -inf.
    """
    bm = np.asarray(block_mask)
    N = k.shape[2]
    O = np.zeros((len(rows), v.shape[-1]))
    L = np.zeros(len(rows))
    for n, (b, h, i) in enumerate(rows):
        m = bm if bm.ndim == 2 else bm[h] if bm.ndim == 3 else bm[b, h]
        kk, vv = _f64(k[b, h]), _f64(v[b, h])
        s = scale * (kk @ _f64(q[b, h, i]))
        vis = m[i // block, np.arange(N) // block] != 0
        if causal:
            vis &= np.arange(N) <= i
        if not vis.any():
            L[n] = -np.inf
            continue
        s = np.where(vis, s, -np.inf)
        mx = s.max()
        e = np.exp(s - mx)
        O[n] = (e @ vv) / e.sum()
        L[n] = mx + np.log(e.sum())
    return O, L


def attention_rows(q, k, v, scale, causal, rows):
    """The definition for selected query rows only.

    ``rows`` is a sequence of (b, h, i).  Each row costs O(N d), so this checks
    sampled outputs of workloads whose full S would not fit in host memory.
    Returns (O_rows [R, d], L_rows [R]) in float64.
    """
    out_o = []
    out_l = []
    for (b, h, i) in rows:
        kk = _f64(k[b, h])
        vv = _f64(v[b, h])
        qi = _f64(q[b, h, i])
        s = scale * (kk @ qi)
        if causal:
            s[np.arange(kk.shape[0]) > i] = -np.inf
        m = s.max()
        if not np.isfinite(m):
            out_o.append(np.zeros(vv.shape[1]))
            out_l.append(-np.inf)
            continue
        e = np.exp(s - m)
        l = e.sum()
        out_o.append((e @ vv) / l)
        out_l.append(m + math.log(l))
    return np.array(out_o), np.array(out_l)


def attention_online_tiled(q, k, v, scale, causal=False, block_q=16, block_kv=16):
    """The one-pass tiled algorithm, step by step, in float64.

    Follows [P2] 2.2 and [P3] "算法概述": fix one block of queries, stream every
    block of keys and values past it, and keep, per query row, the largest
    score seen so far m, the softmax denominator l relative to m, and the
    un-normalised output acc.  For each key block:
        S~    = scale * Q_blk K_blk^T          (masked entries -inf)
        m_new = max(m, rowmax(S~))
        P~    = e^{S~ - m_new}
        l     = e^{m - m_new} * l + rowsum(P~)   (old part rescaled, new part added)
        acc   = e^{m - m_new} * acc + P~ V_blk
    and after the last block O = acc / l, L = m + ln l.  The normalisation is
    applied once at the end (the pages' own per-step form divides and
    re-multiplies by l each step; both give the same O).  The pages also give
    the transposed loop order (key blocks outside); it reaches the same
    numbers, so only this one is written.  Used only to show that the
    recurrence reaches ``attention``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    O = np.zeros((B, H, N, v.shape[-1]))
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i0 in range(0, N, block_q):
                i1 = min(i0 + block_q, N)
                Qb = q[b, h, i0:i1]
                m = np.full(i1 - i0, -np.inf)
                l = np.zeros(i1 - i0)
                acc = np.zeros((i1 - i0, v.shape[-1]))
                for j0 in range(0, Nk, block_kv):
                    j1 = min(j0 + block_kv, Nk)
                    S = scale * (Qb @ k[b, h, j0:j1].T)
                    if causal:
                        ii = np.arange(i0, i1)[:, None]
                        jj = np.arange(j0, j1)[None, :]
                        S[jj > ii] = -np.inf
                    m_new = np.maximum(m, S.max(axis=1))
                    base = np.where(np.isfinite(m_new), m_new, 0.0)
                    P = np.exp(S - base[:, None])
                    alpha = np.where(np.isfinite(m), np.exp(m - base), 0.0)
                    l = alpha * l + P.sum(axis=1)
                    acc = alpha[:, None] * acc + P @ v[b, h, j0:j1]
                    m = m_new
                dead = l == 0.0
                O[b, h, i0:i1] = np.where(dead[:, None], 0.0,
                                          acc / np.where(dead, 1.0, l)[:, None])
                L[b, h, i0:i1] = np.where(dead, -np.inf,
                                          m + np.log(np.where(dead, 1.0, l)))
    return O, L


def attention_partial(q, k, v, scale, causal, kv_lo, kv_hi):
    """Attention statistics over the key range [kv_lo, kv_hi) only.

    Returns (m, l, acc): the row maximum of the visible scores in the range,
    the denominator relative to it, and the un-normalised sum of e^{S - m} V.
    An empty or fully masked range gives m = -inf, l = 0, acc = 0.  Several
    such partials combine with ``merge_partials`` (the rule for a
    concatenation, [P3] "瓦片注意力计算", extended to the output because the
    product with V is linear).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    dv = v.shape[-1]
    m = np.full((B, H, N), -np.inf)
    l = np.zeros((B, H, N))
    acc = np.zeros((B, H, N, dv))
    if kv_hi <= kv_lo:
        return m, l, acc
    for b in range(B):
        for h in range(H):
            S = scale * (q[b, h] @ k[b, h, kv_lo:kv_hi].T)
            if causal:
                S[_causal_mask(N, kv_lo, kv_hi)] = -np.inf
            mm = S.max(axis=1)
            base = np.where(np.isfinite(mm), mm, 0.0)
            E = np.exp(S - base[:, None])
            m[b, h] = mm
            l[b, h] = E.sum(axis=1)
            acc[b, h] = E @ v[b, h, kv_lo:kv_hi]
    return m, l, acc


def merge_partials(parts):
    """Combine partials from ``attention_partial`` into (O, L).

    m = max over parts; each part's l and acc are weighted by e^{m_p - m}
    (zero for an empty part); O = sum(acc) / sum(l), L = m + ln sum(l).
    """
    ms = np.stack([p[0] for p in parts])
    m = ms.max(axis=0)
    base = np.where(np.isfinite(m), m, 0.0)
    l = np.zeros_like(m)
    acc = np.zeros_like(parts[0][2])
    for (mp, lp, ap) in parts:
        w = np.where(np.isfinite(mp), np.exp(mp - base), 0.0)
        l = l + w * lp
        acc = acc + w[..., None] * ap
    dead = l == 0.0
    O = np.where(dead[..., None], 0.0, acc / np.where(dead, 1.0, l)[..., None])
    L = np.where(dead, -np.inf, m + np.log(np.where(dead, 1.0, l)))
    return O, L
