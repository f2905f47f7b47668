"""Softmax algorithms of the pages, in float64 (test infrastructure only).

Each function follows one passage; the recurrences are written element by
element, in the pages' order, so that they can be read against the text.
"""

import math

import numpy as np


def _vec(x):
    return np.asarray(x, dtype=np.float64).reshape(-1)


def softmax_naive(x):
    """Unsafe softmax e^{x_i} / sum_j e^{x_j}.

    [P1] "(Safe) Softmax" and [P2] 2.1: the textbook formula, which overflows
    once some x_i is large (exp(1000) is inf in float64, and inf/inf is NaN).
    Kept only to show that failure.
    """
    x = _vec(x)
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(x)
        return e / e.sum()


def softmax_3pass(x):
    """Safe softmax in three passes over x ([P1] "(Safe) Softmax").

    pass 1: m_N = max_j x_j
    pass 2: d_N = sum_j e^{x_j - m_N}
    pass 3: a_i = e^{x_i - m_N} / d_N
    Subtracting the maximum makes every exponent <= 0; by shift invariance
    ([P3] "瓦片注意力计算") the result equals the unsafe formula where that
    one does not overflow.
    """
    x = _vec(x)
    m = -math.inf
    for xi in x:
        m = max(m, float(xi))
    d = 0.0
    for xi in x:
        d += math.exp(float(xi) - m)
    return np.array([math.exp(float(xi) - m) / d for xi in x])


def online_normaliser_states(x):
    """States (m_i, d'_i) of the online normaliser after each element.

    [P1] "从3-pass到2-pass" and [P2] 2.1: read the elements one at a time,
    keeping the running maximum m_i and a running denominator d'_i taken
    relative to m_i.  When the maximum grows, the old denominator is scaled
    by e^{m_{i-1} - m_i} (the page's garbled factor read as this product; it is
    the only reading under which d'_N equals d_N, as the page requires):

        m_i   = max(m_{i-1}, x_i)
        d'_i  = d'_{i-1} * e^{m_{i-1} - m_i} + e^{x_i - m_i}

    with m_0 = -inf and d'_0 = 0.  Returns a list of (m_i, d'_i), i = 1..N.
    """
    x = _vec(x)
    m_prev, d_prev = -math.inf, 0.0
    states = []
    for xi in x:
        xi = float(xi)
        m = max(m_prev, xi)
        scale_old = 0.0 if m_prev == -math.inf else math.exp(m_prev - m)
        d = d_prev * scale_old + math.exp(xi - m)
        states.append((m, d))
        m_prev, d_prev = m, d
    return states


def softmax_2pass_online(x):
    """2-pass online softmax ([P1] "从3-pass到2-pass").

    pass 1: the online normaliser gives (m_N, d'_N) in one sweep;
    pass 2: a_i = e^{x_i - m_N} / d'_N.
    """
    x = _vec(x)
    m_n, d_n = online_normaliser_states(x)[-1]
    return np.array([math.exp(float(xi) - m_n) / d_n for xi in x])


def softmax_stats(x):
    """(m(x), l(x)) of one block: its maximum and sum_j e^{x_j - m(x)}.

    These are the per-block statistics of [P3] "瓦片注意力计算".  An empty
    block has m = -inf and l = 0, the identity of ``merge_stats``.
    """
    x = _vec(x)
    if x.size == 0:
        return -math.inf, 0.0
    m = float(np.max(x))
    l = math.fsum(math.exp(float(xi) - m) for xi in x)
    return m, l


def merge_stats(a, b):
    """Statistics of the concatenation [x1, x2] from those of x1 and x2.

    [P3] "瓦片注意力计算": m = max(m1, m2) and
    l = e^{m1 - m} * l1 + e^{m2 - m} * l2.
    """
    m1, l1 = a
    m2, l2 = b
    m = max(m1, m2)
    if m == -math.inf:
        return -math.inf, 0.0
    w1 = 0.0 if m1 == -math.inf else math.exp(m1 - m)
    w2 = 0.0 if m2 == -math.inf else math.exp(m2 - m)
    return m, w1 * l1 + w2 * l2


def softmax_blocked(x, splits):
    """Softmax computed block by block and merged with ``merge_stats``.

    ``splits`` are the cut points (sorted indices in 0..N) that divide x into
    consecutive blocks.  The blocks' statistics are merged left to right; the
    outputs are then e^{x_i - m} / l with the merged (m, l).
    """
    x = _vec(x)
    cuts = [0] + sorted(int(s) for s in splits) + [x.size]
    stats = (-math.inf, 0.0)
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        stats = merge_stats(stats, softmax_stats(x[lo:hi]))
    m, l = stats
    return np.array([math.exp(float(xi) - m) / l for xi in x])
