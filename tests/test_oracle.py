"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself: the worked example
of the online normaliser, closed forms, a pure-Python brute force with
``math.fsum``, library routines (scipy's softmax, torch's CPU attention in
float64), and invariants of softmax and attention.  The last group plants
plausible mistakes in copies of the oracle and shows that some pin fails for
each of them.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import exact_attention as oatt
from oracle import softmax as osm

HERE = os.path.dirname(__file__)


# ----------------------------------------------------------------------------
# helpers


def _rand(rng, *shape, sd=1.0):
    return rng.standard_normal(shape) * sd


def brute_attention(q, k, v, scale, causal):
    """Attention with scalar loops, math.exp and math.fsum (tiny inputs only)."""
    B, H, N, d = q.shape
    dv = v.shape[-1]
    O = np.zeros((B, H, N, dv))
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                vis = [j for j in range(k.shape[2]) if (not causal or j <= i)]
                s = [scale * math.fsum(float(q[b, h, i, t]) * float(k[b, h, j, t])
                                       for t in range(d)) for j in vis]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                tot = math.fsum(e)
                for t in range(dv):
                    O[b, h, i, t] = math.fsum(e[n] * float(v[b, h, j, t])
                                              for n, j in enumerate(vis)) / tot
                L[b, h, i] = m + math.log(tot)
    return O, L


# ----------------------------------------------------------------------------
# pin checks, written as functions of an implementation so that the mutation
# tests below can run them against planted mistakes


def check_worked_example(states_fn):
    with open(os.path.join(HERE, "golden", "online_softmax_worked_example.json")) as f:
        g = json.load(f)
    x = g["x"]
    states = states_fn(x)
    assert len(states) == len(x)
    ms = [s[0] for s in states]
    assert ms == g["max_after_step"]
    changes = [i + 1 for i in range(1, len(ms)) if ms[i] != ms[i - 1]]
    assert changes == g["max_changes_at_steps"]
    for kstep, (m, dval) in enumerate(states, start=1):
        closed = math.fsum(math.exp(xj - m) for xj in x[:kstep])
        assert abs(dval - closed) <= 1e-15 * closed, (kstep, dval, closed)
    # the final normaliser gives the safe softmax of the whole vector
    m_n, d_n = states[-1]
    tot = math.fsum(math.exp(xj) for xj in x)
    for xj in x:
        assert abs(math.exp(xj - m_n) / d_n - math.exp(xj) / tot) <= 1e-15


def check_brute_force(att):
    rng = np.random.default_rng(7)
    for N in (1, 2, 3, 5, 8, 16):
        for d in (1, 4, 8):
            for causal in (False, True):
                q = _rand(rng, 1, 2, N, d)
                k = _rand(rng, 1, 2, N, d)
                v = _rand(rng, 1, 2, N, d)
                scale = 1.0 / math.sqrt(d)
                O, L = att(q, k, v, scale, causal)
                Ob, Lb = brute_attention(q, k, v, scale, causal)
                np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-13)
                np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-13)


def check_closed_forms(att):
    rng = np.random.default_rng(11)
    N, d = 12, 5
    v = _rand(rng, 1, 1, N, d)
    q = _rand(rng, 1, 1, N, d)
    zeros = np.zeros((1, 1, N, d))
    # K = 0: every score is 0, attention is uniform over the visible keys.
    O, L = att(q, zeros, v, 0.7, False)
    np.testing.assert_allclose(O[0, 0], np.tile(v[0, 0].mean(axis=0), (N, 1)), atol=1e-14)
    np.testing.assert_allclose(L[0, 0], np.full(N, math.log(N)), atol=1e-14)
    O, L = att(q, zeros, v, 0.7, True)
    prefix = np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    np.testing.assert_allclose(O[0, 0], prefix, atol=1e-14)
    np.testing.assert_allclose(L[0, 0], np.log(np.arange(1, N + 1)), atol=1e-14)
    # N = 1: the only key gets weight 1.
    q1, k1, v1 = (_rand(rng, 2, 3, 1, d) for _ in range(3))
    O, L = att(q1, k1, v1, 0.3, False)
    np.testing.assert_allclose(O, v1, atol=1e-15)
    np.testing.assert_allclose(L, 0.3 * np.einsum("bhnd,bhnd->bhn", q1, k1), atol=1e-14)
    # V = 1: every output is 1 (rows of P sum to 1).
    k = _rand(rng, 1, 1, N, d)
    O, _ = att(q, k, np.ones((1, 1, N, d)), 0.5, True)
    np.testing.assert_allclose(O, 1.0, atol=1e-14)
    # One key dominating by a margin of ~1e3 takes all the weight.
    kd = _rand(rng, 1, 1, N, d) * 0.01
    kd[0, 0, 4] = q[0, 0, 7] * 400.0
    O, _ = att(q[:, :, 7:8], kd, v, 1.0, False)
    np.testing.assert_allclose(O[0, 0, 0], v[0, 0, 4], atol=1e-12)
    # V = I (square): O is P itself; rows are distributions, causal zeros above
    # the diagonal.
    k = _rand(rng, 1, 1, N, N)
    qq = _rand(rng, 1, 1, N, N)
    eye = np.eye(N)[None, None]
    for causal in (False, True):
        P, _ = att(qq, k, eye, 0.4, causal)
        assert np.all(P >= 0)
        np.testing.assert_allclose(P.sum(axis=-1), 1.0, atol=1e-14)
        if causal:
            assert np.all(np.triu(P[0, 0], 1) == 0)
        else:
            assert np.all(P > 0)


def check_library(att):
    """torch's CPU attention in float64 and scipy's logsumexp as references."""
    rng = np.random.default_rng(5)
    B, H, N, d = 2, 3, 33, 16
    q, k, v = (_rand(rng, B, H, N, d) for _ in range(3))
    scale = 1.0 / math.sqrt(d)
    for causal in (False, True):
        O, L = att(q, k, v, scale, causal)
        Ot = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            is_causal=causal, scale=scale).numpy()
        np.testing.assert_allclose(O, Ot, atol=1e-12)
        S = scale * np.matmul(q, np.swapaxes(k, -1, -2))
        if causal:
            S = np.where(np.triu(np.ones((N, N), bool), 1), -np.inf, S)
        np.testing.assert_allclose(L, scipy.special.logsumexp(S, axis=-1), atol=1e-12)


def check_invariants(att):
    rng = np.random.default_rng(3)
    B, H, N, d = 1, 2, 20, 6
    q, k, v, v2 = (_rand(rng, B, H, N, d) for _ in range(4))
    O, L = att(q, k, v, 0.5, False)
    # Permuting keys and values together changes nothing (non-causal).
    perm = rng.permutation(N)
    Op, Lp = att(q, k[:, :, perm], v[:, :, perm], 0.5, False)
    np.testing.assert_allclose(Op, O, atol=1e-13)
    np.testing.assert_allclose(Lp, L, atol=1e-13)
    # O is linear in V.
    O2, _ = att(q, k, v2, 0.5, False)
    O3, _ = att(q, k, 2.0 * v - 3.0 * v2, 0.5, False)
    np.testing.assert_allclose(O3, 2.0 * O - 3.0 * O2, atol=1e-13)
    # Permuting queries permutes outputs.
    Oq, Lq = att(q[:, :, perm], k, v, 0.5, False)
    np.testing.assert_allclose(Oq, O[:, :, perm], atol=1e-13)
    np.testing.assert_allclose(Lq, L[:, :, perm], atol=1e-13)


ATTENTION_PINS = (check_brute_force, check_closed_forms, check_library, check_invariants)


def _tiled(block_q, block_kv):
    def att(q, k, v, scale, causal):
        return oatt.attention_online_tiled(q, k, v, scale, causal, block_q, block_kv)
    return att


def _by_rows(q, k, v, scale, causal):
    B, H, N, _ = q.shape
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(N)]
    o, l = oatt.attention_rows(q, k, v, scale, causal, rows)
    return o.reshape(B, H, N, -1), l.reshape(B, H, N)


def _by_partials(q, k, v, scale, causal):
    N = k.shape[2]
    cuts = [0, N // 3, N // 3, (2 * N) // 3, N]
    parts = [oatt.attention_partial(q, k, v, scale, causal, a, b)
             for a, b in zip(cuts[:-1], cuts[1:])]
    return oatt.merge_partials(parts)


def _block_sparse_all_ones(block):
    def att(q, k, v, scale, causal):
        nbq, nbk = -(-q.shape[2] // block), -(-k.shape[2] // block)
        return oracle.attention_block_sparse(q, k, v, scale, causal,
                                             np.ones((nbq, nbk), np.uint8), block)
    return att


IMPLEMENTATIONS = {
    "definition": oracle.attention,
    "block_sparse_all_ones_b4": _block_sparse_all_ones(4),
    "block_sparse_all_ones_b64": _block_sparse_all_ones(64),
    "tiled_4x4": _tiled(4, 4),
    "tiled_3x5": _tiled(3, 5),
    "tiled_16x7": _tiled(16, 7),
    "rows": _by_rows,
    "partials": _by_partials,
}


# ----------------------------------------------------------------------------
# softmax pins


def test_worked_example():
    check_worked_example(osm.online_normaliser_states)


def test_worked_example_rescale_step():
    """At step 3 the new denominator is the old one times e^{2-3} plus e^0."""
    (_, d1), (_, d2), (_, d3) = osm.online_normaliser_states([2.0, 1.0, 3.0])
    assert d1 == 1.0
    assert d2 == 1.0 + math.exp(-1.0)
    assert abs(d3 - (d2 * math.exp(-1.0) + 1.0)) <= 1e-16


@pytest.mark.parametrize("spread", [1.0, 10.0, 1e3])
def test_softmax_variants_agree(spread):
    rng = np.random.default_rng(int(spread))
    for n in (1, 2, 7, 64, 200):
        x = _rand(rng, n, sd=spread)
        ref = scipy.special.softmax(x)
        for got in (osm.softmax_3pass(x), osm.softmax_2pass_online(x),
                    osm.softmax_blocked(x, sorted(rng.integers(0, n + 1, size=3)))):
            np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-300)


def test_blocked_every_split():
    rng = np.random.default_rng(1)
    x = _rand(rng, 12, sd=4.0)
    m, l = osm.softmax_stats(x)
    assert m == x.max()
    for cut in range(13):
        mm, ll = osm.merge_stats(osm.softmax_stats(x[:cut]), osm.softmax_stats(x[cut:]))
        assert mm == m
        assert abs(ll - l) <= 1e-14 * l
        np.testing.assert_allclose(osm.softmax_blocked(x, [cut]),
                                   scipy.special.softmax(x), rtol=1e-14)


def test_merge_stats_two_scalars():
    for a, b in [(0.0, 0.0), (1.0, -2.0), (-5.0, 3.0), (700.0, 699.0)]:
        m, l = osm.merge_stats((a, 1.0), (b, 1.0))
        assert m == max(a, b)
        assert abs(l - (math.exp(a - m) + math.exp(b - m))) <= 1e-15
    assert osm.merge_stats((-math.inf, 0.0), (2.0, 3.0)) == (2.0, 3.0)


def test_shift_invariance():
    rng = np.random.default_rng(2)
    x = _rand(rng, 50, sd=5.0)
    for c in (-300.0, 1.5, 1e3):
        np.testing.assert_allclose(osm.softmax_3pass(x + c), osm.softmax_3pass(x), rtol=1e-12)
        np.testing.assert_allclose(osm.softmax_2pass_online(x + c),
                                   osm.softmax_2pass_online(x), rtol=1e-12)


def test_naive_overflows_safe_does_not():
    x = [1000.0, 1.0, 2.0]
    naive = osm.softmax_naive(x)
    assert np.isnan(naive[0])
    for fn in (osm.softmax_3pass, osm.softmax_2pass_online):
        s = fn(x)
        assert np.all(np.isfinite(s))
        assert s[0] == 1.0
        assert abs(s.sum() - 1.0) <= 1e-15


def test_softmax_sums_to_one_and_positive():
    rng = np.random.default_rng(9)
    for _ in range(20):
        x = _rand(rng, 31, sd=30.0)
        for fn in (osm.softmax_3pass, osm.softmax_2pass_online):
            s = fn(x)
            assert np.all(s >= 0)
            assert abs(math.fsum(s) - 1.0) <= 1e-14


# ----------------------------------------------------------------------------
# attention pins, for every way the oracle can compute attention


@pytest.mark.parametrize("impl", sorted(IMPLEMENTATIONS))
@pytest.mark.parametrize("pin", ATTENTION_PINS, ids=lambda f: f.__name__)
def test_attention_pins(impl, pin):
    pin(IMPLEMENTATIONS[impl])


@pytest.mark.parametrize("causal", [False, True])
def test_tiled_reaches_definition_with_large_logits(causal):
    """Logits of several hundred (as in the stress workload) and ragged tiles."""
    rng = np.random.default_rng(4)
    B, H, N, d = 2, 2, 37, 8
    q = _rand(rng, B, H, N, d, sd=3.0) + rng.uniform(-20, 20, (B, H, N, 1)) * math.sqrt(d)
    k = _rand(rng, B, H, N, d, sd=3.0)
    v = _rand(rng, B, H, N, d)
    scale = 1.0 / math.sqrt(d)
    O, L = oracle.attention(q, k, v, scale, causal)
    assert np.abs(L).max() > 100.0
    for bq, bk in [(1, 1), (8, 8), (5, 16), (37, 37), (64, 3)]:
        Ot, Lt = oatt.attention_online_tiled(q, k, v, scale, causal, bq, bk)
        np.testing.assert_allclose(Ot, O, atol=1e-12)
        np.testing.assert_allclose(Lt, L, atol=1e-11, rtol=1e-14)


def test_rows_match_full():
    rng = np.random.default_rng(6)
    q, k, v = (_rand(rng, 2, 2, 50, 8) for _ in range(3))
    for causal in (False, True):
        O, L = oracle.attention(q, k, v, 0.3, causal)
        rows = [(1, 0, 0), (0, 1, 49), (1, 1, 17)]
        o, l = oracle.attention_rows(q, k, v, 0.3, causal, rows)
        for n, (b, h, i) in enumerate(rows):
            np.testing.assert_allclose(o[n], O[b, h, i], atol=1e-14)
            assert abs(l[n] - L[b, h, i]) <= 1e-13


def test_empty_partials_are_identity():
    rng = np.random.default_rng(8)
    q, k, v = (_rand(rng, 1, 1, 6, 3) for _ in range(3))
    full = oatt.attention_partial(q, k, v, 1.0, False, 0, 6)
    empty = oatt.attention_partial(q, k, v, 1.0, False, 3, 3)
    O, L = oatt.merge_partials([empty, full, empty])
    Od, Ld = oracle.attention(q, k, v, 1.0, False)
    np.testing.assert_allclose(O, Od, atol=1e-14)
    np.testing.assert_allclose(L, Ld, atol=1e-14)


# ----------------------------------------------------------------------------
# planted mistakes: each mutant of the oracle must fail at least one pin


def _mutant_no_scale(q, k, v, scale, causal):
    return oracle.attention(q, k, v, 1.0, causal)


def _mutant_transposed_scores(q, k, v, scale, causal):
    # S = scale * K Q^T instead of Q K^T (a transposed operand).
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    B, H, N, d = q.shape
    O = np.zeros_like(v)
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            S = scale * (k[b, h] @ q[b, h].T)
            if causal:
                S[np.triu(np.ones((N, N), bool), 1)] = -np.inf
            m = S.max(1)
            E = np.exp(S - m[:, None])
            O[b, h] = (E / E.sum(1)[:, None]) @ v[b, h]
            L[b, h] = m + np.log(E.sum(1))
    return O, L


def _mutant_mask_off_by_one(q, k, v, scale, causal):
    # hides the diagonal too (j >= i), except row 0 which would be empty
    if not causal:
        return oracle.attention(q, k, v, scale, causal)
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    B, H, N, d = q.shape
    O, L = oracle.attention(q, k, v, scale, True)
    for b in range(B):
        for h in range(H):
            for i in range(1, N):
                o, l = oracle.attention_rows(q[b:b + 1, h:h + 1, :, :], k[b:b + 1, h:h + 1, :i],
                                             v[b:b + 1, h:h + 1, :i], scale, False,
                                             [(0, 0, i)])
                O[b, h, i], L[b, h, i] = o[0], l[0]
    return O, L


def _mutant_lse_without_max(q, k, v, scale, causal):
    O, L = oracle.attention(q, k, v, scale, causal)
    Lm = np.zeros_like(L)
    q64, k64 = np.asarray(q, np.float64), np.asarray(k, np.float64)
    S = scale * np.matmul(q64, np.swapaxes(k64, -1, -2))
    if causal:
        N = S.shape[-1]
        S = np.where(np.triu(np.ones((N, N), bool), 1), -np.inf, S)
    Lm = L - S.max(-1)
    return O, Lm


def _mutant_tiled_alpha_inverted(q, k, v, scale, causal):
    # the rescale factor taken as e^{m_new - m} instead of e^{m - m_new}
    orig = np.exp
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    B, H, N, d = q.shape
    O = np.zeros_like(v)
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            acc = np.zeros((N, d))
            for j0 in range(0, N, 3):
                j1 = min(j0 + 3, N)
                S = scale * (q[b, h] @ k[b, h, j0:j1].T)
                if causal:
                    S[np.arange(j0, j1)[None, :] > np.arange(N)[:, None]] = -np.inf
                m_new = np.maximum(m, S.max(1))
                base = np.where(np.isfinite(m_new), m_new, 0.0)
                P = orig(S - base[:, None])
                alpha = np.where(np.isfinite(m), orig(base - m), 0.0)
                l = alpha * l + P.sum(1)
                acc = alpha[:, None] * acc + P @ v[b, h, j0:j1]
                m = m_new
            O[b, h] = acc / l[:, None]
            L[b, h] = m + np.log(l)
    return O, L


def _mutant_tiled_no_rescale(q, k, v, scale, causal):
    # drops the rescale of the old denominator and output (a dropped term)
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    B, H, N, d = q.shape
    O = np.zeros_like(v)
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            acc = np.zeros((N, d))
            for j0 in range(0, N, 3):
                j1 = min(j0 + 3, N)
                S = scale * (q[b, h] @ k[b, h, j0:j1].T)
                if causal:
                    S[np.arange(j0, j1)[None, :] > np.arange(N)[:, None]] = -np.inf
                m_new = np.maximum(m, S.max(1))
                base = np.where(np.isfinite(m_new), m_new, 0.0)
                P = np.exp(S - base[:, None])
                l = l + P.sum(1)
                acc = acc + P @ v[b, h, j0:j1]
                m = m_new
            O[b, h] = acc / l[:, None]
            L[b, h] = m + np.log(l)
    return O, L


def _mutant_softmax_wrong_axis(q, k, v, scale, causal):
    # normalises over queries (columns of S) instead of over keys (rows)
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    B, H, N, d = q.shape
    O = np.zeros_like(v)
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            S = scale * (q[b, h] @ k[b, h].T)
            if causal:
                S[np.triu(np.ones((N, N), bool), 1)] = -np.inf
            m = S.max(0)
            E = np.exp(S - m[None, :])
            O[b, h] = (E / E.sum(0)[None, :]) @ v[b, h]
            L[b, h] = m + np.log(E.sum(0))
    return O, L


MUTANTS = {
    "no_scale": _mutant_no_scale,
    "transposed_scores": _mutant_transposed_scores,
    "mask_off_by_one": _mutant_mask_off_by_one,
    "lse_without_max": _mutant_lse_without_max,
    "tiled_alpha_inverted": _mutant_tiled_alpha_inverted,
    "tiled_no_rescale": _mutant_tiled_no_rescale,
    "softmax_wrong_axis": _mutant_softmax_wrong_axis,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name):
    mutant = MUTANTS[name]
    caught = []
    for pin in ATTENTION_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mutant)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"


def _states_alpha_inverted(x):
    m_prev, d_prev, out = -math.inf, 0.0, []
    for xi in x:
        m = max(m_prev, xi)
        f = 0.0 if m_prev == -math.inf else math.exp(m - m_prev)
        d = d_prev * f + math.exp(xi - m)
        out.append((m, d))
        m_prev, d_prev = m, d
    return out


def _states_subtracted_factor(x):
    # the page's garbled form e^{m_{i-1}} - e^{m_i} taken literally
    m_prev, d_prev, out = -math.inf, 0.0, []
    for xi in x:
        m = max(m_prev, xi)
        f = 0.0 if m_prev == -math.inf else math.exp(m_prev) - math.exp(m)
        d = d_prev * f + math.exp(xi - m)
        out.append((m, d))
        m_prev, d_prev = m, d
    return out


@pytest.mark.parametrize("states_fn", [_states_alpha_inverted, _states_subtracted_factor])
def test_worked_example_catches_wrong_rescale(states_fn):
    with pytest.raises(AssertionError):
        check_worked_example(states_fn)


# ----------------------------------------------------------------------------
# block-sparse pins: the mask itself


def brute_attention_masked(q, k, v, scale, visible):
    """Scalar loops with math.exp / math.fsum; visible(b, h, i, j) -> bool."""
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, v.shape[-1]))
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                vis = [j for j in range(N) if visible(b, h, i, j)]
                if not vis:
                    L[b, h, i] = -math.inf
                    continue
                s = [scale * math.fsum(float(q[b, h, i, t]) * float(k[b, h, j, t])
                                       for t in range(d)) for j in vis]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                tot = math.fsum(e)
                for t in range(v.shape[-1]):
                    O[b, h, i, t] = math.fsum(e[n] * float(v[b, h, j, t])
                                              for n, j in enumerate(vis)) / tot
                L[b, h, i] = m + math.log(tot)
    return O, L


def check_block_mask_brute_force(att_bs):
    """Random masks (per head), tiny blocks, ragged N, with and without causal."""
    rng = np.random.default_rng(21)
    for N, block in ((5, 2), (8, 3), (13, 4)):
        nb = -(-N // block)
        B, H, d = 1, 2, 3
        q, k, v = (_rand(rng, B, H, N, d) for _ in range(3))
        bm = (rng.random((H, nb, nb)) < 0.5).astype(np.uint8)
        bm[0, 0, :] = 0  # an empty block row: its queries see nothing
        for causal in (False, True):
            O, L = att_bs(q, k, v, 0.6, causal, bm, block)

            def visible(b, h, i, j):
                return bool(bm[h, i // block, j // block]) and (not causal or j <= i)
            Ob, Lb = brute_attention_masked(q, k, v, 0.6, visible)
            np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-13)
            assert np.array_equal(np.isneginf(L), np.isneginf(Lb))
            fin = np.isfinite(Lb)
            np.testing.assert_allclose(L[fin], Lb[fin], rtol=0, atol=1e-13)
            assert np.all(O[np.isneginf(Lb)] == 0)


def check_block_mask_closed_forms(att_bs):
    rng = np.random.default_rng(22)
    B, H, N, d, block = 2, 3, 12, 4, 4
    q, k, v = (_rand(rng, B, H, N, d) for _ in range(3))
    nb = N // block
    # block-diagonal: every block of queries attends to its own block of keys only
    O, L = att_bs(q, k, v, 0.5, False, np.eye(nb, dtype=np.uint8), block)
    for r in range(nb):
        sl = slice(r * block, (r + 1) * block)
        Or, Lr = oracle.attention(q[:, :, sl], k[:, :, sl], v[:, :, sl], 0.5, False)
        np.testing.assert_allclose(O[:, :, sl], Or, atol=1e-14)
        np.testing.assert_allclose(L[:, :, sl], Lr, atol=1e-14)
    # an all-zero mask: nothing is visible anywhere
    O, L = att_bs(q, k, v, 0.5, True, np.zeros((nb, nb), np.uint8), block)
    assert np.all(O == 0) and np.all(np.isneginf(L))
    # lower block-triangle with causal equals plain causal attention
    O, L = att_bs(q, k, v, 0.5, True, np.tril(np.ones((nb, nb), np.uint8)), block)
    Oc, Lc = oracle.attention(q, k, v, 0.5, True)
    np.testing.assert_allclose(O, Oc, atol=1e-14)
    np.testing.assert_allclose(L, Lc, atol=1e-14)


def check_block_mask_invariants(att_bs):
    rng = np.random.default_rng(23)
    B, H, N, d, block = 2, 2, 10, 3, 3
    nb = -(-N // block)
    q, k, v = (_rand(rng, B, H, N, d) for _ in range(3))
    bm = (rng.random((B, H, nb, nb)) < 0.6).astype(np.uint8)
    O, L = att_bs(q, k, v, 0.4, False, bm, block)
    # keys and values that no query sees do not matter
    seen = oracle.expand_block_mask(bm[0, 0], N, block).any(axis=0)
    k2, v2 = k.copy(), v.copy()
    k2[0, 0, ~seen] += 100.0
    v2[0, 0, ~seen] -= 7.0
    O2, L2 = att_bs(q, k2, v2, 0.4, False, bm, block)
    np.testing.assert_allclose(O2[0, 0], O[0, 0], atol=1e-14)
    np.testing.assert_allclose(L2[0, 0], L[0, 0], atol=1e-14)
    # a mask shared by all heads equals the same mask given per head
    shared = bm[1, 0]
    Os, Ls = att_bs(q, k, v, 0.4, True, shared, block)
    Op, Lp = att_bs(q, k, v, 0.4, True, np.broadcast_to(shared, (B, H, nb, nb)).copy(), block)
    np.testing.assert_array_equal(Os, Op)
    np.testing.assert_array_equal(Ls, Lp)


BLOCK_MASK_PINS = (check_block_mask_brute_force, check_block_mask_closed_forms,
                   check_block_mask_invariants)


@pytest.mark.parametrize("pin", BLOCK_MASK_PINS, ids=lambda f: f.__name__)
def test_block_mask_pins(pin):
    pin(oracle.attention_block_sparse)


def test_expand_block_mask_ragged():
    bm = np.array([[1, 0], [0, 1]], np.uint8)
    e = oracle.expand_block_mask(bm, 5, 3)
    want = np.zeros((5, 5), bool)
    want[:3, :3] = True
    want[3:, 3:] = True
    np.testing.assert_array_equal(e, want)


def _mutant_mask_transposed(q, k, v, scale, causal, bm, block):
    # reads the block mask as [key block, query block]
    bm = np.asarray(bm)
    return oracle.attention_block_sparse(q, k, v, scale, causal, np.swapaxes(bm, -1, -2), block)


def _mutant_mask_ignored(q, k, v, scale, causal, bm, block):
    nb = np.asarray(bm).shape[-1]
    return oracle.attention_block_sparse(q, k, v, scale, causal, np.ones((nb, nb), np.uint8),
                                         block)


def _mutant_mask_shifted_block(q, k, v, scale, causal, bm, block):
    # block of an index taken as (index + 1) // block (an off-by-one)
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    B, H, N, d = q.shape
    bm = np.asarray(bm)
    nb = bm.shape[-1]
    full = np.broadcast_to(bm if bm.ndim == 4 else bm[None] if bm.ndim == 3 else bm[None, None],
                           (B, H, nb, nb))
    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))
    idx = np.minimum((np.arange(N) + 1) // block, nb - 1)
    for b in range(B):
        for h in range(H):
            vis = full[b, h][np.ix_(idx, idx)] != 0
            if causal:
                vis &= np.arange(N)[None, :] <= np.arange(N)[:, None]
            S = np.where(vis, scale * (q[b, h] @ k[b, h].T), -np.inf)
            m = S.max(1)
            dead = ~np.isfinite(m)
            ms = np.where(dead, 0.0, m)
            E = np.exp(S - ms[:, None])
            l = E.sum(1)
            O[b, h] = np.where(dead[:, None], 0.0, (E / np.where(dead, 1.0, l)[:, None]) @ v[b, h])
            L[b, h] = np.where(dead, -np.inf, ms + np.log(np.where(dead, 1.0, l)))
    return O, L


@pytest.mark.parametrize("mutant", [_mutant_mask_transposed, _mutant_mask_ignored,
                                    _mutant_mask_shifted_block], ids=lambda f: f.__name__)
def test_block_mask_pins_catch_planted_mistakes(mutant):
    caught = []
    for pin in BLOCK_MASK_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mutant)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, "no block-mask pin caught the planted mistake"


def test_block_sparse_rows_match_full():
    rng = np.random.default_rng(24)
    B, H, N, d, block = 2, 3, 23, 4, 5
    q, k, v = (_rand(rng, B, H, N, d) for _ in range(3))
    nb = -(-N // block)
    for bm in ((rng.random((nb, nb)) < 0.5).astype(np.uint8),
               (rng.random((H, nb, nb)) < 0.5).astype(np.uint8),
               (rng.random((B, H, nb, nb)) < 0.5).astype(np.uint8)):
        bm[..., 1, :] = 0  # block row 1 sees nothing
        for causal in (False, True):
            O, L = oracle.attention_block_sparse(q, k, v, 0.7, causal, bm, block)
            rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(N)]
            o, l = oracle.attention_block_sparse_rows(q, k, v, 0.7, causal, bm, rows, block)
            np.testing.assert_allclose(o.reshape(O.shape), O, atol=1e-14)
            assert np.array_equal(np.isneginf(l.reshape(L.shape)), np.isneginf(L))
            fin = np.isfinite(L)
            np.testing.assert_allclose(l.reshape(L.shape)[fin], L[fin], atol=1e-13)


# ----------------------------------------------------------------------------
# backward pins


def _phi(q, k, v, do, scale, causal):
    O, _ = oracle.attention(q, k, v, scale, causal)
    return float(np.sum(O * do))


def check_backward_finite_differences(bwd):
    """Central differences of <dO, O(Q, K, V)> through the pinned forward oracle."""
    rng = np.random.default_rng(31)
    for N, d, causal in ((4, 3, False), (5, 2, True), (3, 4, True)):
        q, k, v, do = (_rand(rng, 1, 2, N, d) for _ in range(4))
        scale = 0.8
        dq, dk, dv = bwd(q, k, v, do, scale, causal)
        h = 1e-6
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args = {"q": q, "k": k, "v": v}
                fp = _phi(**{**args, name: xp}, do=do, scale=scale, causal=causal)
                fm = _phi(**{**args, name: xm}, do=do, scale=scale, causal=causal)
                assert abs((fp - fm) / (2 * h) - g[idx]) <= 1e-7, (name, idx)


def check_backward_library(bwd):
    """torch autograd through its CPU attention in float64."""
    rng = np.random.default_rng(32)
    B, H, N, d = 2, 2, 19, 8
    q, k, v, do = (_rand(rng, B, H, N, d) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    for causal in (False, True):
        tq, tk, tv = (torch.from_numpy(a.copy()).requires_grad_() for a in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                               scale=scale)
        out.backward(torch.from_numpy(do))
        dq, dk, dv = bwd(q, k, v, do, scale, causal)
        np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


def check_backward_invariants(bwd):
    rng = np.random.default_rng(33)
    B, H, N, d = 1, 2, 15, 5
    q, k, v, do = (_rand(rng, B, H, N, d) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, do, 0.6, causal)
        # rows of P sum to 1: the value gradients add up to the output gradients
        np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)
        # rows of dS sum to 0: the key gradients add up to zero
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
        # shifting every key by one vector leaves P, hence every gradient, unchanged
        c = _rand(rng, 1, 1, 1, d)
        dq2, dk2, dv2 = bwd(q, k + c, v, do, 0.6, causal)
        np.testing.assert_allclose(dq2, dq, atol=1e-12)
        np.testing.assert_allclose(dk2, dk, atol=1e-12)
        np.testing.assert_allclose(dv2, dv, atol=1e-12)
        # linear in dO
        do2 = _rand(rng, B, H, N, d)
        g1 = bwd(q, k, v, do2, 0.6, causal)
        g2 = bwd(q, k, v, 2.0 * do - do2, 0.6, causal)
        for a, b_, c_ in zip((dq, dk, dv), g1, g2):
            np.testing.assert_allclose(c_, 2.0 * a - b_, atol=1e-12)


BACKWARD_PINS = (check_backward_finite_differences, check_backward_library,
                 check_backward_invariants)


@pytest.mark.parametrize("pin", BACKWARD_PINS, ids=lambda f: f.__name__)
def test_backward_pins(pin):
    pin(oracle.attention_backward)


def _mutant_bwd_no_d(q, k, v, do, scale, causal):
    # drops the row term sum_k P_ik dP_ik of the softmax Jacobian
    q, k, v, do = (np.asarray(a, np.float64) for a in (q, k, v, do))
    B, H, N, d = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            S = scale * (q[b, h] @ k[b, h].T)
            if causal:
                S[np.triu(np.ones((N, N), bool), 1)] = -np.inf
            E = np.exp(S - S.max(1, keepdims=True))
            P = E / E.sum(1, keepdims=True)
            dv[b, h] = P.T @ do[b, h]
            dS = P * (do[b, h] @ v[b, h].T)
            dq[b, h] = scale * dS @ k[b, h]
            dk[b, h] = scale * dS.T @ q[b, h]
    return dq, dk, dv


def _mutant_bwd_dk_transposed_operand(q, k, v, do, scale, causal):
    # dK from dS instead of dS^T (a transposed operand)
    q, k, v, do = (np.asarray(a, np.float64) for a in (q, k, v, do))
    B, H, N, d = q.shape
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, causal)
    for b in range(B):
        for h in range(H):
            S = scale * (q[b, h] @ k[b, h].T)
            if causal:
                S[np.triu(np.ones((N, N), bool), 1)] = -np.inf
            E = np.exp(S - S.max(1, keepdims=True))
            P = E / E.sum(1, keepdims=True)
            dP = do[b, h] @ v[b, h].T
            dS = P * (dP - (P * dP).sum(1, keepdims=True))
            dk[b, h] = scale * (dS @ q[b, h])
    return dq, dk, dv


def _mutant_bwd_no_scale(q, k, v, do, scale, causal):
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, causal)
    return dq / scale, dk, dv


@pytest.mark.parametrize("mutant", [_mutant_bwd_no_d, _mutant_bwd_dk_transposed_operand,
                                    _mutant_bwd_no_scale], ids=lambda f: f.__name__)
def test_backward_pins_catch_planted_mistakes(mutant):
    caught = []
    for pin in BACKWARD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mutant)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, "no backward pin caught the planted mistake"
