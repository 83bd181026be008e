"""Pins of the oracle's decision margins, on which the parity rule excuses a
GPU/oracle mismatch (oracle/parity.py). Each margin is the distance of one
decision from its cut, so it is pinned by behaviour, not by its formula: moving
the knob that the decision compares (top_p, min_p, the uniform) by slightly
less than the margin must change nothing, and by slightly more, in the right
direction, must change the outcome. Tiny vocabularies with forced ties, both
filter modes, plus a brute-force recount of the top-p margin from the set
definitions.

Pages: gowda.ai "Chapter 39", section 39.2 (top-p keeps the smallest head
reaching top_p, min-p compares with min_p times the largest p) and section
39.4 (eq. 39.3: accept iff u < min(1, p/q); eq. 39.4: residual draw);
legost.in "Choosing the next word", "Where the randomness comes from" (the
inverse-CDF walk over the kept tokens).
"""
import numpy as np
import pytest

import oracle
from oracle.sampler import Params, draw_from, spec_verify_row, support

IN, OUT = 1.0 - 1e-6, 1.0 + 1e-6   # just inside / just past the margin


def rows_and_params(seed, n):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        V = int(rng.integers(2, 9))
        l = rng.normal(0, 1.5, V)
        if rng.random() < 0.5:                    # forced ties
            l = np.round(l * 2) / 2
        T = float(rng.choice([0.5, 1.0, 2.0]))
        k = int(rng.integers(0, V + 1))
        p = float(rng.uniform(0.05, 0.95))
        m = float(rng.choice([0.0, rng.uniform(0.01, 0.6)]))
        mode = int(rng.integers(0, 2))
        yield l, Params(T, k, p, m, mode)


def with_(prm, **kw):
    d = dict(temperature=prm.temperature, top_k=prm.top_k, top_p=prm.top_p, min_p=prm.min_p,
             mode=prm.mode)
    d.update(kw)
    return Params(**d)


def test_margin_p_is_the_distance_to_the_nearest_top_p_flip():
    checked = 0
    for l, prm in rows_and_params(1, 3000):
        s = support(l, prm)
        mp = s.margin_p
        if not np.isfinite(mp) or mp < 1e-9:
            continue
        lo, hi = prm.top_p - mp * OUT, prm.top_p + mp * OUT
        if lo < 0.0 or hi >= 1.0:
            continue
        for d in (-mp * IN, mp * IN):             # inside: the kept set stays
            assert np.array_equal(support(l, with_(prm, top_p=prm.top_p + d)).keep, s.keep), \
                (l, prm, d)
        flips = [not np.array_equal(support(l, with_(prm, top_p=t)).keep, s.keep)
                 for t in (lo, hi)]
        assert any(flips), (l, prm, mp)           # past it: some top-p decision turns
        checked += 1
    assert checked > 300


def test_margin_m_is_the_distance_to_the_nearest_min_p_flip():
    checked = 0
    for l, prm in rows_and_params(2, 6000):
        if prm.min_p == 0.0:
            continue
        s = support(l, prm)
        mm = s.margin_m
        if not np.isfinite(mm) or mm < 1e-9:
            continue
        lo, hi = prm.min_p - mm * OUT, prm.min_p + mm * OUT
        if lo <= 0.0 or hi >= 1.0:
            continue
        for d in (-mm * IN, mm * IN):
            assert np.array_equal(support(l, with_(prm, min_p=prm.min_p + d)).keep, s.keep), \
                (l, prm, d)
        flips = [not np.array_equal(support(l, with_(prm, min_p=t)).keep, s.keep)
                 for t in (lo, hi)]
        assert any(flips), (l, prm, mm)
        checked += 1
    assert checked > 300


def test_margin_p_by_enumeration_of_tie_groups():
    """The top-p margin recounted from the set definitions: for every token,
    the mass of the tokens with a strictly larger logit (an O(V^2) double
    loop, no sort), its distance from top_p * Z_ref, over the tokens whose
    top-p decision can change the kept set."""
    for l, prm in rows_and_params(3, 1500):
        s = support(l, prm)
        V = l.size
        p = s.p
        k_keep = [(0 < prm.top_k < V) is False or sum(l[j] > l[i] for j in range(V)) < prm.top_k
                  for i in range(V)]
        z_ref = 1.0
        if prm.mode == oracle.SEQUENTIAL and 0 < prm.top_k < V:
            z_ref = sum(p[i] for i in range(V) if k_keep[i])
        m_keep = [not (0 < prm.min_p < 1) or p[i] >= prm.min_p * p.max() for i in range(V)]
        best = np.inf
        for i in range(V):
            if l[i] == l.max() or not k_keep[i] or not m_keep[i]:
                continue
            above = sum(p[j] for j in range(V) if l[j] > l[i])
            best = min(best, abs(above - prm.top_p * z_ref) / z_ref)
        assert (best == np.inf and s.margin_p == np.inf) or abs(best - s.margin_p) <= 1e-12, \
            (l, prm, best, s.margin_p)


def test_draw_margin_is_the_distance_to_the_interval_end():
    rng = np.random.default_rng(4)
    checked = 0
    for _ in range(4000):
        V = int(rng.integers(1, 9))
        w = rng.random(V) * (rng.random(V) < 0.8)
        keep = w > 0
        if not keep.any():
            continue
        u = float(rng.random())
        tok, m = draw_from(w, keep, u)
        if m < 1e-9:
            continue
        for d in (-m * IN, m * IN):
            if 0.0 <= u + d < 1.0:
                assert draw_from(w, keep, u + d)[0] == tok, (w, u, d)
        outs = [draw_from(w, keep, x)[0] != tok for x in (u - m * OUT, u + m * OUT)
                if 0.0 <= x < 1.0]
        # past the margin the token turns, unless the near end is 0 or 1
        near_end = min(u, 1.0 - u) <= m * OUT
        assert any(outs) or near_end, (w, u, m)
        checked += 1
    assert checked > 2000


def test_verify_decisions_accept_and_draw():
    """Decision.accept is the distance of u0 from a = min(1, p~/q~) at the
    position consulted; Decision.draw the distance of u1 from the residual
    draw's interval end (uniforms substituted through the test hook)."""
    rng = np.random.default_rng(5)
    checked_a = checked_d = 0
    for _ in range(1500):
        V, K = int(rng.integers(2, 7)), int(rng.integers(1, 4))
        tgt = rng.normal(0, 1.2, (K + 1, V))
        dft = tgt[:K] + rng.normal(0, 1.0, (K, V))
        xs = rng.integers(0, V, K)
        prm = {"temperature": float(rng.choice([0.7, 1.0])), "top_k": int(rng.integers(0, V + 1))}
        U = rng.random((K + 1, 2))
        r = spec_verify_row(tgt, dft, xs, prm, 0, 0, 0, uniforms=U)
        j = r.n_accepted if r.n_accepted < K else None
        if j is None:
            continue
        d = r.margins[j]                      # the rejecting position
        if d.accept > 1e-9 and U[j, 0] + d.accept * OUT < 1.0:
            U2 = U.copy()
            U2[j, 0] -= d.accept * IN         # still at or above a: still rejected
            assert spec_verify_row(tgt, dft, xs, prm, 0, 0, 0, uniforms=U2).n_accepted == j
            U2[j, 0] = U[j, 0] - d.accept * OUT   # below a: accepted now
            if U2[j, 0] >= 0.0:
                assert spec_verify_row(tgt, dft, xs, prm, 0, 0, 0, uniforms=U2).n_accepted > j
                checked_a += 1
        if d.draw > 1e-9:
            tok = r.tokens[j]
            for s_ in (-1, 1):
                U2 = U.copy()
                U2[j, 1] += s_ * d.draw * IN
                if 0.0 <= U2[j, 1] < 1.0:
                    assert spec_verify_row(tgt, dft, xs, prm, 0, 0, 0, uniforms=U2).tokens[j] == tok
            turned = []
            for s_ in (-1, 1):
                U2 = U.copy()
                U2[j, 1] += s_ * d.draw * OUT
                if 0.0 <= U2[j, 1] < 1.0:
                    turned.append(spec_verify_row(tgt, dft, xs, prm, 0, 0, 0,
                                                  uniforms=U2).tokens[j] != tok)
            if turned:
                assert any(turned) or min(U[j, 1], 1 - U[j, 1]) <= d.draw * OUT
                checked_d += 1
    assert checked_a > 50 and checked_d > 50
