"""The oracle's constrained decoding (gowda.ai "Chapter 39 Decoding &
Speculative Sampling", section 39.3: a constraint is a mask; disallowed logits
become -inf before softmax, which conditions the distribution on the allowed
set; an empty allowed set is an invalid state) and the log-probability of the
drawn token, pinned against closed forms, brute-force enumeration of the
uniform and the conditioning identity."""
import math

import numpy as np
import pytest

from oracle.sampler import (ROW_EMPTY, ROW_OK, Params, allowed_from_words, draw_from,
                            log_p_tilde, mask_logits, sample_row, support)


def test_bit_layout():
    # token i is bit i % 32 of word i // 32
    words = np.array([0b101, 0, 1 << 31], dtype=np.uint32)
    assert np.flatnonzero(allowed_from_words(words, 96)).tolist() == [0, 2, 95]
    assert np.flatnonzero(allowed_from_words(words, 70)).tolist() == [0, 2]


def test_conditioning_closed_form():
    # logits (2, 1, 0) with token 0 disallowed at T = 1: p~ = (0, e/(1+e), 1/(1+e))
    l = np.array([2.0, 1.0, 0.0])
    s = support(mask_logits(l, [False, True, True]), Params(1.0))
    e = math.e
    assert np.allclose(s.p_tilde, [0.0, e / (1 + e), 1 / (1 + e)], rtol=1e-15, atol=0)
    assert math.isclose(log_p_tilde(mask_logits(l, [False, True, True]), s.keep, 1, 1.0),
                        1.0 - math.log(1 + e), rel_tol=1e-14)
    assert math.isclose(log_p_tilde(mask_logits(l, [False, True, True]), s.keep, 2, 1.0),
                        -math.log(1 + e), rel_tol=1e-14)


def test_conditioning_by_enumerating_the_uniform():
    # the masked draw's marginal equals softmax restricted to the allowed set,
    # counted over a fine grid of uniforms (no formula shared with the oracle)
    rng = np.random.default_rng(3)
    V = 12
    l = rng.normal(0, 1.5, V)
    allowed = rng.random(V) < 0.5
    allowed[3] = True
    T = 0.7
    s = support(mask_logits(l, allowed), Params(T))
    n = 200_000
    counts = np.zeros(V)
    for u in (np.arange(n) + 0.5) / n:
        counts[draw_from(s.p, s.keep, u)[0]] += 1
    expect = np.where(allowed, np.exp(l / T), 0.0)
    expect /= expect.sum()
    assert np.allclose(counts / n, expect, atol=2.0 / n)


def test_filters_see_the_masked_distribution():
    # min-p measures against the largest ALLOWED p: logits (5, 1, 0.5), token 0
    # disallowed, min_p 0.5: p2/p1 = e^-0.5 = 0.61 >= 0.5 keeps both; measured
    # against the unmasked max both would go
    l = mask_logits(np.array([5.0, 1.0, 0.5]), [False, True, True])
    assert np.flatnonzero(support(l, Params(1.0, min_p=0.5)).keep).tolist() == [1, 2]
    # top-k counts allowed tokens only
    l = mask_logits(np.array([5.0, 4.0, 3.0, 2.0]), [False, True, True, True])
    assert np.flatnonzero(support(l, Params(1.0, top_k=2)).keep).tolist() == [1, 2]
    # top-p over the conditioned distribution: (1, 1, 0, -inf masked) at T=1,
    # p~ = (e, e, 1)/(2e+1); top_p 0.5 keeps the top tie group {0, 1} only
    l = mask_logits(np.array([1.0, 1.0, 0.0, 9.0]), [True, True, True, False])
    assert np.flatnonzero(support(l, Params(1.0, top_p=0.5)).keep).tolist() == [0, 1]


def test_empty_and_nonfinite_masked():
    l = np.array([1.0, 2.0, -np.inf])
    assert sample_row(l, dict(temperature=1.0), 1, 0, 0, allowed=[False, False, True]).status == ROW_EMPTY
    assert sample_row(l, dict(temperature=1.0), 1, 0, 0, allowed=[False, False, False]).status == ROW_EMPTY
    # a disallowed NaN or +inf is replaced like any other logit
    l = np.array([np.nan, 0.5, np.inf, 0.0])
    r = sample_row(l, dict(temperature=1.0), 1, 0, 0, allowed=[False, True, False, True])
    assert r.status == ROW_OK and r.token in (1, 3)


def test_greedy_and_logprob_of_the_draw():
    l = np.array([3.0, 2.5, -1.0, 2.5])
    r = sample_row(l, dict(temperature=0.0), 1, 0, 0, allowed=[False, True, True, True])
    assert (r.token, r.logprob) == (1, 0.0)          # lowest id of the allowed maxima
    for step in range(20):
        r = sample_row(l, dict(temperature=0.9, top_k=3), 7, 2, step, allowed=[True, True, False, True])
        p = np.exp(np.array([3.0, 2.5, 2.5]) / 0.9)
        p /= p.sum()
        assert math.isclose(r.logprob, math.log(p[[0, 1, 3].index(r.token)]), rel_tol=1e-13)
