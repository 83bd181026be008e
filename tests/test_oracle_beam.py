"""Pins of the oracle's beam-search step (gowda.ai chapter 39, section 39.1,
eq. 39.1 and Listing 39.1; scratchllm.com "Beam search"), each against
something other than the oracle's own enumeration."""
import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import log_softmax

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def test_two_step_example_beam_beats_greedy():
    """The page's example: step 1 gives A 0.6 and B 0.4; after A the next
    token is "continue" 0.4 or one of two others at 0.3; after B it is "end"
    at 0.9 (the page leaves the other 0.1 open: here spread evenly over the
    three other continuations, which keeps "end" the best). Greedy finds
    probability 0.24, a beam of 2 finds B, end with 0.36."""
    g = GOLD["beam_two_steps"]
    vocab = ["A", "B", "continue", "other1", "other2", "end"]
    ix = {w: i for i, w in enumerate(vocab)}

    def probs(d):
        p = np.zeros(len(vocab))
        for w, q in d.items():
            p[ix[w]] = q
        return p

    after_b = probs(g["after_B"])
    rest = 1.0 - after_b.sum()
    for w in ("continue", "other1", "other2"):
        after_b[ix[w]] = rest / 3
    table = {(): probs(g["step1"]), (ix["A"],): probs(g["after_A"]), (ix["B"],): after_b}

    def next_logits(prefix):
        with np.errstate(divide="ignore"):
            return np.log(table[tuple(prefix)])

    greedy = oracle.beam_search(next_logits, (), 2, 1)
    assert [vocab[t] for t in greedy[0][0]] == ["A", "continue"]
    assert abs(np.exp(greedy[0][1]) - g["greedy_probability"]) < 1e-12
    beams = oracle.beam_search(next_logits, (), 2, 2)
    assert [vocab[t] for t in beams[0][0]] == g["beam_best"]
    assert abs(np.exp(beams[0][1]) - g["beam_probability"]) < 1e-12


def test_beam_of_v_to_the_t_is_exhaustive():
    """With B = V^t the search keeps every sequence (P2: exact for B = V^t):
    after t steps the beams are all V^t sequences with their log-probability
    sums, which brute force over the sequences gives independently
    (scipy's log_softmax per position)."""
    V, t = 3, 3
    rng = np.random.default_rng(0)
    table = {}

    def next_logits(prefix):
        key = tuple(prefix)
        if key not in table:
            table[key] = rng.normal(0, 2, V)
        return table[key]

    beams = oracle.beam_search(next_logits, (), t, V ** t)
    got = {p: s for p, s in beams}
    assert len(got) == V ** t
    for seq in itertools.product(range(V), repeat=t):
        want = sum(log_softmax(next_logits(seq[:k]))[seq[k]] for k in range(t))
        assert abs(got[seq] - want) < 1e-12, seq
    scores = [s for _, s in beams]
    assert scores == sorted(scores, reverse=True)


def test_shift_of_a_beam_row_changes_nothing():
    rng = np.random.default_rng(1)
    v = rng.normal(0, 1.5, (4, 50))
    s = rng.normal(-3, 1, 4)
    a = oracle.beam_step(v, s, 4)
    v2 = v.copy()
    v2[2] += 17.25
    b = oracle.beam_step(v2, s, 4)
    assert np.array_equal(a.parent, b.parent) and np.array_equal(a.token, b.token)
    np.testing.assert_allclose(a.score, b.score, rtol=0, atol=1e-12)


def test_equal_scores_keep_enumeration_order():
    """Two identical beams: the first one's candidates come first, and within
    a beam equal logits go in token order."""
    row = np.array([1.0, 3.0, 3.0, 0.0])
    r = oracle.beam_step(np.stack([row, row]), [0.5, 0.5], 4)
    assert list(zip(r.parent, r.token)) == [(0, 1), (0, 2), (1, 1), (1, 2)]


def test_dead_beams_and_bad_rows():
    rng = np.random.default_rng(2)
    v = rng.normal(0, 1, (3, 10))
    r = oracle.beam_step(v, [-np.inf, 0.0, -np.inf], 3)
    assert r.status == oracle.ROW_OK and set(r.parent) == {1}
    r = oracle.beam_step(v, [-np.inf] * 3, 3)
    assert r.status == oracle.ROW_EMPTY
    v[1, 4] = np.nan
    assert oracle.beam_step(v, [0.0] * 3, 3).status == oracle.ROW_NONFINITE
    dead = np.full((2, 5), -np.inf)
    dead[1] = [0.0, 1.0, 2.0, 3.0, 4.0]
    r = oracle.beam_step(dead, [0.0, 0.0], 2)
    assert list(r.parent) == [1, 1] and list(r.token) == [4, 3]
