"""The oracle against the numbers the pages print (tests/golden/worked_examples.json)."""
import json
import math
import os

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle.sampler import Params, support, sample_row, accept_probability, residual

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def kept_ids(s):
    return np.flatnonzero(s.keep).tolist()


def test_min_p_cut_high_confidence():
    g = GOLD["min_p_cut_high_confidence"]
    for row in g["rows"]:
        p = np.array(row["p"])
        s = support(np.log(p), Params(1.0, min_p=g["min_p"]))
        assert kept_ids(s) == row["kept"]
        # the cut sits at min_p * p_max = 0.09
        assert math.isclose(g["min_p"] * s.p.max(), 0.09, rel_tol=1e-12)


def test_min_p_cut_low_confidence():
    g = GOLD["min_p_cut_low_confidence"]
    p = np.array([g["p_head"]] * g["n_head"] + g["p_tail"])
    assert math.isclose(p.sum(), 1.0, rel_tol=1e-12)
    s = support(np.log(p), Params(1.0, min_p=g["min_p"]))
    assert s.keep[: g["n_head"]].all()
    assert s.keep[g["n_head"]:].tolist() == g["kept_tail"]
    assert s.kept_count >= 20          # "dozens" of reasonable choices survive


@pytest.mark.parametrize("case", GOLD["temperature_odds"]["cases"])
def test_temperature_odds_law(case):
    logits = np.array([math.log(case["ratio_at_T1"]), 0.0, -1.0, -3.0])
    s = support(logits, Params(case["T"]))
    assert math.isclose(s.p_tilde[0] / s.p_tilde[1], case["ratio"], rel_tol=1e-12)


def test_temperature_limits():
    """T -> 0 concentrates on the favourite; T -> inf tends to uniform."""
    rng = np.random.default_rng(7)
    for _ in range(50):
        l = rng.normal(0, 2, 64)
        l[rng.integers(64)] = l.max() + 0.5          # unique max with a gap
        s = support(l, Params(1e-3))
        assert np.delete(s.p_tilde, np.argmax(l)).max() < 1e-100
        for row in range(4):
            assert sample_row(l, Params(1e-3), 11, row, 0).token == int(np.argmax(l))
        assert sample_row(l, Params(0.0), 11, 0, 0).token == int(np.argmax(l))
        hot = support(l, Params(1e9)).p_tilde
        assert np.allclose(hot, 1 / 64, rtol=1e-6)


def test_nucleus_eight_words():
    g = GOLD["nucleus_eight_words"]
    l = np.array(g["logits"])
    s = support(l, Params(1.0, top_p=0.8))
    assert kept_ids(s) == g["top_p_0_8_kept"]
    assert abs(s.p[0] - g["girl_share_about"]) < 0.01
    assert s.p[0] < 0.8 <= s.p[0] + s.p[1]       # girl alone short, girl+boy past 0.8
    assert kept_ids(support(l, Params(1.0, top_k=3))) == g["top_k_3_kept"]
    # Draws over many rows follow p~ on {girl, boy}
    n = 20000
    toks = np.array([sample_row(l, Params(1.0, top_p=0.8), 5, b, 3).token for b in range(n)])
    assert set(np.unique(toks)) <= {0, 1}
    obs = np.bincount(toks, minlength=2)[:2]
    exp = s.p_tilde[:2] * n
    assert stats.chisquare(obs, exp).pvalue > 1e-3


def test_nucleus_single_token():
    g = GOLD["nucleus_one_token"]
    rest = (1 - g["p_top"]) / 99
    p = np.array([g["p_top"]] + [rest] * 99)
    s = support(np.log(p), Params(1.0, top_p=g["top_p"]))
    assert s.kept_count == g["kept_count"]


def test_exercise_39_1():
    g = GOLD["exercise_39_1"]
    p = np.array(g["p"])
    l = np.log(p)
    sk = support(l, Params(1.0, top_k=g["top_k"]), p=p)
    sp = support(l, Params(1.0, top_p=g["top_p"]), p=p)
    sm = support(l, Params(1.0, min_p=g["min_p"]), p=p)
    assert kept_ids(sk) == g["top_k_kept"]
    assert kept_ids(sp) == g["top_p_kept"]
    assert kept_ids(sm) == g["min_p_kept"]      # 0.15 >= 0.3 * 0.5 holds in binary64
    assert sm.margin_m == 0.0                   # ... exactly on the cut
    peaks = {"k": sk.p_tilde.max(), "p": sp.p_tilde.max(), "m": sm.p_tilde.max()}
    assert math.isclose(peaks["k"], 2 / 3) and math.isclose(peaks["p"], 2 / 3)
    assert peaks["m"] < peaks["k"]


def test_acceptance_table():
    for row in GOLD["acceptance_table"]["rows"]:
        p_t = np.array([row["p"], 1 - row["p"]])
        q_t = np.array([row["q"], 1 - row["q"]])
        assert math.isclose(accept_probability(p_t, q_t, 0), row["accept"], rel_tol=1e-12)


def test_three_token_example():
    g = GOLD["three_token_example"]
    p, q = np.array(g["p"]), np.array(g["q"])
    assert math.isclose(accept_probability(p, q, 0), g["accept_token0"], rel_tol=1e-12)
    assert accept_probability(p, q, 1) == g["accept_token1"]
    r = residual(p, q)
    assert np.allclose(r, g["residual"], atol=1e-15)
    assert np.allclose(r / r.sum(), g["residual_normalised"], atol=1e-15)
    assert math.isclose(oracle.acceptance_probability(p, q), g["total_acceptance"], rel_tol=1e-12)
    via_accept = q[1] * accept_probability(p, q, 1)
    via_reject = (1 - oracle.acceptance_probability(p, q)) * (r / r.sum())[1]
    assert math.isclose(via_accept, g["p_token1_via_accept"], rel_tol=1e-12)
    assert math.isclose(via_reject, g["p_token1_via_reject"], rel_tol=1e-12)


def test_equal_distributions():
    g = GOLD["equal_distributions"]
    rng = np.random.default_rng(3)
    for _ in range(20):
        p = rng.dirichlet(np.ones(12))
        assert math.isclose(oracle.acceptance_probability(p, p), g["acceptance"], rel_tol=1e-12)
        assert residual(p, p).sum() == g["residual_mass"]
        for x in range(12):
            assert accept_probability(p, p, x) == 1.0


def _block_inputs(alphas):
    """Per position j: target p_j = (alpha_j, 1 - alpha_j), draft q_j = (1, 0).
    The draft always proposes token 0, which is kept with probability alpha_j,
    so sum_x min(p_j, q_j) = alpha_j."""
    K = len(alphas)
    tgt = np.empty((K + 1, 2))
    dft = np.empty((K, 2))
    for j, a in enumerate(alphas):
        tgt[j] = [math.log(a), math.log(1 - a)]
        dft[j] = [0.0, -np.inf]
    tgt[K] = [0.0, 0.0]
    return tgt, dft, [0] * K


def test_exercise_39_3_by_simulation():
    g = GOLD["exercise_39_3"]
    assert math.isclose(oracle.expected_accepted_prefix(g["alphas"]), g["expected_accepted"])
    tgt, dft, xs = _block_inputs(g["alphas"])
    n = 20000
    acc = np.array([oracle.spec_verify_row(tgt, dft, xs, Params(1.0), 17, b, 0).n_accepted
                    for b in range(n)])
    se = acc.std() / math.sqrt(n)
    assert abs(acc.mean() - g["expected_accepted"]) < 4 * se


def test_expected_tokens_per_block():
    g = GOLD["expected_tokens_per_block"]
    a, K = g["alpha"], g["K"]
    closed = (1 - a ** (K + 1)) / (1 - a)
    series = sum((i + 1) * a ** i * (1 - a) for i in range(K)) + (K + 1) * a ** K
    assert math.isclose(closed, g["expected_tokens"]) and math.isclose(series, closed)
    tgt, dft, xs = _block_inputs([a] * K)
    n = 20000
    emitted = np.array([oracle.spec_verify_row(tgt, dft, xs, Params(1.0), 23, b, 1).n_accepted + 1
                        for b in range(n)])
    se = emitted.std() / math.sqrt(n)
    assert abs(emitted.mean() - g["expected_tokens"]) < 4 * se
