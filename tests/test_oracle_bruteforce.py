"""The oracle against brute force on tiny vocabularies and against closed forms.

The brute force here states each filter straight from its definition, with
loops over tokens and over candidate supports, so that a slip in the oracle's
sort/searchsorted formulation (a wrong side, an off-by-one, a tie split) shows.
"""
import itertools
import math

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle.sampler import Params, support, draw_from, sample_row, JOINT, SEQUENTIAL


def brute_kept(l, prm):
    V = len(l)
    T = prm.temperature
    e = [math.exp((x - max(l)) / T) for x in l]
    Z = sum(e)
    p = [x / Z for x in e]
    keep = [True] * V
    if 0 < prm.top_k < V:
        for i in range(V):
            greater = sum(1 for j in range(V) if l[j] > l[i])
            keep[i] = keep[i] and greater < prm.top_k
    topk_set = list(keep)
    if prm.top_p < 1:
        z_ref = 1.0
        if prm.mode == SEQUENTIAL and 0 < prm.top_k < V:
            z_ref = sum(p[i] for i in range(V) if topk_set[i])
        # Candidate supports: unions of whole tie groups, taken from the top
        # down. Pick the smallest one (at least one group) whose mass reaches
        # top_p * z_ref; if none does, everything stays.
        values = sorted(set(l), reverse=True)
        chosen = None
        for m in range(1, len(values) + 1):
            members = [i for i in range(V) if l[i] >= values[m - 1]]
            if sum(p[i] for i in members) >= prm.top_p * z_ref:
                chosen = set(members)
                break
        if chosen is None:
            chosen = set(range(V))
        keep = [keep[i] and i in chosen for i in range(V)]
    if 0 < prm.min_p < 1:
        pm = max(p)
        keep = [keep[i] and p[i] >= prm.min_p * pm for i in range(V)]
    return np.array(keep), np.array(p)


def tiny_rows(seed, n):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        V = int(rng.integers(1, 9))
        pool = rng.normal(0, 1.5, V)
        l = rng.choice(pool, V)          # draws with replacement force ties
        yield np.round(l, 2)


@pytest.mark.parametrize("mode", [JOINT, SEQUENTIAL])
def test_filters_match_brute_force(mode):
    checked = 0
    for l in tiny_rows(100 + mode, 150):
        V = len(l)
        for k in range(0, V + 1):
            for top_p in (0.0, 0.1, 0.35, 0.5, 0.8, 0.95, 1.0):
                for min_p in (0.0, 0.05, 0.3, 0.7):
                    for T in (0.5, 1.0, 2.0):
                        prm = Params(T, k, top_p, min_p, mode)
                        s = support(l, prm)
                        keep, p = brute_kept(list(l), prm)
                        if not np.array_equal(s.keep, keep):
                            # only a decision sitting on its cut may differ by rounding
                            assert min(s.margin_p, s.margin_m) < 1e-12, (l, prm)
                        else:
                            checked += 1
                        assert np.allclose(s.p, p, rtol=1e-12)
    assert checked > 10000


def test_kept_set_is_a_threshold_set():
    """Every filter keeps a set of the form {i : l_i >= tau}."""
    for l in tiny_rows(7, 300):
        for k, top_p, min_p in itertools.product((0, 1, 2, 5), (0.3, 0.9, 1.0), (0.0, 0.2)):
            s = support(l, Params(1.0, k, top_p, min_p))
            assert s.keep[np.argmax(l)]
            assert np.array_equal(s.keep, l >= s.threshold)


def test_draw_matches_interval_enumeration():
    rng = np.random.default_rng(9)
    for _ in range(300):
        V = int(rng.integers(1, 9))
        w = rng.random(V) * (rng.random(V) > 0.3)
        w[rng.integers(V)] += 0.1
        keep = rng.random(V) > 0.3
        keep[np.argmax(w)] = True
        kept = [i for i in range(V) if keep[i]]
        Z = sum(w[i] for i in kept)
        # interval of each kept token, in id order, by direct enumeration
        ends, run = [], 0.0
        for i in kept:
            ends.append((i, run, run + w[i]))
            run += w[i]
        us = list(rng.random(40)) + [0.0, 1 - 2 ** -32] + [lo / Z for _, lo, _ in ends]
        for u in us:
            want = None
            for i, lo, hi in ends:
                if lo <= u * Z < hi:
                    want = i
                    break
            if want is None:              # only past the last total by rounding
                want = max(i for i in kept if w[i] > 0)
            got, margin = draw_from(w, keep, u)
            assert got == want, (w, keep, u)
            assert margin >= 0


def test_speculative_output_is_exactly_p():
    """P(out = y) = sum_x q(x) a(x) 1{x=y} + P(reject) r(y) equals p(y) (P1
    'Speculative decoding'; P2 section 39.4), and sum (p-q)+ = 1 - sum min(p,q)
    (Exercise 39.2)."""
    rng = np.random.default_rng(11)
    for _ in range(500):
        V = int(rng.integers(2, 17))
        p = rng.dirichlet(np.ones(V) * rng.uniform(0.2, 3))
        q = rng.dirichlet(np.ones(V) * rng.uniform(0.2, 3))
        a = np.array([oracle.accept_probability(p, q, x) for x in range(V)])
        r = oracle.residual(p, q)
        assert math.isclose(r.sum(), 1 - oracle.acceptance_probability(p, q), abs_tol=1e-15)
        reject = float(np.sum(q * (1 - a)))
        out = q * a + (reject * r / r.sum() if r.sum() > 0 else 0)
        assert np.allclose(out, p, atol=1e-15)


def test_sampler_chi_square():
    """Draws over many rows (the Philox row index varies) follow p~."""
    l = np.array([1.0, 0.2, 0.7, -0.4, 0.7, -2.0, 0.3, -1.0, 1.0, 0.0])
    prm = Params(0.9, top_k=6, top_p=0.9, min_p=0.05)
    s = support(l, prm)
    n = 30000
    toks = np.array([sample_row(l, prm, 99, b, 4).token for b in range(n)])
    obs = np.bincount(toks, minlength=len(l))
    assert (obs[~s.keep] == 0).all()
    exp = s.p_tilde[s.keep] * n
    assert stats.chisquare(obs[s.keep], exp).pvalue > 1e-3


def test_speculative_marginal_with_a_different_draft():
    """The first emitted token follows the target p~ whatever the draft (the
    check the first page names, with more samples): the draft token is drawn
    from q by the sampler itself, then verified."""
    tgt_l = np.log(np.array([0.2, 0.5, 0.3]))
    dft_l = np.log(np.array([0.5, 0.3, 0.2]))
    n = 30000
    first = np.empty(n, dtype=int)
    for b in range(n):
        x = sample_row(dft_l, Params(1.0), 31, b, 7).token
        res = oracle.spec_verify_row(np.stack([tgt_l, tgt_l]), dft_l[None, :], [x],
                                     Params(1.0), 31, b, 7)
        first[b] = res.tokens[0]
    obs = np.bincount(first, minlength=3)
    assert stats.chisquare(obs, np.array([0.2, 0.5, 0.3]) * n).pvalue > 1e-3


def test_greedy_speculation_equals_greedy_decoding():
    rng = np.random.default_rng(13)
    for b in range(200):
        K, V = int(rng.integers(1, 6)), int(rng.integers(2, 40))
        tgt = rng.normal(0, 1, (K + 1, V))
        dft = rng.normal(0, 1, (K, V))
        argmaxes = [int(np.argmax(tgt[j])) for j in range(K + 1)]
        xs = [argmaxes[j] if rng.random() < 0.7 else int(rng.integers(V)) for j in range(K)]
        res = oracle.spec_verify_row(tgt, dft, xs, Params(0.0), 1, b, 0)
        n = res.n_accepted
        assert res.tokens[: n + 1] == argmaxes[: n + 1]
        assert all(t == -1 for t in res.tokens[n + 1:])
        assert all(xs[j] == argmaxes[j] for j in range(n))
        assert n == K or xs[n] != argmaxes[n]


def test_bad_rows():
    assert sample_row(np.array([0.0, np.nan]), Params(1.0), 0, 0, 0).status == oracle.ROW_NONFINITE
    assert sample_row(np.array([0.0, np.inf]), Params(1.0), 0, 0, 0).status == oracle.ROW_NONFINITE
    assert sample_row(np.array([-np.inf] * 3), Params(1.0), 0, 0, 0).status == oracle.ROW_EMPTY
    r = sample_row(np.array([-np.inf, 1.0, -np.inf]), Params(1.0, top_k=2), 0, 0, 0)
    assert r.status == oracle.ROW_OK and r.token == 1 and r.support.kept_count == 1
    with pytest.raises(oracle.InvalidParams):
        sample_row(np.zeros(3), Params(-1.0), 0, 0, 0)
    with pytest.raises(oracle.InvalidParams):
        sample_row(np.zeros(3), Params(1.0, top_p=-0.1), 0, 0, 0)
    with pytest.raises(oracle.InvalidParams):
        sample_row(np.zeros(3), Params(float("nan")), 0, 0, 0)
    with pytest.raises(oracle.InvalidParams):
        sample_row(np.zeros(3), Params(1e-31), 0, 0, 0)
