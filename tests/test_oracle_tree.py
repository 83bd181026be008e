"""Pins of the oracle's tree (multi-candidate) verify step: exactness of the
output distribution, agreement with plain speculative decoding where the
draft equals the target, greedy decoding by hand, and invalid inputs."""
import numpy as np
import pytest
from scipy.stats import chisquare

import oracle


def test_first_token_is_distributed_as_the_target():
    """Three candidates drawn independently from q~ at the root, each kept
    with the residual rule: the first emitted token follows p~ (the property
    that makes speculative decoding exact, P2 section 39.4), here with a
    top-k filter on both distributions. 20000 independent steps."""
    rng = np.random.default_rng(11)
    V, m = 6, 3
    prm = {"temperature": 0.8, "top_k": 4}
    tgt_root = np.array([1.0, 0.2, -0.5, 0.7, -2.0, 0.1])
    dft_root = np.array([0.1, 1.2, 0.3, -0.4, 0.8, -1.0])
    p = oracle.support(tgt_root, oracle.Params.of(prm)).p_tilde
    q = oracle.support(dft_root, oracle.Params.of(prm)).p_tilde
    N = m + 1
    parent = [-1] + [0] * m
    target = np.stack([tgt_root] + [rng.normal(0, 1, V) for _ in range(m)])
    draft = np.stack([dft_root] + [rng.normal(0, 1, V) for _ in range(m)])
    counts = np.zeros(V)
    trials = 20000
    for t in range(trials):
        toks = [0] + list(rng.choice(V, m, p=q))
        r = oracle.tree_verify_row(target, draft, parent, toks, prm, 7, t % 4096, t // 4096)
        counts[r.tokens[0]] += 1
    expected = p * trials
    keep = expected > 0
    assert counts[~keep].sum() == 0
    assert chisquare(counts[keep], expected[keep]).pvalue > 1e-3


def test_draft_equal_to_target_keeps_the_first_child_everywhere():
    """With q~ = p~ every first child is kept (acceptance 1), so the output is
    the path of first children and one draw at its leaf."""
    rng = np.random.default_rng(2)
    V = 50
    parent = [-1, 0, 0, 1, 1, 3]
    rows = rng.normal(0, 1, (6, V))
    toks = [0, 7, 9, 3, 4, 11]
    r = oracle.tree_verify_row(rows, rows, parent, toks, {"temperature": 1.0}, 3, 0, 0)
    assert r.path == [1, 3, 5] and r.tokens[:3] == [7, 3, 11] and len(r.tokens) == 4


def test_greedy_by_hand():
    """Root argmax is token 1: of the root's children (tokens 2, 1) the second
    is kept; its argmax 0 has no child, so 0 is emitted and the step ends."""
    V = 3
    target = np.array([[0.0, 2.0, 1.0], [5.0, 0.0, 0.0], [0.0, 0.0, 9.0]])
    r = oracle.tree_verify_row(target, target, [-1, 0, 0], [0, 2, 1], {"temperature": 0.0}, 1, 0, 0)
    assert r.tokens == [1, 2] and r.path == [2]
    # no child holds the argmax: emit it and stop
    r = oracle.tree_verify_row(target, target, [-1, 0, 0], [0, 2, 0], {"temperature": 0.0}, 1, 0, 0)
    assert r.tokens == [1] and r.path == []


def test_invalid_inputs():
    rng = np.random.default_rng(3)
    t = rng.normal(0, 1, (3, 10))
    prm = {"temperature": 1.0}
    assert oracle.tree_verify_row(t, t, [-1, 1, 0], [0, 1, 2], prm, 1, 0, 0).status == oracle.INVALID_TREE
    assert oracle.tree_verify_row(t, t, [-1, 0, 0], [0, 1, 10], prm, 1, 0, 0).status == oracle.ROW_BADTOKEN
    bad = t.copy(); bad[2, 4] = np.nan
    assert oracle.tree_verify_row(bad, t, [-1, 0, 0], [0, 1, 2], prm, 1, 0, 0).status == oracle.ROW_NONFINITE
    # a leaf's draft row is never read
    assert oracle.tree_verify_row(t, bad, [-1, 0, 0], [0, 1, 2], prm, 1, 0, 0).status == oracle.ROW_OK
