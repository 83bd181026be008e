"""Pins of the oracle's repetition penalty (legost.in "Choosing the next word",
section "The repetition penalty": every token of the look-back window has its
logit divided by r when positive, multiplied by r otherwise), each against
something other than the oracle's own formula."""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def test_penalty_one_changes_nothing():
    rng = np.random.default_rng(0)
    l = rng.normal(0, 3, 500)
    out = oracle.repetition_penalty(l, rng.integers(0, 500, 64), 1.0)
    assert np.array_equal(out, l)


def test_window_is_a_set_and_padding_is_ignored():
    """Repeats and order in the window do not matter; ids outside [0, V) are
    padding."""
    rng = np.random.default_rng(1)
    V = 300
    l = rng.normal(0, 2, V).astype(np.float32).astype(np.float64)
    base = rng.choice(V, 20, replace=False)
    a = oracle.repetition_penalty(l, base, 1.3)
    noisy = np.concatenate([base, base[::-1], [-1, V, V + 7, -100], base[:5]])
    rng.shuffle(noisy)
    b = oracle.repetition_penalty(l, noisy, 1.3)
    assert np.array_equal(a, b)
    untouched = np.setdiff1d(np.arange(V), base)
    assert np.array_equal(a[untouched], l[untouched])


def test_both_branches_lower_the_logit():
    """For r > 1 a positive logit moves towards zero and a non-positive one
    away from it: every penalised logit is at most the original, zero stays."""
    l = np.array([5.0, 0.25, 0.0, -0.0, -0.5, -7.0, -np.inf])
    out = oracle.repetition_penalty(l, range(l.size), 1.7)
    assert np.all(out <= l)
    assert np.all(out[:2] > 0) and np.all(out[:2] < l[:2])
    assert out[2] == 0.0 and out[3] == 0.0
    assert np.all(out[4:6] < l[4:6]) and out[6] == -np.inf


def test_hand_computed_example_changes_the_greedy_token():
    """Logits (3.0, 2.9, 1.0) with token 0 in the window and r = 1.1: 3.0 / 1.1
    = 2.7272... falls below 2.9, so greedy decoding moves to token 1."""
    l = np.array([3.0, 2.9, 1.0])
    assert oracle.sample_row(l, {"temperature": 0.0}, 1, 0, 0).token == 0
    r = oracle.sample_row(l, {"temperature": 0.0}, 1, 0, 0, history=[0], penalty=1.1)
    assert r.token == 1
    out = oracle.repetition_penalty(l, [0], 1.1)
    assert abs(out[0] - 2.727272727) < 1e-6


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_whole_window_equals_a_temperature(sign):
    """With every token in the window and every logit of one sign, the
    penalised softmax is a softmax at another temperature: z / r at T is z at
    T * r (all z > 0), z * r at T is z at T / r (all z <= 0). Compares the
    renormalised distributions p~ of the full chain (float32 rounding of the
    penalised logits is the only difference)."""
    rng = np.random.default_rng(2)
    V, r, T = 400, 1.25, 0.8
    l = (sign * rng.uniform(0.05, 6.0, V)).astype(np.float32).astype(np.float64)
    prm = {"temperature": T, "top_k": 50, "top_p": 0.9}
    pen = oracle.sample_row(l, prm, 3, 0, 0, history=range(V), penalty=r)
    t_eq = T * r if sign > 0 else T / r
    ref = oracle.sample_row(l, dict(prm, temperature=t_eq), 3, 0, 0)
    assert pen.support.kept_count == ref.support.kept_count
    np.testing.assert_allclose(pen.support.p_tilde, ref.support.p_tilde, rtol=1e-5, atol=1e-12)


def test_bf16_rounding_matches_torch():
    """round_to_element(bf16) against torch's float32 -> bfloat16 conversion
    (round to nearest even), including exact halfway cases of both parities."""
    rng = np.random.default_rng(3)
    f = rng.normal(0, 50, 4000).astype(np.float32)
    bits = f.view(np.uint32)
    halfway = ((bits & 0xFFFF0000) | 0x8000).astype(np.uint32).view(np.float32)
    x = np.concatenate([f, halfway, np.array([0.0, -0.0, 3.3e38, -3.3e38], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    got = oracle.round_to_element(x.astype(np.float64), "bf16")
    assert np.array_equal(got, want)


def test_penalised_bf16_logits_stay_bf16_values():
    rng = np.random.default_rng(4)
    bits = (rng.normal(0, 4, 1000).astype(np.float32).view(np.uint32) & 0xFFFF0000)
    l = bits.view(np.float32).astype(np.float64)
    out = oracle.repetition_penalty(l, range(1000), 1.1, "bf16")
    ob = out.astype(np.float32).view(np.uint32)
    assert np.all((ob & 0xFFFF) == 0)
    assert np.all(out <= l)
