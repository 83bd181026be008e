"""The oracle's Philox4x32-10 against an independent implementation and for uniformity."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
from scipy import stats

from oracle.philox import (philox4x32_10, philox_scalar, sampler_counters, seed_key,
                           uniforms_from_words, DOMAIN_SAMPLE, DOMAIN_SPEC)

PIN_SRC = os.path.join(os.path.dirname(__file__), "golden", "philox_rocrand_pin.cpp")


def random_cases(n, seed=5):
    rng = np.random.default_rng(seed)
    keys = rng.integers(0, 2 ** 32, (n, 2), dtype=np.uint64)
    ctrs = rng.integers(0, 2 ** 32, (n, 4), dtype=np.uint64)
    keys[:4] = [[0, 0], [0xFFFFFFFF, 0xFFFFFFFF], [1, 0], [0, 1]]
    ctrs[:4] = [[0, 0, 0, 0], [0xFFFFFFFF] * 4, [1, 2, 3, 4], [0, 0, 0, 1]]
    return keys, ctrs


def engine_reachable(ctrs):
    """rocRAND reaches counter word 1 through a 64-bit count of outputs (4 per
    counter), so only c1 < 2^30 is reachable there."""
    c = ctrs.copy()
    c[:, 1] &= (1 << 30) - 1
    return c


def test_vector_and_scalar_agree():
    keys, ctrs = random_cases(200)
    for k, c in zip(keys, ctrs):
        v = philox4x32_10(c[None, :], k)[0].tolist()
        assert v == philox_scalar(c.tolist(), k.tolist())


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_against_rocrand_engine():
    """rocRAND ships a host-callable Philox4x32-10 engine: an implementation
    written independently of this oracle. Both must give the same words for
    arbitrary keys and counters."""
    keys, ctrs = random_cases(400, seed=8)
    ctrs = engine_reachable(ctrs)
    with tempfile.TemporaryDirectory() as td:
        exe = os.path.join(td, "pin")
        subprocess.run(["hipcc", "-O1", PIN_SRC, "-o", exe], check=True,
                       capture_output=True)
        inp = "".join("%x %x %x %x %x %x\n" % (k[0], k[1], *c) for k, c in zip(keys, ctrs))
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    got = np.array([[int(w, 16) for w in line.split()] for line in out.strip().splitlines()],
                   dtype=np.uint64)
    for i, (k, c) in enumerate(zip(keys, ctrs)):
        assert philox4x32_10(c[None, :], k)[0].tolist() == got[i].tolist()


def test_uniformity_and_independence():
    c = sampler_counters(np.arange(1 << 20), 0, 12345, DOMAIN_SAMPLE)
    w = philox4x32_10(c, seed_key(0x5EED0003))
    for col in range(4):
        hist = np.bincount((w[:, col] >> 16).astype(np.int64), minlength=1 << 16)
        assert stats.chisquare(hist).pvalue > 1e-4
    u = uniforms_from_words(w[:, 0])
    assert 0.0 <= u.min() and u.max() < 1.0
    # neighbouring rows, steps and domains do not repeat words
    w2 = philox4x32_10(sampler_counters(np.arange(1 << 20), 0, 12346, DOMAIN_SAMPLE),
                       seed_key(0x5EED0003))
    w3 = philox4x32_10(sampler_counters(np.arange(1 << 20), 0, 12345, DOMAIN_SPEC),
                       seed_key(0x5EED0003))
    assert np.mean(w[:, 0] == w2[:, 0]) < 1e-4 and np.mean(w[:, 0] == w3[:, 0]) < 1e-4
    assert abs(np.corrcoef(u, uniforms_from_words(w[:, 1]))[0, 1]) < 5e-3


def test_counter_layout():
    c = sampler_counters([7], 3, (5 << 32) | 9, DOMAIN_SPEC)[0].tolist()
    assert c == [7, 3 | (1 << 16), 9, 5]
    assert seed_key(0x0123456789ABCDEF) == (0x89ABCDEF, 0x01234567)
