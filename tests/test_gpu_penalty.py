"""GPU parity of the repetition penalty (legost.in "Choosing the next word",
section "The repetition penalty") through sample_rows_ex, alone and with an
allowed-token mask, against the oracle, through the C ABI."""
import numpy as np
import pytest

from tests.gpu_common import (Tally, compare, compare_logprob, gpu_available, run_ex,
                              run_sample, to_dev, torch)

import oracle
import token_sampling_row_amd as tsr
from token_sampling_row_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def make_sampler(seed):
    return tsr.Sampler(0, max_rows=4096, max_vocab=1 << 18, max_k=8, seed=seed)


def print_case(name, **kw):
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


PARAMS = [
    dict(temperature=0.9, top_k=50, top_p=0.95, min_p=0.1),
    dict(temperature=1.0),
    dict(temperature=1.2, top_p=0.9),
    dict(temperature=0.7, top_k=5),
    dict(temperature=0.0),
]


def windows(values, H, rng):
    """Per row: a window of H ids mixing the row's largest logits (the row
    max moves), neighbours in one chunk, the last id, repeats and padding."""
    rows, V = values.shape
    out = np.empty((rows, H), dtype=np.int32)
    for b in range(rows):
        top = np.argsort(-values[b], kind="stable")[:8]
        pool = np.concatenate([top, [V - 1, 0, min(1, V - 1), min(2, V - 1)],
                               rng.integers(0, V, 40), [-1, V, V + 5, 2 ** 30]])
        w = rng.choice(pool, H)
        w[: min(H, 3)] = top[: min(H, 3)]
        out[b] = w
    return out


def check(s, seed, data, dtype, prm, step, hist, penalty, words=None, probs=False):
    values = oracle.values_from_stored(data, dtype)
    rows, V = values.shape
    allowed = None if words is None else [oracle.allowed_from_words(words[b], V)
                                          for b in range(rows)]
    refs = [oracle.sample_row(values[b], prm, seed, b, step,
                              None if allowed is None else allowed[b],
                              history=hist[b], penalty=penalty, dtype=dtype)
            for b in range(rows)]
    got = run_ex(s, to_dev(data, dtype), prm, step, words=words, hist=hist, penalty=penalty,
                 probs=probs)
    t = compare(got, refs, list(range(rows)), values, greedy=prm.get("temperature") == 0.0)
    n = compare_logprob(got, refs, list(range(rows)))
    return t, n, got


@pytest.mark.parametrize("dtype,V", [("f32", 7), ("f32", 1000), ("f32", 70001),
                                     ("f32", 131072), ("bf16", 40), ("bf16", 1000),
                                     ("bf16", 128256), ("bf16", 160001)])
@pytest.mark.parametrize("H", [1, 17, 64])
def test_penalty_grid(dtype, V, H):
    """Rows held in registers and streamed rows; windows of 1, 17 and 64 ids."""
    rng = np.random.default_rng(V * 7 + H + (1 if dtype == "bf16" else 0))
    rows = [-a * np.log(rng.permutation(V) + 1.0) + rng.normal(0, 0.5, V)
            for a in (0.2, 0.6, 1.0, 1.4)]
    rows.append(rng.normal(0, 2.0, V))             # positive and negative logits
    rows.append(np.full(V, 1.5))                   # one tie group: the window splits it
    data = np.stack(rows).astype(np.float32)
    if dtype == "bf16":
        data = wl.f32_to_bf16_bits(data)
    values = oracle.values_from_stored(data, dtype)
    hist = windows(values, H, rng)
    seed = 4000 + V + H
    tally, nlp = Tally(), 0
    with make_sampler(seed) as s:
        for i, prm in enumerate(PARAMS):
            for pen in (1.1, 2.0):
                print_case("penalty_grid", dtype=dtype, V=V, H=H, params=prm, r=pen)
                t, n, _ = check(s, seed, data, dtype, prm, i, hist, pen, probs=V <= 70001)
                tally.rows += t.rows
                tally.token_excused += t.token_excused
                nlp += n
    print(f"penalty V={V} {dtype} H={H}: rows={tally.rows} logprob rows={nlp} "
          f"excused={tally.token_excused}", flush=True)


def test_penalty_with_mask_and_unaligned_rows():
    """The penalty before an allowed-token mask, in aligned rows and in rows
    whose start is not 16-byte aligned."""
    rng = np.random.default_rng(9)
    V = 5003
    base = rng.normal(0, 1.5, (12, V + 3)).astype(np.float32)
    seed = 777
    with make_sampler(seed) as s:
        for off in (0, 1):
            x = to_dev(base, "f32")[:, off:V + off]
            data = np.ascontiguousarray(base[:, off:V + off])
            values = oracle.values_from_stored(data, "f32")
            hist = windows(values, 32, rng)
            words = wl.allowed_words(5, 12, V, "p=0.3")
            for i, prm in enumerate(PARAMS):
                print_case("penalty_mask", offset=off, params=prm)
                allowed = [oracle.allowed_from_words(words[b], V) for b in range(12)]
                refs = [oracle.sample_row(values[b], prm, seed, b, i, allowed[b],
                                          history=hist[b], penalty=1.3) for b in range(12)]
                got = run_ex(s, x, prm, i, words=words, hist=hist, penalty=1.3)
                compare(got, refs, list(range(12)), values, greedy=prm["temperature"] == 0.0)
                compare_logprob(got, refs, list(range(12)))


def test_penalty_one_and_empty_window_equal_sample_rows():
    w = wl.config(3)
    seed = wl.philox_seed(3)
    hist = np.tile(np.arange(64, dtype=np.int32), (w.rows, 1))
    with make_sampler(seed) as s:
        x = to_dev(w.data, w.dtype)
        print_case("penalty_off")
        a = run_sample(s, x, w.runs[0], 5, diag=True)
        b = run_ex(s, x, w.runs[0], 5, hist=hist, penalty=1.0)
        c = run_ex(s, x, w.runs[0], 5, hist=hist[:, :0], penalty=1.5)
    for k in ("token", "status", "kept_count", "threshold", "kept_mass"):
        assert np.array_equal(a[k], b[k]) and np.array_equal(a[k], c[k]), k


def test_penalty_workload_full_size():
    """The 256 x 128256 bf16 workload with its full chain, a 64-token window
    per row (r = 1.1), every row checked."""
    w = wl.config(3)
    seed = wl.philox_seed(3)
    rng = np.random.default_rng(31)
    values = oracle.values_from_stored(w.data, w.dtype)
    hist = windows(values, 64, rng)
    with make_sampler(seed) as s:
        print_case("penalty_full", workload=w.name)
        t, n, _ = check(s, seed, w.data, w.dtype, w.runs[0], 0, hist, 1.1)
    print(f"penalty full: rows={t.rows} logprob rows={n} in_band={t.in_band} "
          f"token_excused={t.token_excused}", flush=True)
    assert t.rows == 256 and n >= 250


def test_invalid_penalty_arguments():
    import ctypes
    V = 100
    x = to_dev(np.zeros((2, V), np.float32), "f32")
    with make_sampler(1) as s:
        for pen, H in ((0.9, 4), (float("nan"), 4), (1.1, 65)):
            hist = torch.zeros((2, H), dtype=torch.int32, device=x.device)
            with pytest.raises(tsr.TsrError):
                s.sample_rows_ex(x, {"temperature": 1.0}, 0, history=hist, penalty=pen)
