"""GPU parity of sample_rows_masked (constrained decoding: an allowed-token
bitmask applied before every step, gowda.ai chapter 39, section 39.3) and of
the log-probability it returns for each drawn token, against the oracle,
through the C ABI."""
import numpy as np
import pytest

from tests.gpu_common import (Tally, compare, compare_logprob, gpu_available, run_masked,
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


def check(s, seed, data, dtype, words, prm, step, probs=False):
    """Run the masked sampler and the oracle on the same rows; compare
    everything. Returns (tally, logprob rows checked)."""
    values = oracle.values_from_stored(data, dtype)
    rows, V = values.shape
    allowed = None if words is None else [oracle.allowed_from_words(words[b], V)
                                          for b in range(rows)]
    refs = [oracle.sample_row(values[b], prm, seed, b, step,
                              None if allowed is None else allowed[b]) for b in range(rows)]
    got = run_masked(s, to_dev(data, dtype), words, prm, step, diag=True, probs=probs)
    greedy = prm.get("temperature", 1.0) == 0.0
    t = compare(got, refs, list(range(rows)), values, greedy=greedy)
    n = compare_logprob(got, refs, list(range(rows)))
    return t, n


MASK_KINDS = ["all", "none", "p=0.5", "p=0.02", "few=1", "few=7", "few=300", "block"]

PARAMS = [
    dict(temperature=0.9, top_k=50, top_p=0.95, min_p=0.1),
    dict(temperature=0.9, top_k=50, top_p=0.95, min_p=0.1, mode=1),
    dict(temperature=1.0),
    dict(temperature=1.5, top_p=0.9),
    dict(temperature=1.0, top_k=1000),
    dict(temperature=0.7, top_k=20),
    dict(temperature=0.0),
]


def masked_rows(V, dtype, rng):
    """Zipf-like rows (one per mask kind), plus a copy of row 0 whose top
    tokens are disallowed (the kept set must move down the ranking), plus a
    row with NaN and +inf at disallowed ids only."""
    k = len(MASK_KINDS)
    rows = [-a * np.log(rng.permutation(V) + 1.0) + rng.normal(0, 0.5, V)
            for a in np.linspace(0.3, 1.3, k)]
    rows.append(rows[0].copy())
    bad = rng.normal(0, 1, V)
    rows.append(bad)
    data = np.stack(rows).astype(np.float32)
    if dtype == "bf16":
        data = wl.f32_to_bf16_bits(data)
    return data


def words_for(data, dtype, seed, rng):
    rows, V = data.shape
    k = len(MASK_KINDS)
    ws = [wl.allowed_words(seed + i, 1, V, kind)[0] for i, kind in enumerate(MASK_KINDS)]
    vals = oracle.values_from_stored(data, dtype)
    # row k: every token of the ten largest logits' values is disallowed
    top = np.argsort(-vals[k], kind="stable")[:10]
    keep = np.ones(((V + 31) // 32) * 32, dtype=bool)
    keep[top] = False
    # row k + 1: NaN and +inf sit where the mask is 0
    allow = rng.random(V) < 0.7
    allow[0] = True
    off = np.nonzero(~allow)[0]
    if off.size:
        vals_bad = data[k + 1].copy()
        if dtype == "bf16":
            vals_bad[off[0]] = 0x7FC0            # NaN
            vals_bad[off[-1]] = 0x7F80           # +inf
        else:
            vals_bad[off[0]] = np.nan
            vals_bad[off[-1]] = np.inf
        data[k + 1] = vals_bad
    keep2 = np.zeros_like(keep)
    keep2[:V] = allow
    for m in (keep, keep2):
        ws.append((m.reshape(-1, 32).astype(np.uint64) << np.arange(32, dtype=np.uint64))
                  .sum(axis=1).astype(np.uint32))
    return np.stack(ws)


@pytest.mark.parametrize("dtype,V", [("f32", 1), ("f32", 33), ("f32", 1000), ("f32", 4099),
                                     ("f32", 70001), ("f32", 131072),
                                     ("bf16", 1), ("bf16", 40), ("bf16", 1000),
                                     ("bf16", 70001), ("bf16", 128256), ("bf16", 160001)])
def test_masked_grid(dtype, V):
    """Every mask kind under every parameter set, in rows held in registers
    (f32 up to 77824 ids, bf16 up to 155648) and in streamed rows."""
    rng = np.random.default_rng(V * 3 + (1 if dtype == "bf16" else 0))
    data = masked_rows(V, dtype, rng)
    words = words_for(data, dtype, 100 + V, rng)
    seed = 999 + V
    tally, nlp = Tally(), 0
    with make_sampler(seed) as s:
        for i, prm in enumerate(PARAMS):
            print_case("masked_grid", dtype=dtype, V=V, params=prm)
            t, n = check(s, seed, data, dtype, words, prm, i, probs=V <= 70001)
            tally.rows += t.rows
            tally.token_excused += t.token_excused
            tally.support_excused += t.support_excused
            nlp += n
    print(f"masked V={V} {dtype}: rows={tally.rows} logprob rows={nlp} "
          f"excused token={tally.token_excused} support={tally.support_excused}", flush=True)
    assert nlp > 0


def test_empty_and_nonfinite_rows_under_mask():
    """An allowed set without a finite logit is the empty state (status 2,
    token -1, log p NaN); NaN or +inf at allowed ids is still non-finite."""
    V = 5000
    rng = np.random.default_rng(11)
    base = rng.normal(0, 1, V).astype(np.float32)
    rows = [base.copy() for _ in range(4)]
    rows[1][17] = np.nan                   # allowed NaN
    rows[2][18] = np.inf                   # disallowed +inf only
    rows[3][:] = -np.inf
    rows[3][4000] = 1.0                    # its only finite logit is disallowed
    data = np.stack(rows)
    allow = np.ones((4, ((V + 31) // 32) * 32), dtype=bool)
    allow[2, 18] = False
    allow[3, 4000] = False
    words = (allow.reshape(4, -1, 32).astype(np.uint64) << np.arange(32, dtype=np.uint64)) \
        .sum(axis=2).astype(np.uint32)
    seed = 4242
    with make_sampler(seed) as s:
        for i, prm in enumerate([dict(temperature=0.8, top_p=0.9), dict(temperature=0.0)]):
            print_case("masked_bad_rows", params=prm)
            got = run_masked(s, to_dev(data, "f32"), words, prm, i)
            assert got["status"].tolist() == [0, 1, 0, 2]
            assert got["token"][1] == -1 and got["token"][3] == -1
            assert np.isnan(got["logprob"][1]) and np.isnan(got["logprob"][3])
            assert got["token"][2] != 18
            check(s, seed, data, "f32", words, prm, i)


def test_null_mask_matches_sample_rows():
    """allowed = NULL is sample_rows: the same tokens and diagnostics, plus
    log p~ of each draw."""
    w = wl.config(3)
    seed = wl.philox_seed(3)
    prm = w.runs[0]
    with make_sampler(seed) as s:
        x = to_dev(w.data, w.dtype)
        print_case("null_mask", workload=w.name)
        a = run_sample(s, x, prm, 3, diag=True)
        b = run_masked(s, x, None, prm, 3, diag=True)
    for k in ("token", "status", "kept_count", "threshold", "kept_mass"):
        assert np.array_equal(a[k], b[k]), k
    assert np.all(b["logprob"] <= 0.0)


@pytest.mark.parametrize("kind", ["p=0.5", "few=40"])
def test_masked_workload_full_size(kind):
    """The 256 x 128256 bf16 workload with its full filter chain, every row
    under a mask, all rows checked, log p~ included."""
    w = wl.config(3)
    seed = wl.philox_seed(3)
    words = wl.allowed_words(31, w.rows, w.vocab, kind)
    with make_sampler(seed) as s:
        print_case("masked_full", workload=w.name, mask=kind)
        t, n = check(s, seed, w.data, w.dtype, words, w.runs[0], 0)
    print(f"masked full {kind}: rows={t.rows} logprob rows={n} in_band={t.in_band} "
          f"token_excused={t.token_excused} support_excused={t.support_excused}", flush=True)
    assert t.rows == 256 and n >= 250


def test_logprob_unmasked_workload_sampled_rows():
    """log p~ without a mask on the 1024 x 151936 bf16 workload (streamed
    rows), every 32nd row."""
    w = wl.config(5)
    seed = wl.philox_seed(5)
    rows = list(range(0, w.rows, 32))
    values = oracle.values_from_stored(w.data, w.dtype)
    for run, prm in enumerate(w.runs):
        refs = [oracle.sample_row(values[b], prm, seed, b, run) for b in rows]
        with make_sampler(seed) as s:
            print_case("logprob_c5", run=run)
            got = run_masked(s, to_dev(w.data, w.dtype), None, prm, run, diag=True)
        compare(got, refs, rows, values)
        assert compare_logprob(got, refs, rows) >= len(rows) - 2
