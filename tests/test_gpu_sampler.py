"""GPU parity of greedy_argmax and sample_rows against the oracle, through the C ABI."""
import numpy as np
import pytest

from tests.gpu_common import (BAND, Tally, compare, device, gpu_available, report, run_sample,
                              to_dev, torch)
from oracle.parity import parity_sample_batch

import oracle
import token_sampling_row_amd as tsr
from token_sampling_row_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def sampler():
    s = tsr.Sampler(0, max_rows=1 << 17, max_vocab=1 << 18, max_k=8, seed=0x5EED0001)
    yield s
    s.close()


def make_sampler(seed):
    return tsr.Sampler(0, max_rows=1 << 17, max_vocab=1 << 18, max_k=8, seed=seed)


def vals(data, dtype):
    return oracle.values_from_stored(data, dtype)


def print_case(name, **kw):
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


# ---------------------------------------------------------------- Philox

def test_philox_words_bit_exact():
    seed = 0x0123456789ABCDEF
    rng = np.random.default_rng(1)
    ctr = rng.integers(0, 2 ** 32, (4096, 4), dtype=np.uint64).astype(np.uint32)
    print_case("philox", n=4096)
    with make_sampler(seed) as s:
        got = s.philox(torch.from_numpy(ctr.view(np.int32)).to(device())).cpu().numpy()
    want = oracle.philox4x32_10(ctr, oracle.philox.seed_key(seed))
    assert np.array_equal(got.view(np.uint32), want)


# ---------------------------------------------------------------- greedy

@pytest.mark.parametrize("cfg", [2, 3])
def test_greedy_configs(sampler, cfg):
    w = wl.config(cfg)
    print_case("greedy", cfg=cfg, rows=w.rows, vocab=w.vocab)
    x = to_dev(w.data, w.dtype)
    ref = oracle.greedy_batch(vals(w.data, w.dtype))
    st = torch.empty(w.rows, dtype=torch.int32, device=device())
    got = sampler.greedy_argmax(x, status=st).cpu().numpy()
    assert np.array_equal(got, np.array([t for t, _ in ref]))
    assert (st.cpu().numpy() == 0).all()
    res = run_sample(sampler, x, {"temperature": 0.0}, 0, diag=True)
    assert np.array_equal(res["token"], got)


def edge_rows(V, rng):
    rows = []
    r = rng.normal(0, 1, V).astype(np.float32)
    rows.append(r.copy())                                  # plain
    t = np.round(rng.normal(0, 1, V), 1).astype(np.float32)
    t[V // 3] = t[V - 1] = t.max() + 1                     # tied maximum: lowest id wins
    rows.append(t)
    n = r.copy(); n[V // 2] = np.nan; rows.append(n)       # NaN
    p = r.copy(); p[V - 1] = np.inf; rows.append(p)        # +inf
    rows.append(np.full(V, -np.inf, np.float32))           # empty
    m = np.full(V, -np.inf, np.float32); m[V - 1] = -3.0   # one finite logit at the end
    rows.append(m)
    z = np.zeros(V, np.float32); z[::2] = -0.0             # +0 and -0 tie
    rows.append(z)
    h = np.full(V, -1e30, np.float32); h[0] = 3e38         # extreme finite values
    rows.append(h)
    return np.stack(rows)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 3, 5, 8, 63, 64, 1000, 4097, 8192, 32000, 65537, 128256,
                               200003])
def test_greedy_edges(sampler, dtype, V):
    rng = np.random.default_rng(V)
    rows = edge_rows(V, rng)
    data = wl.f32_to_bf16_bits(rows) if dtype == "bf16" else rows
    print_case("greedy_edges", dtype=dtype, V=V)
    x = to_dev(data, dtype)
    ref = oracle.greedy_batch(vals(data, dtype))
    st = torch.empty(rows.shape[0], dtype=torch.int32, device=device())
    got = sampler.greedy_argmax(x, status=st).cpu().numpy()
    assert got.tolist() == [t for t, _ in ref]
    assert st.cpu().numpy().tolist() == [s for _, s in ref]


def test_sample_strided_and_unaligned():
    rng = np.random.default_rng(4)
    V = 3001
    base = rng.normal(0, 1.5, (24, V + 5)).astype(np.float32)
    x = to_dev(base, "f32")[:, 3:V + 3]          # rows not 16-byte aligned
    values = oracle.values_from_stored(np.ascontiguousarray(base[:, 3:V + 3]), "f32")
    seed = 5150
    with make_sampler(seed) as s:
        for i, prm in enumerate([dict(temperature=0.8, top_k=40, top_p=0.9, min_p=0.05),
                                 dict(temperature=1.0), dict(temperature=0.0)]):
            print_case("strided_sample", params=prm)
            refs = [oracle.sample_row(values[b], prm, seed, b, i) for b in range(24)]
            got = run_sample(s, x, prm, i, diag=True)
            compare(got, refs, list(range(24)), values, greedy=prm["temperature"] == 0.0)


@pytest.mark.parametrize("dtype,V", [("f32", 50257), ("f32", 77823), ("bf16", 50257),
                                     ("bf16", 128255), ("bf16", 151935), ("bf16", 160001)])
def test_sample_unaligned_contiguous(dtype, V):
    """A contiguous batch of an odd vocabulary: rows start on every 2- or
    4-byte offset and are read with 16-byte loads at that alignment into the
    register rows (the last case is wider than the register file and
    streams); narrow and wide kept sets, no filter and greedy, against the
    oracle on every row."""
    rng = np.random.default_rng(V + (7 if dtype == "bf16" else 0))
    rows = [-a * np.log(rng.permutation(V) + 1.0) + rng.normal(0, 0.5, V)
            for a in np.linspace(0.2, 1.4, 11)]
    r = rng.normal(0, 1, V)
    r[rng.random(V) < 0.3] = -np.inf
    rows.append(r)
    data = np.stack(rows).astype(np.float32)
    if dtype == "bf16":
        data = wl.f32_to_bf16_bits(data)
    values = vals(data, dtype)
    seed = 6060 + V
    grid = [dict(temperature=0.9, top_k=50, top_p=0.95, min_p=0.1), dict(temperature=1.0),
            dict(temperature=1.5, top_p=0.9), dict(temperature=0.0),
            dict(temperature=0.8, min_p=0.2)]
    with make_sampler(seed) as s:
        x = to_dev(data, dtype)
        assert x.stride(0) == V
        for i, prm in enumerate(grid):
            print_case("unaligned_contiguous", dtype=dtype, V=V, params=prm)
            refs = [oracle.sample_row(values[b], prm, seed, b, i) for b in range(len(rows))]
            got = run_sample(s, x, prm, i, diag=True)
            compare(got, refs, list(range(len(rows))), values,
                    greedy=prm["temperature"] == 0.0)


@pytest.mark.parametrize("dtype,V", [("bf16", 50257), ("bf16", 128255), ("f32", 160001)])
def test_greedy_unaligned_contiguous(sampler, dtype, V):
    """greedy_argmax over a contiguous batch of an odd vocabulary (rows off
    16-byte boundaries; the last case streams), ties and -inf included."""
    rng = np.random.default_rng(V)
    data = np.round(rng.normal(0, 2, (9, V)), 1).astype(np.float32)
    data[1, :] = -np.inf
    data[1, V - 1] = 0.5                       # only the last id is finite
    data[2, :] = 3.0                           # one tie group: id 0
    data[3, ::2] = -np.inf
    if dtype == "bf16":
        data = wl.f32_to_bf16_bits(data)
    values = vals(data, dtype)
    print_case("greedy_unaligned", dtype=dtype, V=V)
    got = sampler.greedy_argmax(to_dev(data, dtype)).cpu().numpy()
    assert got.tolist() == [int(np.argmax(r)) for r in values]


def test_greedy_strided_and_unaligned(sampler):
    rng = np.random.default_rng(3)
    V = 1001
    base = rng.normal(0, 1, (16, V + 3)).astype(np.float32)
    x = to_dev(base, "f32")[:, 1:V + 1]          # row stride V + 3, rows not 16-byte aligned
    print_case("greedy_strided", V=V)
    got = sampler.greedy_argmax(x).cpu().numpy()
    assert got.tolist() == [int(np.argmax(r[1:V + 1])) for r in base]


# ---------------------------------------------------------------- sampler, workloads

def check_workload(sampler_seed, w, params, step, rows=None, probs_rows=None):
    """sample_rows on a whole workload batch, once as the benchmark calls it and
    once with every diagnostic (kept set, kept mass, dense p~), against the
    oracle on ``rows`` (default every row; p~ on ``probs_rows``, default every
    row), in a pool of host processes. Prints the parity counts."""
    values = vals(w.data, w.dtype)
    with make_sampler(sampler_seed) as s:
        x = to_dev(w.data, w.dtype)
        plain = run_sample(s, x, params, step)                       # as the bench runs it
        full = run_sample(s, x, params, step, diag=True, probs=True)
    assert np.array_equal(plain["token"], full["token"])
    t = parity_sample_batch(values, params, sampler_seed, step, full, rows=rows,
                            probs_rows=probs_rows)
    report(f"{w.name} {params}", t)
    assert t.out_of_band == 0, t.notes[:5]
    return t


def test_config1(sampler):
    w = wl.config(1)
    print_case("config1")
    check_workload(wl.philox_seed(1), w, w.runs[0], 0)


@pytest.mark.parametrize("run", [1, 2])
def test_config2_runs(run):
    w = wl.config(2)
    print_case("config2", run=run)
    check_workload(wl.philox_seed(2), w, w.runs[run], run)


def test_config3_full_chain():
    w = wl.config(3)
    print_case("config3")
    t = check_workload(wl.philox_seed(3), w, w.runs[0], 0)
    assert t.rows == 256 and t.probs_rows == 256


@pytest.mark.parametrize("run", [0, 1])
def test_config5_all_rows(run):
    """Every row of the 1024 x 151936 batch (p~ on every 8th row); also counts
    mismatches a 1e-9 band would not excuse (the wide nucleus has ~9e-6 of
    kept mass per token, so ~20% of its draws sit within 1e-6 of an end)."""
    w = wl.config(5)
    print_case("config5", run=run)
    t = check_workload(wl.philox_seed(5), w, w.runs[run], run, probs_rows=range(0, 1024, 8))
    assert t.rows == 1024


# ---------------------------------------------------------------- sampler, edges

PARAM_GRID = [
    dict(temperature=1.0),
    dict(temperature=0.8, top_k=40, top_p=0.9, min_p=0.05),
    dict(temperature=0.8, top_k=40, top_p=0.9, min_p=0.05, mode=1),
    dict(temperature=1.3, top_k=5, top_p=0.5, mode=1),
    dict(temperature=1.0, top_k=1),
    dict(temperature=1.0, top_p=0.0),
    dict(temperature=2.0, top_p=0.95),
    dict(temperature=0.5, min_p=0.999),
    dict(temperature=1e-3),
    dict(temperature=50.0, top_k=3000),
    dict(temperature=0.9, top_k=2500, top_p=0.99),
    dict(temperature=1.0, min_p=1e-6),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 3, 7, 100, 1000, 4099, 20000, 70001, 131072])
def test_small_grid(dtype, V):
    rng = np.random.default_rng(V + (7 if dtype == "bf16" else 0))
    rows = []
    for q in (0.0, 0.5):                            # q > 0 quantises logits: many ties
        for a in (1.0, 0.2):
            r = -a * np.log(rng.permutation(V) + 1.0) + rng.normal(0, 0.5, V)
            if q:
                r = np.round(r / q) * q
            rows.append(r)
    r = rng.normal(0, 1, V); r[rng.random(V) < 0.3] = -np.inf; r[0] = 0.0
    rows.append(r)                                  # -inf holes
    rows.append(np.zeros(V))                        # one tie group
    data = np.stack(rows).astype(np.float32)
    if dtype == "bf16":
        data = wl.f32_to_bf16_bits(data)
    values = vals(data, dtype)
    seed = 1234 + V
    tally = Tally()
    with make_sampler(seed) as s:
        x = to_dev(data, dtype)
        for i, prm in enumerate(PARAM_GRID):
            print_case("grid", dtype=dtype, V=V, params=prm)
            refs = [oracle.sample_row(values[b], prm, seed, b, i) for b in range(len(rows))]
            got = run_sample(s, x, prm, i, diag=True, probs=True)
            compare(got, refs, list(range(len(rows))), values, tally=tally)
    report(f"grid V={V} {dtype}", tally)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [70000, 151936, 160001])
def test_general_path_wide_supports(V, dtype):
    """Kept sets far larger than the LDS candidate buffer (the histogram path),
    in rows held in registers and in rows too wide for them (streamed). In
    bf16, rows of large-magnitude logits take the exact value histogram (one
    bf16 value per bin), rows near zero its per-element bins and fallbacks;
    a row of large positive logits spanning more than 32 below its maximum
    puts many values in the histogram's last (mixed) bin, and -inf holes sit
    inside chunks of otherwise single-value bins."""
    rng = np.random.default_rng(5)
    rows = [rng.normal(0, 0.3, V),                          # flat: huge nucleus
            np.round(rng.normal(0, 0.3, V), 2),             # flat with heavy ties
            np.concatenate([np.zeros(V // 2), np.full(V - V // 2, -0.001)]),  # 2 big groups
            -0.05 * np.log(rng.permutation(V) + 1.0),
            rng.normal(-12.0, 1.5, V),                      # every value |v| >= 8 (in bf16)
            -np.log(rng.permutation(V) + 1.0) + rng.normal(0, 0.5, V),   # mixed magnitudes
            rng.normal(40.0, 12.0, V)]                      # large positive, wide span
    holes = -np.log(rng.permutation(V) + 1.0) + rng.normal(-6.0, 0.5, V)
    holes[rng.random(V) < 0.05] = -np.inf                   # -inf holes among |v| >= 4
    rows.append(holes)
    data = np.stack(rows).astype(np.float32)
    if dtype == "bf16":
        data = wl.f32_to_bf16_bits(data)
    values = vals(data, dtype)
    seed = 77
    grid = [dict(temperature=1.0, top_p=0.9), dict(temperature=1.0, top_p=0.5, mode=1),
            dict(temperature=1.0, min_p=0.5), dict(temperature=1.0, top_k=30000),
            dict(temperature=1.0, top_k=60000, top_p=0.7),
            dict(temperature=1.0, top_k=60000, top_p=0.7, mode=1),
            dict(temperature=0.7, top_p=0.999, min_p=0.2), dict(temperature=1.0),
            dict(temperature=40.0, top_p=0.9)]   # mass far below the maximum counts
    with make_sampler(seed) as s:
        x = to_dev(data, dtype)
        for i, prm in enumerate(grid):
            print_case("general", V=V, dtype=dtype, params=prm)
            refs = [oracle.sample_row(values[b], prm, seed, b, i) for b in range(len(rows))]
            got = run_sample(s, x, prm, i, diag=True, probs=True)
            compare(got, refs, list(range(len(rows))), values)


@pytest.mark.parametrize("V", [70001, 151936])
def test_topk_chunk_max_bound_bf16(V):
    """Top-k alone on bf16 rows held in registers with k above the candidate
    sketch (the value histogram counts only bins at or above the k-th largest
    chunk maximum): flat rows, heavy ties at the boundary, -inf holes, rows
    of one or two tie groups, and k at and past the bound's limit (eight
    chunk maxima per thread)."""
    rng = np.random.default_rng(V + 11)
    rows = [rng.normal(0, 0.3, V),
            np.round(rng.normal(0, 0.3, V), 1),                           # large tie groups
            -np.log(rng.permutation(V) + 1.0) + rng.normal(0, 0.5, V),
            rng.normal(-12.0, 1.5, V),
            np.concatenate([np.zeros(V // 2), np.full(V - V // 2, -0.001)]),
            np.zeros(V)]
    holes = -np.log(rng.permutation(V) + 1.0) + rng.normal(-6.0, 0.5, V)
    holes[rng.random(V) < 0.3] = -np.inf
    rows.append(holes)
    sparse = np.full(V, -np.inf)
    sparse[rng.choice(V, 1500, replace=False)] = rng.normal(0, 1, 1500)   # fewer finite than k
    rows.append(sparse)
    data = wl.f32_to_bf16_bits(np.stack(rows).astype(np.float32))
    values = vals(data, "bf16")
    seed = 404
    nc = -(-V // (8 * 512))
    grid = [dict(temperature=1.0, top_k=129), dict(temperature=1.5, top_k=1024),
            dict(temperature=0.7, top_k=nc * 64), dict(temperature=1.0, top_k=nc * 64 + 1),
            dict(temperature=1.0, top_k=700, min_p=0.01)]
    tally = Tally()
    with make_sampler(seed) as s:
        x = to_dev(data, "bf16")
        for i, prm in enumerate(grid):
            print_case("topk_bound", V=V, params=prm)
            refs = [oracle.sample_row(values[b], prm, seed, b, i) for b in range(len(rows))]
            got = run_sample(s, x, prm, i, diag=True, probs=True)
            compare(got, refs, list(range(len(rows))), values, tally=tally)
    report(f"top-k bound V={V}", tally)


@pytest.mark.parametrize("dtype,V", [("bf16", 151937), ("bf16", 155647), ("f32", 77823),
                                     ("f32", 65537)])
def test_widest_register_rows_ragged(dtype, V):
    """Rows of 33 to 38 chunk rows per thread whose vocabulary ends inside a
    16-byte chunk: the chunk rows past the 32nd sit at fixed register indices
    and the last chunk is partial; every filter family and the unfiltered
    walk."""
    rng = np.random.default_rng(V * 3 + (1 if dtype == "bf16" else 0))
    rows = [-np.log(rng.permutation(V) + 1.0) + rng.normal(0, 0.5, V),
            rng.normal(0, 0.3, V),
            np.round(rng.normal(-6, 1.0, V), 1)]
    tail = rng.normal(-20, 1, V)
    tail[-3:] = 5.0                                   # the maximum in the partial last chunk
    rows.append(tail)
    holes = rng.normal(0, 1, V)
    holes[rng.random(V) < 0.4] = -np.inf
    rows.append(holes)
    data = np.stack(rows).astype(np.float32)
    if dtype == "bf16":
        data = wl.f32_to_bf16_bits(data)
    values = vals(data, dtype)
    seed = 515
    grid = [dict(temperature=1.0), dict(temperature=1.5, top_p=0.9),
            dict(temperature=1.5, top_k=1024), dict(temperature=0.9, top_k=50, top_p=0.95, min_p=0.1),
            dict(temperature=0.0)]
    tally = Tally()
    with make_sampler(seed) as s:
        x = to_dev(data, dtype)
        for i, prm in enumerate(grid):
            print_case("widest_ragged", dtype=dtype, V=V, params=prm)
            refs = [oracle.sample_row(values[b], prm, seed, b, i) for b in range(len(rows))]
            got = run_sample(s, x, prm, i, diag=True, probs=True)
            compare(got, refs, list(range(len(rows))), values, greedy=prm["temperature"] == 0.0,
                    tally=tally)
    report(f"widest ragged V={V} {dtype}", tally)


def test_bad_rows_and_status(sampler):
    V = 5000
    rng = np.random.default_rng(2)
    rows = edge_rows(V, rng)
    values = vals(rows, "f32")
    prm = dict(temperature=0.9, top_k=50, top_p=0.95, min_p=0.1)
    print_case("bad_rows")
    refs = [oracle.sample_row(values[b], prm, 0x5EED0001, b, 0) for b in range(len(rows))]
    got = run_sample(sampler, to_dev(rows, "f32"), prm, 0, diag=True)
    compare(got, refs, list(range(len(rows))), values)


def test_determinism_and_step(sampler):
    w = wl.config(3, rows=64)
    x = to_dev(w.data, w.dtype)
    print_case("determinism")
    a = sampler.sample_rows(x, {"temperature": 1.5}, 5).cpu().numpy()
    b = sampler.sample_rows(x, {"temperature": 1.5}, 5).cpu().numpy()
    c = sampler.sample_rows(x, {"temperature": 1.5}, 6).cpu().numpy()
    assert np.array_equal(a, b)
    assert (a != c).mean() > 0.5


def test_token_histogram_chi_square(sampler):
    """Many copies of one row: tokens follow p~ (eq. 39.2)."""
    from scipy import stats
    l = np.array([1.0, 0.2, 0.7, -0.4, 0.7, -2.0, 0.3, -1.0, 1.0, 0.0] * 4, dtype=np.float32)
    prm = dict(temperature=0.9, top_k=12, top_p=0.9, min_p=0.05)
    s = oracle.support(l.astype(np.float64), oracle.Params.of(prm))
    n = 1 << 17
    print_case("chi_square", n=n)
    x = to_dev(np.tile(l, (n, 1)), "f32")
    toks = sampler.sample_rows(x, prm, 11).cpu().numpy()
    obs = np.bincount(toks, minlength=len(l))
    assert (obs[~s.keep] == 0).all()
    assert stats.chisquare(obs[s.keep], s.p_tilde[s.keep] * n).pvalue > 1e-4
