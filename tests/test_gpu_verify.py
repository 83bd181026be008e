"""GPU parity of spec_verify against the oracle, through the C ABI."""
import numpy as np
import pytest

from tests.gpu_common import BAND, Tally, device, gpu_available, report, to_dev, torch
from oracle.parity import compare_verify_row

import oracle
import token_sampling_row_amd as tsr
from token_sampling_row_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def print_case(name, **kw):
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def oracle_drafts(draft_vals, params, seed, step):
    """Draft tokens drawn by the oracle sampler from q, one per (row, position)."""
    B, K, _ = draft_vals.shape
    xs = np.empty((B, K), dtype=np.int32)
    for b in range(B):
        for j in range(K):
            xs[b, j] = oracle.sample_row(draft_vals[b, j], params, seed, b * K + j, step).token
    return xs


def run_verify(seed, tgt, dft, xs, params, step, dtype="f32"):
    B, K1, V = tgt.shape
    with tsr.Sampler(0, max_rows=max(B, 1), max_vocab=V, max_k=K1 - 1, seed=seed) as s:
        st = torch.full((B,), -7, dtype=torch.int32, device=device())
        toks, acc = s.spec_verify(to_dev(tgt, dtype),
                                  to_dev(dft, dtype) if dft is not None else None,
                                  torch.from_numpy(np.ascontiguousarray(xs)).to(device()),
                                  params, step, out_status=st)
        torch.cuda.synchronize()
        return toks.cpu().numpy(), acc.cpu().numpy(), st.cpu().numpy()


def check(tgt_vals, dft_vals, xs, params, seed, step, got, name="verify"):
    """Every sequence against oracle.spec_verify_row under the parity rule (a
    mismatch is excused only by the decisions of the first position where
    the outputs differ); returns the tally."""
    toks, acc, st = got
    t = Tally()
    for b in range(tgt_vals.shape[0]):
        r = oracle.spec_verify_row(tgt_vals[b], dft_vals[b], xs[b], params, seed, b, step)
        compare_verify_row(t, b, r, toks[b], acc[b], st[b])
    report(f"{name} {params}", t)
    return t


@pytest.mark.parametrize("run", [0, 1])
def test_config4(run):
    w = wl.config(4)
    K = w.extra["K"]
    prm = w.runs[run]
    seed = wl.philox_seed(4)
    tv = oracle.values_from_stored(w.data, w.dtype)
    dv = oracle.values_from_stored(w.extra["draft"], w.dtype)
    xs = oracle_drafts(dv, {"temperature": 1.0}, seed, 1000)
    print_case("config4", run=run, params=prm)
    got = run_verify(seed, w.data, w.extra["draft"], xs, prm, run)
    t = check(tv, dv, xs, prm, seed, run, got, name="config4")
    toks, acc, _ = got
    print(f"config4 run {run}: acceptance={acc.mean() / K:.3f} tokens/verify="
          f"{(acc + 1).mean():.3f} excused={t.token_excused}", flush=True)


def test_greedy_verify_equals_greedy_decoding():
    rng = np.random.default_rng(4)
    B, K, V = 128, 5, 3000
    tgt = rng.normal(0, 1, (B, K + 1, V)).astype(np.float32)
    am = tgt.argmax(-1)
    xs = np.where(rng.random((B, K)) < 0.8, am[:, :K], rng.integers(0, V, (B, K))).astype(np.int32)
    print_case("greedy_verify")
    toks, acc, st = run_verify(1, tgt, None, xs, {"temperature": 0.0}, 0)
    for b in range(B):
        n = acc[b]
        assert list(toks[b, :n + 1]) == list(am[b, :n + 1])
        assert (toks[b, n + 1:] == -1).all()
        assert all(xs[b, j] == am[b, j] for j in range(n))
        assert n == K or xs[b, n] != am[b, n]
    assert (st == 0).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [2, 3, 17, 1000, 4097])
def test_verify_edges(dtype, V):
    rng = np.random.default_rng(V)
    B, K = 12, 3
    tgt = rng.normal(0, 1.5, (B, K + 1, V)).astype(np.float32)
    dft = (tgt[:, :K] + rng.normal(0, 1.0, (B, K, V))).astype(np.float32)
    tgt[1, 2, V // 2] = np.nan                 # bad target row
    dft[2, 0, :] = -np.inf                     # empty draft row
    tgt[3, 0, :] = 0.0                         # flat target row
    if dtype == "bf16":
        tgt_d, dft_d = wl.f32_to_bf16_bits(tgt), wl.f32_to_bf16_bits(dft)
    else:
        tgt_d, dft_d = tgt, dft
    tv = oracle.values_from_stored(tgt_d, dtype)
    dv = oracle.values_from_stored(dft_d, dtype)
    seed = 99
    for i, prm in enumerate([dict(temperature=1.0), dict(temperature=0.7, top_k=5, top_p=0.9),
                             dict(temperature=1.2, min_p=0.1, mode=1),
                             dict(temperature=0.0)]):
        xs = np.zeros((B, K), dtype=np.int32)
        for b in range(B):
            for j in range(K):
                r = oracle.sample_row(dv[b, j], prm if prm["temperature"] else {"temperature": 1.0},
                                      seed, b * K + j, 50 + i)
                xs[b, j] = r.token if r.token >= 0 else 0
        xs[4, 1] = V                          # out of range draft token
        xs[5, 0] = -1
        print_case("verify_edges", dtype=dtype, V=V, params=prm)
        got = run_verify(seed, tgt_d, dft_d, xs, prm, i, dtype)
        check(tv, dv, xs, prm, seed, i, got)


@pytest.mark.parametrize("dtype,K", [("f32", 1), ("bf16", 1), ("f32", 32), ("bf16", 17)])
def test_verify_draft_lengths(dtype, K):
    """One draft position and the longest drafts (K + 1 lanes of the finishing
    wavefront), on many sequences: drafts mostly the target's own draws, so
    long accepted prefixes occur, with some rows' drafts far from the target."""
    rng = np.random.default_rng(300 + K)
    B, V = 200 if K == 1 else 24, 2000
    tgt = rng.normal(0, 1.5, (B, K + 1, V)).astype(np.float32)
    noise = np.where(rng.random((B, 1, 1)) < 0.8, 0.05, 1.5)
    dft = (tgt[:, :K] + rng.normal(0, 1.0, (B, K, V)) * noise).astype(np.float32)
    if dtype == "bf16":
        tgt_d, dft_d = wl.f32_to_bf16_bits(tgt), wl.f32_to_bf16_bits(dft)
    else:
        tgt_d, dft_d = tgt, dft
    tv = oracle.values_from_stored(tgt_d, dtype)
    dv = oracle.values_from_stored(dft_d, dtype)
    seed = 600 + K
    for i, prm in enumerate([dict(temperature=1.0), dict(temperature=0.0)]):
        xs = oracle_drafts(dv, {"temperature": 1.0}, seed, 70 + i)
        print_case("verify_draft_lengths", dtype=dtype, K=K, params=prm)
        got = run_verify(seed, tgt_d, dft_d, xs, prm, i, dtype)
        check(tv, dv, xs, prm, seed, i, got)
        assert got[1].max() <= K and (got[2] == 0).all()


def test_verify_marginal_equals_target():
    """First emitted token follows p whatever the draft (page 4's three-token
    example, 100k sequences)."""
    from scipy import stats
    p = np.array([0.2, 0.5, 0.3])
    q = np.array([0.5, 0.3, 0.2])
    B = 100000
    tgt = np.tile(np.log(p).astype(np.float32), (B, 2, 1))
    dft = np.tile(np.log(q).astype(np.float32), (B, 1, 1))
    seed = 31
    xs = oracle_drafts(oracle.values_from_stored(dft, "f32"), {"temperature": 1.0}, seed, 7)
    print_case("marginal", B=B)
    toks, acc, st = run_verify(seed, tgt, dft, xs, {"temperature": 1.0}, 7)
    obs = np.bincount(toks[:, 0], minlength=3)
    assert stats.chisquare(obs, p * B).pvalue > 1e-4
    # acceptance rate = sum min(p, q) = 0.7
    assert abs(acc.mean() - 0.7) < 4 * np.sqrt(0.21 / B)
