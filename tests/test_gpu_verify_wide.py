"""GPU parity of spec_verify and tree_verify on rows wider than two register
rows per workgroup (more than 65,536 bf16 or 32,768 fp32 logits: one
workgroup per row records each row's kept set, then one per sequence decides),
against the oracle, through the C ABI. Vocabularies of 128,256 and 151,936
logits (the sizes of the pages' bf16 workloads), ragged and unaligned rows,
the widest rows the build covers, bad rows, and kept sets too large for the
candidate bound (the streaming fallback)."""
import numpy as np
import pytest

from tests.gpu_common import Tally, device, gpu_available, report, to_dev, torch
from oracle.parity import compare_tree_row, compare_verify_row

import oracle
import token_sampling_row_amd as tsr
from token_sampling_row_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

PARAMS = [dict(temperature=1.0),
          dict(temperature=0.8, top_k=50, top_p=0.9),
          dict(temperature=1.2, min_p=0.05, mode=1),
          dict(temperature=1.5, top_p=0.9),             # nucleus of thousands: streaming cut
          dict(temperature=1.0, top_k=5000),            # top-k beyond the LDS candidates
          dict(temperature=0.0)]


def print_case(name, **kw):
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def draft_tokens(dv, tv, prm, seed, step, rng):
    """Drafted ids: the oracle's draw from q~ (T > 0; a filtered-out or empty
    row gives id 0), else the target's argmax or a random id."""
    B, K, V = dv.shape
    xs = np.zeros((B, K), dtype=np.int32)
    for b in range(B):
        for j in range(K):
            if prm["temperature"] > 0:
                r = oracle.sample_row(dv[b, j], prm, seed, b * K + j, 500 + step)
                xs[b, j] = max(r.token, 0)
            else:
                xs[b, j] = np.argmax(tv[b, j]) if rng.random() < 0.7 else rng.integers(0, V)
    return xs


def verify_case(B, K, V, dtype, seed, edges):
    tgt, dft = wl.verify_batch(seed, B, K, V, dtype)
    if edges:
        bad = np.float32(np.nan) if dtype == "f32" else np.uint16(0x7FC0)
        ninf = np.float32(-np.inf) if dtype == "f32" else np.uint16(0xFF80)
        tgt[1, K, V // 3] = bad                   # the bonus row holds a NaN
        dft[2, 0, :] = ninf                       # an empty draft row
        tgt[3, 1, :] = tgt[3, 1, 0]               # a flat target row
    return tgt, dft


def check_verify(s, tgt, dft, xs, prm, seed, step, dtype):
    B, K1, V = tgt.shape
    K = K1 - 1
    tv = oracle.values_from_stored(tgt.reshape(B * K1, V), dtype).reshape(B, K1, V)
    dv = oracle.values_from_stored(dft.reshape(B * K, V), dtype).reshape(B, K, V)
    st = torch.full((B,), -7, dtype=torch.int32, device=device())
    greedy = prm["temperature"] == 0.0
    t_dev = to_dev(tgt.reshape(B * K1, V), dtype).view(B, K1, V)
    d_dev = None if greedy else to_dev(dft.reshape(B * K, V), dtype).view(B, K, V)
    toks, acc = s.spec_verify(t_dev, d_dev, torch.from_numpy(xs).to(device()), prm, step,
                              out_status=st)
    torch.cuda.synchronize()
    toks, acc, st = toks.cpu().numpy(), acc.cpu().numpy(), st.cpu().numpy()
    t = Tally()
    for b in range(B):
        r = oracle.spec_verify_row(tv[b], dv[b], xs[b], prm, seed, b, step)
        compare_verify_row(t, b, r, toks[b], acc[b], st[b])
    report(f"verify wide V={V} {dtype} K={K} {prm}", t)
    return toks, acc, st


@pytest.mark.parametrize("dtype,V,B,K", [("bf16", 128256, 8, 4), ("bf16", 151936, 6, 3),
                                         ("bf16", 100001, 6, 2), ("bf16", 155648, 6, 2),
                                         ("f32", 50257, 6, 3), ("f32", 77824, 6, 2)])
def test_verify_wide(dtype, V, B, K):
    seed = 7000 + V % 997
    tgt, dft = verify_case(B, K, V, dtype, seed, edges=True)
    rng = np.random.default_rng(V)
    tv = oracle.values_from_stored(tgt.reshape(-1, V), dtype).reshape(B, K + 1, V)
    dv = oracle.values_from_stored(dft.reshape(-1, V), dtype).reshape(B, K, V)
    with tsr.Sampler(0, max_rows=64, max_vocab=V, max_k=K, seed=seed) as s:
        for step, prm in enumerate(PARAMS):
            xs = draft_tokens(dv, tv, prm, seed, step, rng)
            xs[4, K - 1] = V if step % 2 == 0 else -1          # a draft id out of range
            print_case("verify_wide", dtype=dtype, V=V, B=B, K=K, params=prm)
            toks, acc, st = check_verify(s, tgt, dft, xs, prm, seed, step, dtype)
            assert st[1] != 0 and st[4] == 3                   # NaN row; bad draft id
            if prm["temperature"] > 0:
                assert st[2] != 0                              # empty draft row


@pytest.mark.parametrize("dtype,V,B,K", [("bf16", 128256, 1, 1), ("f32", 40000, 3, 1),
                                         ("bf16", 70001, 2, 5)])
def test_verify_wide_small_batches(dtype, V, B, K):
    """One draft position, a single sequence, an odd vocabulary: the grid's
    bonus rows last and the slice sums of one sequence."""
    seed = 7400 + V % 991
    tgt, dft = verify_case(B, K, V, dtype, seed, edges=False)
    rng = np.random.default_rng(V + K)
    tv = oracle.values_from_stored(tgt.reshape(-1, V), dtype).reshape(B, K + 1, V)
    dv = oracle.values_from_stored(dft.reshape(-1, V), dtype).reshape(B, K, V)
    with tsr.Sampler(0, max_rows=8, max_vocab=V, max_k=K, seed=seed) as s:
        for step, prm in enumerate(PARAMS):
            xs = draft_tokens(dv, tv, prm, seed, step, rng)
            print_case("verify_wide_small", dtype=dtype, V=V, B=B, K=K, params=prm)
            check_verify(s, tgt, dft, xs, prm, seed, step, dtype)


def test_verify_wide_greedy_is_argmax_decoding():
    """Temperature 0 at 128,256 bf16 logits: the emitted prefix is the
    target's argmax at every position (a property at any size)."""
    B, K, V = 16, 4, 128256
    tgt, _ = wl.verify_batch(7100, B, K, V, "bf16")
    am = np.argmax(wl.bf16_bits_to_f32(tgt), axis=-1)
    rng = np.random.default_rng(3)
    xs = np.where(rng.random((B, K)) < 0.75, am[:, :K], rng.integers(0, V, (B, K))).astype(np.int32)
    with tsr.Sampler(0, max_rows=B, max_vocab=V, max_k=K, seed=1) as s:
        print_case("verify_wide_greedy", V=V)
        toks, acc = s.spec_verify(to_dev(tgt.reshape(-1, V), "bf16").view(B, K + 1, V), None,
                                  torch.from_numpy(xs).to(device()), {"temperature": 0.0}, 0)
        torch.cuda.synchronize()
        toks, acc = toks.cpu().numpy(), acc.cpu().numpy()
    for b in range(B):
        n = acc[b]
        assert list(toks[b, :n + 1]) == list(am[b, :n + 1])
        assert (toks[b, n + 1:] == -1).all()
        assert n == K or xs[b, n] != am[b, n]


def make_trees(rows, N, V, tv, dv, prm, rng):
    parents = np.full((rows, N), -1, dtype=np.int32)
    toks = np.zeros((rows, N), dtype=np.int32)
    P = oracle.Params.of(prm)
    for b in range(rows):
        for n in range(1, N):
            parents[b, n] = rng.integers(0, n)
        for n in range(1, N):
            v = parents[b, n]
            if P.temperature > 0:
                q = oracle.support(dv[b, v], P).p_tilde
                toks[b, n] = rng.choice(V, p=q / q.sum())
            else:
                toks[b, n] = int(np.argmax(tv[b, v])) if rng.random() < 0.5 else rng.integers(0, V)
    return parents, toks


@pytest.mark.parametrize("dtype,V,N", [("bf16", 128256, 7), ("bf16", 151936, 4),
                                       ("f32", 50257, 5)])
def test_tree_wide(dtype, V, N):
    rows = 4
    rng = np.random.default_rng(N * 31 + V)
    tgt, dft = wl.verify_batch(7200 + N, rows, N, V, dtype)
    tdata, ddata = tgt[:, :N].copy(), dft     # N target rows and N draft rows per sequence
    tv = oracle.values_from_stored(tdata.reshape(-1, V), dtype).reshape(rows, N, V)
    dv = oracle.values_from_stored(ddata.reshape(-1, V), dtype).reshape(rows, N, V)
    seed = 7300 + N
    with tsr.Sampler(0, max_rows=64, max_vocab=V, max_k=N, seed=seed) as s:
        for step, prm in enumerate([dict(temperature=1.0), dict(temperature=0.8, top_k=50, top_p=0.9),
                                    dict(temperature=1.5, top_p=0.9), dict(temperature=0.0)]):
            parents, toks = make_trees(rows, N, V, tv, dv, prm, rng)
            print_case("tree_wide", dtype=dtype, V=V, N=N, params=prm)
            greedy = prm["temperature"] == 0.0
            st = torch.full((rows,), -7, dtype=torch.int32, device=device())
            t_dev = to_dev(tdata.reshape(-1, V), dtype).view(rows, N, V)
            d_dev = None if greedy else to_dev(ddata.reshape(-1, V), dtype).view(rows, N, V)
            out_t, out_p, acc = s.tree_verify(t_dev, d_dev, torch.from_numpy(parents).to(device()),
                                              torch.from_numpy(toks).to(device()), prm, step,
                                              status=st)
            torch.cuda.synchronize()
            out_t, out_p = out_t.cpu().numpy(), out_p.cpu().numpy()
            acc, st = acc.cpu().numpy(), st.cpu().numpy()
            t = Tally()
            for b in range(rows):
                r = oracle.tree_verify_row(tv[b], dv[b], parents[b], toks[b], prm, seed, b, step)
                compare_tree_row(t, b, r, out_t[b], out_p[b], acc[b], st[b])
            report(f"tree wide N={N} V={V} {dtype} {prm}", t)
