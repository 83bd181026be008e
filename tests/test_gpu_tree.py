"""GPU parity of tree_verify (multi-candidate speculation: brentwoodlivery.com
"Extensions and Variants"; the acceptance rule of gowda.ai section 39.4 at
each candidate) against the oracle, through the C ABI."""
import numpy as np
import pytest

from tests.gpu_common import Tally, device, gpu_available, report, to_dev, torch
from oracle.parity import compare_tree_row

import oracle
import token_sampling_row_amd as tsr
from token_sampling_row_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def print_case(name, **kw):
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def make_trees(rows, N, V, target, draft, prm, rng, dtype):
    """Random parents (an earlier node each) and, for every node's children,
    tokens drawn from the draft distribution q~ at that node (the oracle's
    chain), so acceptances and rejections both occur."""
    parents = np.full((rows, N), -1, dtype=np.int32)
    toks = np.zeros((rows, N), dtype=np.int32)
    P = oracle.Params.of(prm)
    for b in range(rows):
        for n in range(1, N):
            parents[b, n] = rng.integers(0, n)
        for n in range(1, N):
            v = parents[b, n]
            if P.temperature > 0:
                q = oracle.support(draft[b, v], P).p_tilde
                toks[b, n] = rng.choice(V, p=q / q.sum())
            else:
                toks[b, n] = int(np.argmax(target[b, v])) if rng.random() < 0.5 else rng.integers(0, V)
    return parents, toks


def run_and_check(s, tdata, ddata, dtype, parents, toks, prm, seed, step):
    rows, N, V = tdata.shape
    tv = oracle.values_from_stored(tdata.reshape(rows * N, V), dtype).reshape(rows, N, V)
    dv = oracle.values_from_stored(ddata.reshape(rows * N, V), dtype).reshape(rows, N, V)
    st = torch.full((rows,), -7, dtype=torch.int32, device=device())
    t_dev = to_dev(tdata.reshape(rows * N, V), dtype).view(rows, N, V)
    d_dev = to_dev(ddata.reshape(rows * N, V), dtype).view(rows, N, V)
    greedy = prm.get("temperature", 1.0) == 0.0
    out_t, out_p, acc = s.tree_verify(t_dev, None if greedy else d_dev,
                                      torch.from_numpy(parents).to(device()),
                                      torch.from_numpy(toks).to(device()), prm, step, status=st)
    torch.cuda.synchronize()
    out_t, out_p, acc, st = out_t.cpu().numpy(), out_p.cpu().numpy(), acc.cpu().numpy(), st.cpu().numpy()
    t = Tally()
    for b in range(rows):
        r = oracle.tree_verify_row(tv[b], dv[b], parents[b], toks[b], prm, seed, b, step)
        compare_tree_row(t, b, r, out_t[b], out_p[b], acc[b], st[b])
    report(f"tree N={N} V={V} {dtype} {prm}", t)
    return t.token_excused


@pytest.mark.parametrize("dtype,V", [("f32", 1000), ("f32", 32000), ("bf16", 777), ("bf16", 32000)])
@pytest.mark.parametrize("N", [1, 2, 7, 32])
def test_tree_grid(dtype, V, N):
    rng = np.random.default_rng(V * 3 + N + (1 if dtype == "bf16" else 0))
    rows = 12
    target = rng.normal(0, 1.5, (rows, N, V))
    draft = target + rng.normal(0, 0.7, (rows, N, V))
    tdata = target.astype(np.float32)
    ddata = draft.astype(np.float32)
    if dtype == "bf16":
        tdata, ddata = wl.f32_to_bf16_bits(tdata), wl.f32_to_bf16_bits(ddata)
    tv = oracle.values_from_stored(tdata.reshape(-1, V), dtype).reshape(rows, N, V)
    dv = oracle.values_from_stored(ddata.reshape(-1, V), dtype).reshape(rows, N, V)
    seed = 900 + V + N
    with tsr.Sampler(0, max_rows=256, max_vocab=1 << 16, max_k=31, seed=seed) as s:
        for i, prm in enumerate([dict(temperature=1.0), dict(temperature=0.8, top_k=40, top_p=0.9),
                                 dict(temperature=0.0)]):
            parents, toks = make_trees(rows, N, V, tv, dv, prm, rng, dtype)
            print_case("tree_grid", dtype=dtype, V=V, N=N, params=prm)
            ex = run_and_check(s, tdata, ddata, dtype, parents, toks, prm, seed, i)
            print(f"tree V={V} {dtype} N={N} {prm}: excused {ex}", flush=True)


def test_tree_bad_inputs():
    rng = np.random.default_rng(4)
    rows, N, V = 4, 5, 300
    target = rng.normal(0, 1, (rows, N, V)).astype(np.float32)
    draft = (target + rng.normal(0, 0.5, (rows, N, V))).astype(np.float32)
    parents = np.tile(np.array([-1, 0, 0, 1, 2], dtype=np.int32), (rows, 1))
    toks = rng.integers(0, V, (rows, N)).astype(np.int32)
    parents[1, 3] = 3                 # not an earlier node
    toks[2, 4] = V                    # out of range
    target[3, 2, 7] = np.nan          # a target row with NaN
    with tsr.Sampler(0, max_rows=64, max_vocab=1 << 16, max_k=8, seed=5) as s:
        print_case("tree_bad")
        run_and_check(s, target, draft, "f32", parents, toks, {"temperature": 1.0}, 5, 0)
        st = torch.zeros(rows, dtype=torch.int32, device=device())
        s.tree_verify(to_dev(target.reshape(-1, V), "f32").view(rows, N, V),
                      to_dev(draft.reshape(-1, V), "f32").view(rows, N, V),
                      torch.from_numpy(parents).to(device()), torch.from_numpy(toks).to(device()),
                      {"temperature": 1.0}, 0, status=st)
        assert st.cpu().numpy().tolist() == [0, 5, 3, 1]
