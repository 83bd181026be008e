"""GPU parity of beam_step (gowda.ai chapter 39, section 39.1: eq. 39.1 and
Listing 39.1) against the oracle, through the C ABI."""
import numpy as np
import pytest

from tests.gpu_common import BAND, device, gpu_available, to_dev, torch

import oracle
import token_sampling_row_amd as tsr
from token_sampling_row_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

SCORE_TOL = 1e-5   # log-probabilities: fp32 weights (~2 ulp) summed in fp64, as for log p~


def print_case(name, **kw):
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def run_beam(s, data, dtype, scores, beam):
    x = to_dev(data, dtype)
    sc = torch.from_numpy(np.asarray(scores, dtype=np.float64)).to(device())
    groups = data.shape[0] // beam
    st = torch.full((groups,), -7, dtype=torch.int32, device=device())
    par, tok, score = s.beam_step(x, sc, beam, status=st)
    torch.cuda.synchronize()
    return par.cpu().numpy(), tok.cpu().numpy(), score.cpu().numpy(), st.cpu().numpy()


def check(data, dtype, scores, beam):
    """Every group against oracle.beam_step; returns the number of positions
    excused by the band."""
    values = oracle.values_from_stored(data, dtype)
    groups = data.shape[0] // beam
    with tsr.Sampler(0, max_rows=4096, max_vocab=1 << 18) as s:
        par, tok, score, st = run_beam(s, data, dtype, scores, beam)
    excused = 0
    for g in range(groups):
        rows = slice(g * beam, (g + 1) * beam)
        r = oracle.beam_step(values[rows], np.asarray(scores)[rows], beam)
        assert st[g] == r.status, (g, st[g], r.status)
        if r.status == oracle.ROW_NONFINITE:
            assert (par[g] == -1).all() and (tok[g] == -1).all() and np.isnan(score[g]).all()
            continue
        for k in range(beam):
            want = r.score[k]
            if not np.isfinite(want):
                assert par[g, k] == -1 and tok[g, k] == -1 and score[g, k] == -np.inf, (g, k)
                continue
            if (par[g, k], tok[g, k]) == (r.parent[k], r.token[k]):
                assert abs(score[g, k] - want) <= SCORE_TOL * max(1.0, abs(want)), \
                    (g, k, score[g, k], want)
            else:
                near = r.gap[k] <= BAND or (k > 0 and r.gap[k - 1] <= BAND)
                assert near, (g, k, par[g, k], tok[g, k], r.parent[k], r.token[k], r.gap[k])
                assert abs(score[g, k] - want) <= SCORE_TOL * max(1.0, abs(want)) + BAND
                excused += 1
    return excused


def beam_rows(groups, beam, V, dtype, rng):
    rows = []
    for g in range(groups):
        a = (0.3, 0.8, 1.2, 2.0)[g % 4]
        for b in range(beam):
            r = -a * np.log(rng.permutation(V) + 1.0) + rng.normal(0, 0.5, V)
            if g % 5 == 3:
                r = np.round(r * 2) / 2          # ties
            rows.append(r)
    data = np.stack(rows).astype(np.float32)
    return wl.f32_to_bf16_bits(data) if dtype == "bf16" else data


@pytest.mark.parametrize("dtype,V", [("f32", 1), ("f32", 5), ("f32", 1000), ("f32", 32000),
                                     ("f32", 77824), ("bf16", 3), ("bf16", 4099),
                                     ("bf16", 128256), ("bf16", 155000)])
@pytest.mark.parametrize("beam", [1, 4, 16])
def test_beam_grid(dtype, V, beam):
    rng = np.random.default_rng(V * 31 + beam + (1 if dtype == "bf16" else 0))
    groups = 12 if V > 100000 else 24
    data = beam_rows(groups, beam, V, dtype, rng)
    scores = rng.normal(-5.0, 2.0, groups * beam)
    scores[1::7] = -np.inf                              # dead beams
    print_case("beam_grid", dtype=dtype, V=V, beam=beam)
    ex = check(data, dtype, scores, beam)
    print(f"beam V={V} {dtype} B={beam}: excused {ex}", flush=True)


def test_beam_ties_and_degenerate_rows():
    """A flat row (every logit tied: the row-wide fallback), a row with a tie
    group of a thousand at the top, an all -inf row, a NaN row, a group with
    every beam dead, and first-step groups (one live beam)."""
    V, beam = 70001, 4
    rng = np.random.default_rng(5)
    rows = [np.zeros(V)]                                            # group 0
    t = rng.normal(-5, 1, V); t[rng.choice(V, 1000, replace=False)] = 2.0
    rows += [t, rng.normal(0, 1, V), np.full(V, -np.inf)]
    rows += [rng.normal(0, 1, V) for _ in range(4)]                 # group 1: NaN
    rows[5][77] = np.nan
    rows += [rng.normal(0, 1, V) for _ in range(4)]                 # group 2: all dead
    rows += [rng.normal(0, 2, V) for _ in range(4)]                 # group 3: first step
    data = np.stack(rows).astype(np.float32)
    scores = np.zeros(16)
    scores[8:12] = -np.inf
    scores[13:16] = -np.inf
    print_case("beam_degenerate")
    check(data, "f32", scores, beam)
    with tsr.Sampler(0, max_rows=64, max_vocab=1 << 18) as s:
        _, _, _, st = run_beam(s, data, "f32", scores, beam)
    assert st.tolist() == [0, 1, 2, 0]


def test_beam_repeated_calls_reset_workspace():
    """Nothing of an earlier call reaches a later one's merge: after a call
    with a NaN group, two calls on clean logits give the same answers and
    every group status 0."""
    rng = np.random.default_rng(7)
    V, beam, groups = 5000, 8, 32
    data = beam_rows(groups, beam, V, "f32", rng)
    bad = data.copy(); bad[3 * beam, 10] = np.nan
    scores = rng.normal(-2, 1, groups * beam)
    with tsr.Sampler(0, max_rows=4096, max_vocab=1 << 18) as s:
        print_case("beam_repeat")
        run_beam(s, bad, "f32", scores, beam)
        a = run_beam(s, data, "f32", scores, beam)
        b = run_beam(s, data, "f32", scores, beam)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    assert (a[3] == 0).all()


def test_beam_argument_errors():
    with tsr.Sampler(0, max_rows=64, max_vocab=1 << 18) as s:
        x = to_dev(np.zeros((34, 100), np.float32), "f32")
        sc = torch.zeros(34, dtype=torch.float64, device=device())
        with pytest.raises(tsr.TsrError):
            s.beam_step(x, sc, 17)                              # beam > 16
        x2 = to_dev(np.zeros((68, 100), np.float32), "f32")
        with pytest.raises(tsr.TsrError):
            s.beam_step(x2, torch.zeros(68, dtype=torch.float64, device=device()), 4)   # > max_rows
        x3 = to_dev(np.zeros((4, 80000), np.float32), "f32")
        with pytest.raises(tsr.TsrError):
            s.beam_step(x3, torch.zeros(4, dtype=torch.float64, device=device()), 4)    # too wide


def test_beam_unaligned_rows():
    """Rows whose start is not 16-byte aligned (16-byte loads at any alignment)."""
    rng = np.random.default_rng(8)
    V, beam = 3001, 4
    base = rng.normal(0, 1.5, (16, V + 3)).astype(np.float32)
    data = np.ascontiguousarray(base[:, 1:V + 1])
    scores = rng.normal(-1, 1, 16)
    values = oracle.values_from_stored(data, "f32")
    with tsr.Sampler(0, max_rows=64, max_vocab=1 << 18) as s:
        x = to_dev(base, "f32")[:, 1:V + 1]
        sc = torch.from_numpy(scores).to(device())
        print_case("beam_unaligned")
        par, tok, score = s.beam_step(x, sc, beam)
        torch.cuda.synchronize()
    for g in range(4):
        r = oracle.beam_step(values[g * beam:(g + 1) * beam], scores[g * beam:(g + 1) * beam], beam)
        assert par[g].cpu().tolist() == list(r.parent) and tok[g].cpu().tolist() == list(r.token)
