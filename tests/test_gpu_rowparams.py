"""GPU parity of per-row sampling parameters (sample_rows_ex with row_params:
every row its own temperature, top-k, top-p, min-p and filter mode, checked
on the device) against the oracle, row by row, through the C ABI."""
import numpy as np
import pytest

from tests.gpu_common import Tally, compare, compare_logprob, device, gpu_available, to_dev, torch

import oracle
import token_sampling_row_amd as tsr
from token_sampling_row_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

CHOICES = [
    dict(temperature=0.9, top_k=50, top_p=0.95, min_p=0.1),
    dict(temperature=0.9, top_k=50, top_p=0.95, min_p=0.1, mode=1),
    dict(temperature=1.0),
    dict(temperature=0.0),
    dict(temperature=1.5, top_p=0.9),
    dict(temperature=0.7, top_k=5),
    dict(temperature=1.0, top_k=3000),
    dict(temperature=0.5, min_p=0.3),
    dict(temperature=2.0, top_k=1),
    dict(temperature=1.0, top_p=0.0),
]
BAD = [dict(temperature=-1.0), dict(temperature=1e-40), dict(temperature=1.0, top_p=-0.5),
       dict(temperature=float("nan")), dict(temperature=1.0, mode=7)]


def run_rows(s, data, dtype, plist, step):
    rows, V = data.shape
    rp = torch.from_numpy(tsr.pack_row_params(plist)).to(device())
    d = dict(status=torch.full((rows,), -7, dtype=torch.int32, device=device()),
             kept_count=torch.full((rows,), -7, dtype=torch.int32, device=device()),
             threshold=torch.full((rows,), float("nan"), dtype=torch.float32, device=device()),
             kept_mass=torch.full((rows,), float("nan"), dtype=torch.float64, device=device()),
             probs=torch.full((rows, V), float("nan"), dtype=torch.float32, device=device()))
    lp = torch.full((rows,), 123.0, dtype=torch.float32, device=device())
    out = s.sample_rows_ex(to_dev(data, dtype), None, step, logprob=lp, diag=d, row_params=rp)
    torch.cuda.synchronize()
    res = {k: t.cpu().numpy() for k, t in d.items()}
    res["token"] = out.cpu().numpy()
    res["logprob"] = lp.cpu().numpy()
    return res


@pytest.mark.parametrize("dtype,V", [("f32", 5), ("f32", 4099), ("f32", 70001), ("f32", 131072),
                                     ("bf16", 1000), ("bf16", 128256), ("bf16", 160001)])
def test_row_params_grid(dtype, V):
    """Each row draws its parameters from a list (greedy, filters of every
    kind, both modes) or an invalid set; rows held in registers and streamed."""
    rng = np.random.default_rng(V + (3 if dtype == "bf16" else 0))
    n = 24
    rows = [-a * np.log(rng.permutation(V) + 1.0) + rng.normal(0, 0.5, V)
            for a in rng.uniform(0.2, 1.4, n)]
    data = np.stack(rows).astype(np.float32)
    if dtype == "bf16":
        data = wl.f32_to_bf16_bits(data)
    values = oracle.values_from_stored(data, dtype)
    plist = [CHOICES[i % len(CHOICES)] for i in rng.permutation(n)]
    plist[3] = BAD[V % len(BAD)]
    plist[17] = BAD[(V + 2) % len(BAD)]
    seed = 6000 + V
    with tsr.Sampler(0, max_rows=4096, max_vocab=1 << 18, seed=seed) as s:
        for step in (0, 1):
            print(f"[case] row_params dtype={dtype} V={V} step={step}", flush=True)
            got = run_rows(s, data, dtype, plist, step)
            for b in (3, 17):
                assert got["status"][b] == tsr.ROW_BADPARAM and got["token"][b] == -1
                assert np.isnan(got["logprob"][b])
            good = [b for b in range(n) if b not in (3, 17)]
            refs = [oracle.sample_row(values[b], plist[b], seed, b, step) for b in good]
            for i, b in enumerate(good):
                greedy = plist[b].get("temperature", 1.0) == 0.0
                compare(got, [refs[i]], [b], values, greedy=greedy)
                if greedy:   # p~ is the point mass at the token (include/tsr.h)
                    assert got["kept_count"][b] == 1 and got["kept_mass"][b] == 1.0
                    assert np.float32(got["threshold"][b]) == np.float32(values[b].max())
                    if "probs" in got:
                        onehot = np.zeros(V, dtype=np.float32)
                        onehot[refs[i].token] = 1.0
                        assert np.array_equal(got["probs"][b], onehot), b
            compare_logprob(got, refs, good)


def test_row_params_uniform_equals_call_params():
    """The same parameters on every row give what the call-level parameters
    give, on the 256 x 128256 bf16 workload."""
    w = wl.config(3)
    seed = wl.philox_seed(3)
    with tsr.Sampler(0, max_rows=4096, max_vocab=1 << 18, seed=seed) as s:
        x = to_dev(w.data, w.dtype)
        print("[case] row_params_uniform", flush=True)
        a = s.sample_rows(x, w.runs[0], 9)
        rp = torch.from_numpy(tsr.pack_row_params([w.runs[0]] * w.rows)).to(device())
        b = s.sample_rows_ex(x, None, 9, row_params=rp)
        torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy(), b.cpu().numpy())
