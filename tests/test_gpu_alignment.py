"""Rows at every element offset inside a 16-byte block, through the entry
points that read rows into registers (and the streaming kernel past the
register file): sample_rows, greedy_argmax, beam_step and spec_verify, against
the oracle. The rows are views into a wider batch whose row stride is a whole
number of 16-byte blocks, so every row starts `off` elements past a block
boundary; the loads are 16 bytes wide at whatever alignment the row has."""
import numpy as np
import pytest

from tests.gpu_common import (BAND, Tally, compare, device, gpu_available, report, run_sample,
                              to_dev, torch)
from oracle.parity import compare_verify_row

import oracle
import token_sampling_row_amd as tsr
from token_sampling_row_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

EPC = {"f32": 4, "bf16": 8}
PARAMS = [dict(temperature=0.9, top_k=50, top_p=0.95, min_p=0.1), dict(temperature=1.0),
          dict(temperature=1.5, top_p=0.9), dict(temperature=0.0)]


def print_case(name, **kw):
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def zipf_rows(rng, rows, width, dtype):
    data = np.stack([-a * np.log(rng.permutation(width) + 1.0) + rng.normal(0.0, 0.5, width)
                     for a in np.linspace(0.3, 1.4, rows)]).astype(np.float32)
    return wl.f32_to_bf16_bits(data) if dtype == "bf16" else data


@pytest.mark.parametrize("dtype,V", [("f32", 4088), ("f32", 77816), ("bf16", 65528),
                                     ("bf16", 127992), ("bf16", 200000)])
def test_sample_and_greedy_at_every_offset(dtype, V):
    """V + 8 elements per stored row: a whole number of 16-byte blocks, so the
    view [off, off + V) of every row starts at the same offset."""
    rows = 6
    rng = np.random.default_rng(V + EPC[dtype])
    data = zipf_rows(rng, rows, V + 8, dtype)
    seed = 9100 + V
    with tsr.Sampler(0, max_rows=64, max_vocab=1 << 18, max_k=8, seed=seed) as s:
        dev = to_dev(data, dtype)
        for off in range(EPC[dtype]):
            x = dev[:, off:off + V]
            values = oracle.values_from_stored(np.ascontiguousarray(data[:, off:off + V]), dtype)
            for i, prm in enumerate(PARAMS):
                print_case("offset_sample", dtype=dtype, V=V, off=off, params=prm)
                refs = [oracle.sample_row(values[b], prm, seed, b, i) for b in range(rows)]
                got = run_sample(s, x, prm, i, diag=True)
                report(f"offset {off} V={V} {dtype} {prm}",
                       compare(got, refs, list(range(rows)), values,
                               greedy=prm["temperature"] == 0.0))
            got = s.greedy_argmax(x).cpu().numpy()
            assert got.tolist() == [int(np.argmax(r)) for r in values], off


@pytest.mark.parametrize("dtype,V", [("f32", 32000), ("bf16", 127992)])
def test_beam_at_every_offset(dtype, V):
    beam, groups = 4, 2
    rng = np.random.default_rng(V * 3 + EPC[dtype])
    data = zipf_rows(rng, beam * groups, V + 8, dtype)
    scores = rng.normal(-3.0, 1.0, beam * groups)
    with tsr.Sampler(0, max_rows=64, max_vocab=1 << 18) as s:
        dev = to_dev(data, dtype)
        sc = torch.from_numpy(scores).to(device())
        for off in range(EPC[dtype]):
            print_case("offset_beam", dtype=dtype, V=V, off=off)
            par, tok, _ = s.beam_step(dev[:, off:off + V], sc, beam)
            torch.cuda.synchronize()
            par, tok = par.cpu().numpy(), tok.cpu().numpy()
            values = oracle.values_from_stored(np.ascontiguousarray(data[:, off:off + V]), dtype)
            for g in range(groups):
                rs = slice(g * beam, (g + 1) * beam)
                r = oracle.beam_step(values[rs], scores[rs], beam)
                for k in range(beam):
                    if (par[g, k], tok[g, k]) != (r.parent[k], r.token[k]):
                        assert r.gap[k] <= BAND or (k > 0 and r.gap[k - 1] <= BAND), (off, g, k)


@pytest.mark.parametrize("dtype,V", [("f32", 4096), ("bf16", 4096), ("bf16", 128000)])
def test_verify_at_every_offset(dtype, V):
    """spec_verify takes contiguous [B, K + 1, V] and [B, K, V] batches: both
    start `off` elements into a buffer, so every row does (V is a multiple of
    eight); the narrow two-row kernel and the wide path."""
    B, K = 4, 3
    rng = np.random.default_rng(V + 11 * EPC[dtype])
    tgt, dft = wl.verify_batch(9200 + V, B, K, V, dtype)
    tv = oracle.values_from_stored(tgt.reshape(-1, V), dtype).reshape(B, K + 1, V)
    dv = oracle.values_from_stored(dft.reshape(-1, V), dtype).reshape(B, K, V)
    seed = 9300 + V
    with tsr.Sampler(0, max_rows=64, max_vocab=1 << 18, max_k=K, seed=seed) as s:
        for off in range(EPC[dtype]):
            pad = np.zeros(off, dtype=tgt.dtype)   # the batches start `off` elements in
            t_dev = to_dev(np.concatenate([pad, tgt.reshape(-1)]), dtype)[off:]
            d_dev = to_dev(np.concatenate([pad, dft.reshape(-1)]), dtype)[off:]
            t_dev = t_dev.view(B, K + 1, V)
            d_dev = d_dev.view(B, K, V)
            for step, prm in enumerate([dict(temperature=1.0), dict(temperature=0.8, top_k=50, top_p=0.9),
                                        dict(temperature=0.0)]):
                greedy = prm["temperature"] == 0.0
                xs = np.zeros((B, K), dtype=np.int32)
                for b in range(B):
                    for j in range(K):
                        xs[b, j] = (int(np.argmax(tv[b, j])) if rng.random() < 0.6
                                    else int(rng.integers(0, V)))
                print_case("offset_verify", dtype=dtype, V=V, off=off, params=prm)
                st = torch.full((B,), -7, dtype=torch.int32, device=device())
                toks, acc = s.spec_verify(t_dev, None if greedy else d_dev,
                                          torch.from_numpy(xs).to(device()), prm, step, out_status=st)
                torch.cuda.synchronize()
                toks, acc, st_h = toks.cpu().numpy(), acc.cpu().numpy(), st.cpu().numpy()
                t = Tally()
                for b in range(B):
                    r = oracle.spec_verify_row(tv[b], dv[b], xs[b], prm, seed, b, step)
                    compare_verify_row(t, b, r, toks[b], acc[b], st_h[b])
                report(f"offset verify {off} V={V} {dtype} {prm}", t)
