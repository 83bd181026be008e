"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same stored bits, and compare row by row.

Parity rule: oracle/parity.py states it (BAND, PROB_RTOL) and applies it row
by row; the one tolerance added here:
  * log p~ of the drawn token (where token and kept set agree): absolute
    error <= LOGP_TOL * max(1, |log p~|). The kernel forms it in float64 from
    float32 weights exp2((v - M) * log2(e) / T), each within a few float32
    ulps (~3e-7 relative, so ~3e-7 absolute in the log), and rounds the result
    to float32 (2^-24 relative); 1e-5 covers both with room to spare.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle.parity import (BAND, F32_NORMAL_MIN, PROB_RTOL, Tally,  # noqa: F401
                           compare_sample_row)

LOGP_TOL = 1e-5

torch = pytest.importorskip("torch")


def gpu_available() -> bool:
    return torch.cuda.is_available()


def device():
    return torch.device("cuda:0")


def to_dev(data: np.ndarray, dtype: str):
    """Stored bits -> device tensor of the right element type."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(data).view(np.int16)).to(device()).view(
            torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(data, dtype=np.float32)).to(device())


def run_sample(sampler, x, params, step, diag=False, probs=False):
    rows, V = x.shape
    d = None
    if diag:
        d = dict(status=torch.full((rows,), -7, dtype=torch.int32, device=x.device),
                 kept_count=torch.full((rows,), -7, dtype=torch.int32, device=x.device),
                 threshold=torch.full((rows,), float("nan"), dtype=torch.float32, device=x.device),
                 kept_mass=torch.full((rows,), float("nan"), dtype=torch.float64, device=x.device),
                 probs=(torch.full((rows, V), float("nan"), dtype=torch.float32, device=x.device)
                        if probs else None))
    out = sampler.sample_rows(x, params, step, diag=d)
    torch.cuda.synchronize()
    res = {"token": out.cpu().numpy()}
    if d:
        for k, t in d.items():
            if t is not None:
                res[k] = t.cpu().numpy()
    return res


def run_masked(sampler, x, words, params, step, diag=True, probs=False):
    """sample_rows_masked through the C ABI; ``words`` is a uint32 [rows, W]
    numpy array or None. Returns token, logprob and the diagnostics."""
    rows, V = x.shape
    allowed = None
    if words is not None:
        allowed = torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(x.device)
    d = None
    if diag:
        d = dict(status=torch.full((rows,), -7, dtype=torch.int32, device=x.device),
                 kept_count=torch.full((rows,), -7, dtype=torch.int32, device=x.device),
                 threshold=torch.full((rows,), float("nan"), dtype=torch.float32, device=x.device),
                 kept_mass=torch.full((rows,), float("nan"), dtype=torch.float64, device=x.device),
                 probs=(torch.full((rows, V), float("nan"), dtype=torch.float32, device=x.device)
                        if probs else None))
    lp = torch.full((rows,), 12345.0, dtype=torch.float32, device=x.device)
    out = sampler.sample_rows_masked(x, allowed, params, step, logprob=lp, diag=d)
    torch.cuda.synchronize()
    res = {"token": out.cpu().numpy(), "logprob": lp.cpu().numpy()}
    if d:
        for k, t in d.items():
            if t is not None:
                res[k] = t.cpu().numpy()
    return res


def run_ex(sampler, x, params, step, words=None, hist=None, penalty=1.0, diag=True,
           probs=False):
    """sample_rows_ex through the C ABI: ``words`` a uint32 [rows, W] mask or
    None, ``hist`` an int32 [rows, H] window or None. Returns token, logprob
    and the diagnostics."""
    rows, V = x.shape
    allowed = history = None
    if words is not None:
        allowed = torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(x.device)
    if hist is not None:
        history = torch.from_numpy(np.ascontiguousarray(hist, dtype=np.int32)).to(x.device)
    d = None
    if diag:
        d = dict(status=torch.full((rows,), -7, dtype=torch.int32, device=x.device),
                 kept_count=torch.full((rows,), -7, dtype=torch.int32, device=x.device),
                 threshold=torch.full((rows,), float("nan"), dtype=torch.float32, device=x.device),
                 kept_mass=torch.full((rows,), float("nan"), dtype=torch.float64, device=x.device),
                 probs=(torch.full((rows, V), float("nan"), dtype=torch.float32, device=x.device)
                        if probs else None))
    lp = torch.full((rows,), 12345.0, dtype=torch.float32, device=x.device)
    out = sampler.sample_rows_ex(x, params, step, allowed=allowed, history=history,
                                 penalty=penalty, logprob=lp, diag=d)
    torch.cuda.synchronize()
    res = {"token": out.cpu().numpy(), "logprob": lp.cpu().numpy()}
    if d:
        for k, t in d.items():
            if t is not None:
                res[k] = t.cpu().numpy()
    return res


def compare_logprob(gpu: dict, refs: list, rows) -> int:
    """log p~ of the drawn tokens: NaN on bad rows, 0 on greedy rows, else the
    oracle's within LOGP_TOL wherever token and kept set agree (elsewhere the
    band rule of compare() already excused the row). Returns rows checked."""
    n = 0
    for i, b in enumerate(rows):
        r = refs[i]
        g = float(gpu["logprob"][b])
        if r.status != 0:
            assert np.isnan(g), (b, g)
            continue
        if r.support is None:          # greedy
            assert g == 0.0, (b, g)
            n += 1
            continue
        if gpu["token"][b] != r.token:
            continue
        s = r.support
        if "kept_count" in gpu and (gpu["kept_count"][b] != s.kept_count or
                                    np.float32(gpu["threshold"][b]) != np.float32(s.threshold)):
            continue
        assert g <= 0.0 or abs(g) <= LOGP_TOL, (b, g)
        assert abs(g - r.logprob) <= LOGP_TOL * max(1.0, abs(r.logprob)), (b, g, r.logprob)
        n += 1
    return n


def compare(gpu: dict, refs: list, rows, values: np.ndarray = None, greedy=False, tally=None,
            check_probs_rows=None) -> Tally:
    """Compare GPU outputs with oracle RowResults row by row under the parity
    rule of oracle.parity (raises ParityError on a mismatch no margin excuses);
    returns the tally of rows, rows in band and excused mismatches."""
    tally = tally if tally is not None else Tally()
    for i, b in enumerate(rows):
        probs = None
        if "probs" in gpu and (check_probs_rows is None or b in check_probs_rows):
            probs = gpu["probs"][b]
        compare_sample_row(
            tally, b, refs[i], gpu["token"][b],
            status=gpu["status"][b] if "status" in gpu else None,
            kept_count=gpu["kept_count"][b] if "kept_count" in gpu else None,
            threshold=gpu["threshold"][b] if "threshold" in gpu else None,
            kept_mass=gpu["kept_mass"][b] if "kept_mass" in gpu else None,
            probs=probs, greedy=greedy)
    return tally


def report(name: str, t: Tally) -> None:
    """One line per compared workload: the counts the parity rule asks for."""
    d = t.as_dict()
    print(f"parity {name}: rows={d['rows']} in_band={d['in_band']} "
          f"in_1e-9={d['in_tight_band']} support_excused={d['support_excused']} "
          f"token_excused={d['token_excused']} excused_above_1e-9={d['excused_above_1e-9']} "
          f"out_of_band={d['out_of_band']} max_p_rel_err={d['max_prob_rel_err']:.3g}", flush=True)
