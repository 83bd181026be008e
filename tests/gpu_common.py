"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same stored bits, and compare row by row.

Parity rule (tolerances written here, used by every GPU test):
  * status, greedy tokens: bit-exact.
  * kept set (|S| and the smallest kept logit): exact, unless the oracle's
    nearest top-p / min-p decision lies within BAND of its cut.
  * sampled token: exact, unless the oracle's uniform lies within BAND of the
    end of the chosen token's CDF interval (or a kept-set decision is within
    BAND, which can move the interval).
  * kept probabilities p~ (eq. 39.2): relative error <= PROB_RTOL where the
    oracle's p~ is a normal float32; kept mass: relative error <= PROB_RTOL.
  * log p~ of the drawn token (where token and kept set agree): absolute
    error <= LOGP_TOL * max(1, |log p~|). The kernel forms it in float64 from
    float32 weights exp2((v - M) * log2(e) / T), each within a few float32
    ulps (~3e-7 relative, so ~3e-7 absolute in the log), and rounds the result
    to float32 (2^-24 relative); 1e-5 covers both with room to spare.
BAND = 1e-6 and PROB_RTOL = 1e-5 are the tolerances the work is held to.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import pytest

BAND = 1e-6
PROB_RTOL = 1e-5
LOGP_TOL = 1e-5
F32_NORMAL_MIN = 1.1754943508222875e-38

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


@dataclass
class Tally:
    rows: int = 0
    token_excused: int = 0
    support_excused: int = 0
    in_band: int = 0
    notes: list = field(default_factory=list)


def compare(gpu: dict, refs: list, rows, values: np.ndarray, greedy=False, tally=None,
            check_probs_rows=None):
    """Compare GPU outputs with oracle RowResults; raise on a mismatch outside the band."""
    tally = tally or Tally()
    for i, b in enumerate(rows):
        r = refs[i]
        tally.rows += 1
        if "status" in gpu:
            assert gpu["status"][b] == r.status, (b, gpu["status"][b], r.status)
        if greedy or r.status != 0:
            assert gpu["token"][b] == r.token, (b, gpu["token"][b], r.token)
            continue
        s = r.support
        sup_margin = min(s.margin_p, s.margin_m)
        if sup_margin <= BAND or r.margin <= BAND:
            tally.in_band += 1
        if "kept_count" in gpu:
            same = gpu["kept_count"][b] == s.kept_count and \
                np.float32(gpu["threshold"][b]) == np.float32(s.threshold)
            if not same:
                assert sup_margin <= BAND, (b, gpu["kept_count"][b], s.kept_count,
                                            gpu["threshold"][b], s.threshold, sup_margin)
                tally.support_excused += 1
                continue
            if "kept_mass" in gpu:
                assert abs(gpu["kept_mass"][b] - s.kept_mass) <= PROB_RTOL * s.kept_mass, \
                    (b, gpu["kept_mass"][b], s.kept_mass)
        if gpu["token"][b] != r.token:
            assert r.margin <= BAND, (b, gpu["token"][b], r.token, r.margin, r.u)
            tally.token_excused += 1
        if "probs" in gpu and (check_probs_rows is None or b in check_probs_rows):
            pg = gpu["probs"][b].astype(np.float64)
            pr = s.p_tilde
            assert np.all(pg[~s.keep] == 0.0), b
            norm = pr >= F32_NORMAL_MIN
            err = np.abs(pg - pr)[norm] / pr[norm]
            assert err.max(initial=0.0) <= PROB_RTOL, (b, err.max())
    return tally
