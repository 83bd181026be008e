"""The parity rule: how a sampler's outputs are compared with the oracle's.

Test infrastructure only (see the package docstring). Plain NumPy over arrays
the caller has already copied to the host; nothing here runs or imports the
product path.

The rule (results identical to the oracle's, with one stated exception):
  * row status, greedy tokens and top-k decisions: exact (they compare input
    values, no rounding is involved);
  * the kept set, compared through |S| and the smallest kept logit: exact,
    unless the oracle's nearest top-p or min-p decision lies within BAND of
    its cut (Support.margin_p / margin_m), in which case the row is excused
    and not compared further;
  * the drawn token, once the kept set has matched: exact, unless the
    oracle's uniform lies within BAND of an end of the chosen token's CDF
    interval (RowResult.margin_draw). Where the kept set was not observed the
    kept set's margins may excuse the token as well;
  * verify / tree: the sequence is compared position by position; at the
    first position where the outputs differ, the mismatch is excused only by
    that position's own decisions (oracle.Decision): the acceptance test and
    the chains' cuts if the acceptance differs, the draw and the cuts if only
    the drawn token differs;
  * kept probabilities p~ (eq. 39.2) and the kept mass: relative error at most
    PROB_RTOL (on normal float32 values of p~).
BAND = 1e-6 and PROB_RTOL = 1e-5 are the tolerances the GPU path is held to.
TIGHT_BAND = 1e-9 is reported beside it: mismatches whose deciding margin is
above 1e-9 would mean an accumulation worse than the GPU path's design (fp64
sums of fp32 weights), and none is expected.

Every excused mismatch, every row whose deciding margins fall in the band and
every mismatch outside it is counted in a Tally, which the tests print and the
benchmark reports.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["BAND", "TIGHT_BAND", "PROB_RTOL", "F32_NORMAL_MIN", "Tally", "ParityError",
           "compare_sample_row", "compare_verify_row", "compare_tree_row"]

BAND = 1e-6
TIGHT_BAND = 1e-9
PROB_RTOL = 1e-5
F32_NORMAL_MIN = 1.1754943508222875e-38


class ParityError(AssertionError):
    pass


@dataclass
class Tally:
    rows: int = 0                 # rows (or sequences) compared
    in_band: int = 0              # rows with a deciding margin within BAND
    in_tight_band: int = 0        # ... within TIGHT_BAND
    support_excused: int = 0      # kept sets that differ, excused by their margin
    token_excused: int = 0        # tokens (or sequences) that differ, excused by their margin
    above_tight: int = 0          # excused mismatches whose deciding margin exceeds TIGHT_BAND
    out_of_band: int = 0          # mismatches no margin excuses (must stay 0)
    probs_rows: int = 0           # rows whose dense p~ was compared
    max_prob_rel_err: float = 0.0  # largest relative error of p~ / the kept mass
    notes: list = field(default_factory=list)
    eff: list = field(default_factory=list)    # per sampled row: e^H of p (effective choices)
    kept: list = field(default_factory=list)   # per sampled row: |S|

    def as_dict(self) -> dict:
        return {"rows": self.rows, "in_band": self.in_band, "in_tight_band": self.in_tight_band,
                "support_excused": self.support_excused, "token_excused": self.token_excused,
                "excused_above_1e-9": self.above_tight, "out_of_band": self.out_of_band,
                "probs_rows": self.probs_rows, "max_prob_rel_err": self.max_prob_rel_err,
                "band": BAND, "prob_rtol": PROB_RTOL}

    def merge(self, other: "Tally") -> "Tally":
        for k in ("rows", "in_band", "in_tight_band", "support_excused", "token_excused",
                  "above_tight", "out_of_band", "probs_rows"):
            setattr(self, k, getattr(self, k) + getattr(other, k))
        self.max_prob_rel_err = max(self.max_prob_rel_err, other.max_prob_rel_err)
        self.notes += other.notes
        self.eff += other.eff
        self.kept += other.kept
        return self

    def shape(self) -> dict:
        """The sampled rows' shape (legost.in "Temperature: one dial for
        boldness": the entropy H of p and its effective number of choices e^H;
        the kept-set size |S|): min / median / max over the rows."""
        out = {}
        for name, xs in (("effective_choices", self.eff), ("kept", self.kept)):
            if xs:
                a = np.asarray(xs, dtype=np.float64)
                out[name] = [float(a.min()), float(np.median(a)), float(a.max())]
        return out


def _fail(t: Tally, strict: bool, msg) -> None:
    t.out_of_band += 1
    t.notes.append(msg)
    if strict:
        raise ParityError(msg)


def _excuse(t: Tally, margin: float, kind: str) -> None:
    if kind == "support":
        t.support_excused += 1
    else:
        t.token_excused += 1
    if margin > TIGHT_BAND:
        t.above_tight += 1


def compare_sample_row(t: Tally, row: int, ref, token: int, status: int | None = None,
                       kept_count: int | None = None, threshold: float | None = None,
                       kept_mass: float | None = None, probs: np.ndarray | None = None,
                       greedy: bool = False, strict: bool = True) -> None:
    """One sampler row. ``ref`` is the oracle's RowResult; the other arguments
    are the GPU's outputs for the row (None where not observed)."""
    t.rows += 1
    if status is not None and int(status) != ref.status:
        _fail(t, strict, ("status", row, int(status), ref.status))
        return
    if greedy or ref.status != 0 or ref.support is None:
        if int(token) != ref.token:
            _fail(t, strict, ("token", row, int(token), ref.token))
        return
    s = ref.support
    ms, md = ref.margin_support, ref.margin_draw
    if min(ms, md) <= BAND:
        t.in_band += 1
    if min(ms, md) <= TIGHT_BAND:
        t.in_tight_band += 1
    if kept_count is not None and threshold is not None:
        same = int(kept_count) == s.kept_count and \
            np.float32(threshold) == np.float32(s.threshold)
        if not same:
            if ms <= BAND:
                _excuse(t, ms, "support")
            else:
                _fail(t, strict, ("kept set", row, int(kept_count), s.kept_count,
                                  float(threshold), s.threshold, ms))
            return
        deciding = md              # the kept set matched: only the draw decides
    else:
        deciding = min(ms, md)
    if kept_mass is not None:
        err = abs(float(kept_mass) - s.kept_mass) / s.kept_mass
        t.max_prob_rel_err = max(t.max_prob_rel_err, err)
        if not err <= PROB_RTOL:
            _fail(t, strict, ("kept mass", row, float(kept_mass), s.kept_mass))
    if int(token) != ref.token:
        if deciding <= BAND:
            _excuse(t, deciding, "token")
        else:
            _fail(t, strict, ("token", row, int(token), ref.token, deciding, ref.u))
    if probs is not None:
        t.probs_rows += 1
        pg = np.asarray(probs, dtype=np.float64)
        if not np.all(pg[~s.keep] == 0.0):
            _fail(t, strict, ("p~ outside S", row))
            return
        pr = s.p_tilde
        norm = pr >= F32_NORMAL_MIN
        err = float((np.abs(pg - pr)[norm] / pr[norm]).max(initial=0.0))
        t.max_prob_rel_err = max(t.max_prob_rel_err, err)
        if not err <= PROB_RTOL:
            _fail(t, strict, ("p~", row, err))


def compare_verify_row(t: Tally, row: int, ref, tokens, n_accepted: int, status: int | None,
                       strict: bool = True) -> None:
    """One speculative-verify sequence. ``ref`` is the oracle's VerifyResult;
    tokens [K+1], n_accepted and status are the GPU's."""
    t.rows += 1
    tokens = [int(x) for x in tokens]
    if status is not None and int(status) != ref.status:
        _fail(t, strict, ("status", row, int(status), ref.status))
        return
    ds = ref.margins
    if ds and min(d.smallest() for d in ds) <= BAND:
        t.in_band += 1
    if ds and min(d.smallest() for d in ds) <= TIGHT_BAND:
        t.in_tight_band += 1
    if tokens == ref.tokens and int(n_accepted) == ref.n_accepted:
        return
    g, o = int(n_accepted), ref.n_accepted
    m = min(g, o)
    K1 = len(ref.tokens)
    ok_shape = 0 <= g < K1 and tokens[:m] == ref.tokens[:m] and \
        all(x == -1 for x in tokens[g + 1:])
    if ref.status != 0 or not ds or not ok_shape or m >= len(ds):
        _fail(t, strict, ("verify", row, tokens, ref.tokens, g, o))
        return
    d = ds[m]
    # acceptance differs at m, or both stopped at m with different tokens
    deciding = min(d.accept, d.support) if g != o else min(d.draw, d.support)
    if deciding <= BAND:
        _excuse(t, deciding, "token")
    else:
        _fail(t, strict, ("verify", row, tokens, ref.tokens, g, o, m, d))


def compare_tree_row(t: Tally, row: int, ref, tokens, path, n_accepted: int,
                     status: int | None, strict: bool = True) -> None:
    """One tree-verify sequence. ``ref`` is the oracle's TreeResult (one
    Decision per visited node); tokens, path [N] (-1 padded), n_accepted and
    status are the GPU's."""
    t.rows += 1
    tokens = [int(x) for x in tokens]
    path = [int(x) for x in path]
    N = len(tokens)
    if status is not None and int(status) != ref.status:
        _fail(t, strict, ("status", row, int(status), ref.status))
        return
    if ref.status != 0:
        if any(x != -1 for x in tokens + path) or int(n_accepted) != 0:
            _fail(t, strict, ("tree bad row", row, tokens, path))
        return
    ds = ref.margins
    if ds and min(d.smallest() for d in ds) <= BAND:
        t.in_band += 1
    if ds and min(d.smallest() for d in ds) <= TIGHT_BAND:
        t.in_tight_band += 1
    want_t = ref.tokens + [-1] * (N - len(ref.tokens))
    want_p = ref.path + [-1] * (N - len(ref.path))
    if tokens == want_t and path == want_p and int(n_accepted) == len(ref.path):
        return
    g = int(n_accepted)
    gp = path[:g]
    # first visited node where the walks part: visit i is the root for i = 0,
    # else path[i - 1]; the walks agree on path[:i]
    i = 0
    while i < min(len(gp), len(ref.path)) and gp[i] == ref.path[i]:
        i += 1
    ok_shape = 0 <= g < N and tokens[:i] == ref.tokens[:i]
    if not ok_shape or i >= len(ds):
        _fail(t, strict, ("tree", row, tokens, want_t, path, want_p))
        return
    d = ds[i]
    if gp == ref.path:            # same walk, different final draw
        deciding = min(d.draw, d.support)
    else:                         # a different child kept (or none) at visit i
        deciding = min(d.accept, d.support)
    if deciding <= BAND:
        _excuse(t, deciding, "token")
    else:
        _fail(t, strict, ("tree", row, tokens, want_t, path, want_p, i, d))


# ---------------------------------------------------------------- batches
# The oracle over a whole batch, in a pool of forked worker processes (the
# oracle is slow: ~40 ms per row of 128256 logits). Workers inherit the job
# through the fork and return one Tally each.

_JOB: dict = {}


def _sample_chunk(rows) -> Tally:
    from .sampler import sample_row
    j = _JOB
    t = Tally()
    g = j["gpu"]
    for b in rows:
        ref = sample_row(j["values"][b], j["params"], j["seed"], b, j["step"])
        if ref.support is not None:
            p = ref.support.p
            nz = p > 0
            t.eff.append(float(np.exp(-np.sum(p[nz] * np.log(p[nz])))))
            t.kept.append(ref.support.kept_count)
        probs = g["probs"][b] if ("probs" in g and b in j["probs_rows"]) else None
        compare_sample_row(t, b, ref, g["token"][b],
                           status=g["status"][b] if "status" in g else None,
                           kept_count=g["kept_count"][b] if "kept_count" in g else None,
                           threshold=g["threshold"][b] if "threshold" in g else None,
                           kept_mass=g["kept_mass"][b] if "kept_mass" in g else None,
                           probs=probs, greedy=j["greedy"], strict=False)
    return t


def parity_sample_batch(values: np.ndarray, params, seed: int, step: int, gpu: dict,
                        rows=None, probs_rows=None, procs: int = 16) -> Tally:
    """Compare a GPU sample_rows result over ``rows`` of a [B, V] batch (float64
    values) with the oracle, in ``procs`` forked processes. ``gpu`` holds host
    arrays: token and, optionally, status, kept_count, threshold, kept_mass,
    probs [B, V] (compared on ``probs_rows``, default every row). Returns the
    merged Tally (not strict: mismatches are counted, never raised)."""
    import multiprocessing as mp
    from .sampler import Params
    rows = list(range(values.shape[0])) if rows is None else list(rows)
    probs_rows = set(rows if probs_rows is None else probs_rows)
    _JOB.clear()
    _JOB.update(values=values, params=params, seed=seed, step=step, gpu=gpu,
                probs_rows=probs_rows, greedy=Params.of(params).temperature == 0.0)
    procs = max(1, min(procs, len(rows)))
    chunks = [rows[i::procs] for i in range(procs)]
    try:
        if procs == 1:
            parts = [_sample_chunk(rows)]
        else:
            with mp.get_context("fork").Pool(procs) as pool:
                parts = pool.map(_sample_chunk, chunks)
    finally:
        _JOB.clear()
    t = Tally()
    for p in parts:
        t.merge(p)
    return t


def parity_verify_batch(target: np.ndarray, draft: np.ndarray, draft_tokens, params,
                        seed: int, step: int, tokens, accepted, status=None) -> Tally:
    """Compare a GPU spec_verify result ([B, K+1] tokens, [B] accepted, [B]
    status or None) with oracle.spec_verify_row on every sequence (not strict)."""
    from .sampler import spec_verify_row
    t = Tally()
    for b in range(target.shape[0]):
        ref = spec_verify_row(target[b], draft[b], draft_tokens[b], params, seed, b, step)
        compare_verify_row(t, b, ref, tokens[b], accepted[b],
                           None if status is None else status[b], strict=False)
    return t
