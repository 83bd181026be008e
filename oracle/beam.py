"""Float64 oracle of one beam-search step. Test infrastructure only (see the
package docstring).

Pages cited:
  [P2] gowda.ai "Chapter 39 Decoding & Speculative Sampling", section 39.1
       (eq. 39.1, Listing 39.1).
  [P4] scratchllm.com "Efficient Inference & Compression", section
       "Beam search" (the two-step example).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .sampler import ROW_EMPTY, ROW_NONFINITE, ROW_OK

__all__ = ["BeamResult", "log_softmax_row", "beam_step", "beam_search"]


def log_softmax_row(l: np.ndarray) -> np.ndarray:
    """log p_i = (z_i - M) - ln sum_j exp(z_j - M), M the row maximum, in
    float64. Reading: a row with no finite logit carries no probability, so
    every token of it gets -inf."""
    l = np.asarray(l, dtype=np.float64)
    if not np.isfinite(l).any():
        return np.full(l.shape, -np.inf)
    m = l.max()
    with np.errstate(divide="ignore"):
        return (l - m) - np.log(np.sum(np.exp(l - m)))


@dataclass
class BeamResult:
    status: int              # ROW_OK, ROW_NONFINITE, or ROW_EMPTY (no finite candidate)
    parent: np.ndarray       # [B] beam the kept candidate extends (index within the group)
    token: np.ndarray        # [B] its token
    score: np.ndarray        # [B] its score, eq. 39.1
    gap: np.ndarray          # [B] score of candidate k minus that of candidate k + 1 in order


def beam_step(values: np.ndarray, scores, beam: int) -> BeamResult:
    """One step of P2 Listing 39.1 for one group: every beam b (row b of
    ``values``, running score scores[b]) is extended by every token i with
    score s_b + log p_b(i) (eq. 39.1 accumulates log-probabilities), and the
    ``beam`` best candidates are kept, best first (all of them when there are
    fewer, as the listing's slice does).

    Readings: candidates of equal score keep the order in which the listing
    enumerates them (beam b, then token i, ascending), since its sort is
    stable; a candidate of score -inf (a dead beam or a token without
    probability) ranks after every finite one; a NaN or +inf logit or score
    in the group leaves nothing defined (NONFINITE); a group without any
    finite candidate is EMPTY. No length penalty or end token (the listing
    omits them)."""
    v = np.asarray(values, dtype=np.float64)
    s = np.asarray(scores, dtype=np.float64)
    nb, V = v.shape
    empty = np.zeros(0)
    if np.isnan(v).any() or np.isposinf(v).any() or np.isnan(s).any() or np.isposinf(s).any():
        return BeamResult(ROW_NONFINITE, empty, empty, empty, empty)
    cand = np.concatenate([s[b] + log_softmax_row(v[b]) for b in range(nb)])
    order = np.argsort(-cand, kind="stable")
    top = order[:beam]                       # fewer when there are fewer candidates
    sc = cand[top]
    nxt = np.append(cand[order[1:top.size + 1]], -np.inf)[:top.size]
    with np.errstate(invalid="ignore"):
        gap = np.where(np.isfinite(sc), sc - nxt, np.inf)
    status = ROW_OK if np.isfinite(sc[0]) else ROW_EMPTY
    return BeamResult(status, top // V, top % V, sc, gap)


def beam_search(next_logits, prompt, steps: int, beam: int):
    """Listing 39.1 driven by beam_step: the beams (prefix, score) after
    ``steps`` extensions of ``prompt``; next_logits(prefix) -> logits."""
    beams = [(tuple(prompt), 0.0)]
    for _ in range(steps):
        rows = np.stack([np.asarray(next_logits(p), dtype=np.float64) for p, _ in beams])
        r = beam_step(rows, [sc for _, sc in beams], beam)
        beams = [(beams[int(b)][0] + (int(t),), float(sc))
                 for b, t, sc in zip(r.parent, r.token, r.score)]
    return beams
