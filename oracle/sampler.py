"""Float64 oracle of the filter chain, the draw and the speculative verify step.

Test infrastructure only (see the package docstring). Every step follows a
passage of the pages; where the pages leave a choice open the reading taken is
named in the docstring of the function that makes it.

Pages cited:
  [P1] fareedkhan-dev.github.io "Inference: Sampling, the KV Cache, Speculative
       Decoding and int8", sections "Picking the next token" and
       "Speculative decoding".
  [P2] gowda.ai "Chapter 39 Decoding & Speculative Sampling", sections 39.1,
       39.2 (eq. 39.2, Listing 39.2), 39.3, 39.4 (eqs. 39.3, 39.4,
       Listings 39.4, 39.5).
  [P3] brentwoodlivery.com "Speculative decoding - Hinglish notes", sections
       "The Algorithm (Step-by-Step)", "Batching Speculation",
       "Temperature and Sampling".
  [P4] scratchllm.com "Efficient Inference & Compression", section
       "Speculative decoding".
  [P5] legost.in "Choosing the next word", sections "Temperature: one dial for
       boldness", "The repetition penalty", "Cutting off the tail: top-k and
       top-p", "Where the randomness comes from, and where it stops".
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .philox import DOMAIN_SAMPLE, DOMAIN_SPEC, draw_words, uniforms_from_words

__all__ = [
    "ROW_OK", "ROW_NONFINITE", "ROW_EMPTY", "ROW_BADTOKEN", "JOINT", "SEQUENTIAL",
    "InvalidParams", "Params", "check_params", "row_status", "greedy_token",
    "softmax", "Support", "support", "draw_from", "sample_row", "sample_batch",
    "greedy_batch", "accept_probability", "residual", "spec_verify_row",
    "spec_verify_batch", "acceptance_probability", "expected_accepted_prefix",
    "values_from_stored", "allowed_from_words", "mask_logits", "log_p_tilde",
    "round_to_element", "repetition_penalty", "HISTORY_MAX", "Decision",
]

ROW_OK, ROW_NONFINITE, ROW_EMPTY, ROW_BADTOKEN = 0, 1, 2, 3
# Smallest positive temperature accepted: below it log2(e) / T leaves float32's
# range in the GPU path, so both sides reject it rather than disagree.
TEMPERATURE_MIN = 1e-30
JOINT, SEQUENTIAL = 0, 1
# The look-back window of the repetition penalty (P5 "The repetition penalty").
HISTORY_MAX = 64


class InvalidParams(ValueError):
    pass


@dataclass(frozen=True)
class Params:
    """Sampling knobs [P1 "Picking the next token"; P2 Listing 39.2].

    temperature  >= 1e-30 samples softmax(z / T); 0 is greedy (the T -> 0 limit, P2
                 section 39.2; P5 "Temperature"). Not clamped.
    top_k        active iff 0 < top_k < V; 0 or >= V switches it off.
    top_p        active iff top_p < 1; must be >= 0.
    min_p        active iff 0 < min_p < 1 (the guard in P1's min-p snippet).
    mode         JOINT: every filter reads the same post-temperature p and the
                 kept set is the intersection, renormalised once (P2 Listing
                 39.2, eq. 39.2). SEQUENTIAL: top-p measures mass against what
                 top-k kept (P5's generation loop: top-k, softmax, then top-p).
    """

    temperature: float = 1.0
    top_k: int = 0
    top_p: float = 1.0
    min_p: float = 0.0
    mode: int = JOINT

    @staticmethod
    def of(d) -> "Params":
        if isinstance(d, Params):
            return d
        return Params(float(d.get("temperature", 1.0)), int(d.get("top_k", 0)),
                      float(d.get("top_p", 1.0)), float(d.get("min_p", 0.0)),
                      int(d.get("mode", JOINT)))


def check_params(p: Params) -> None:
    """Reject what no reading of the pages makes meaningful."""
    for name in ("temperature", "top_p", "min_p"):
        if not np.isfinite(getattr(p, name)):
            raise InvalidParams(f"{name} must be finite")
    if p.temperature < 0 or 0.0 < p.temperature < TEMPERATURE_MIN:
        raise InvalidParams("temperature must be 0 or >= 1e-30")
    if p.top_p < 0:
        raise InvalidParams("top_p must be >= 0")
    if p.mode not in (JOINT, SEQUENTIAL):
        raise InvalidParams("unknown filter mode")


def values_from_stored(data: np.ndarray, dtype: str) -> np.ndarray:
    """Stored fp32 values or bf16 bit patterns -> exact float64 values."""
    if dtype == "bf16":
        bits = np.asarray(data, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(data, dtype=np.float32).astype(np.float64)


def row_status(l: np.ndarray) -> int:
    """A row holding NaN or +inf has no distribution; an all -inf row has an
    empty support, the invalid state of P2 section 39.3."""
    if np.isnan(l).any() or np.isposinf(l).any():
        return ROW_NONFINITE
    if l.size == 0 or np.isneginf(l).all():
        return ROW_EMPTY
    return ROW_OK


def allowed_from_words(words, vocab: int) -> np.ndarray:
    """Allowed set from a packed bitmask: token i is allowed iff bit i % 32 of
    word i // 32 is set (the layout of sample_rows_masked)."""
    w = np.asarray(words, dtype=np.uint32)
    i = np.arange(vocab)
    return ((w[i // 32] >> (i % 32).astype(np.uint32)) & 1).astype(bool)


def mask_logits(l: np.ndarray, allowed) -> np.ndarray:
    """Constrained decoding (P2 section 39.3): every token outside the allowed
    set gets logit -inf before anything else, so every later step (temperature,
    softmax, the filters, eq. 39.2) sees the distribution conditioned on the
    allowed set. Reading: a disallowed entry is replaced whatever its value, a
    NaN or +inf included (the page's mask_logits selects -inf without reading
    the logit)."""
    return np.where(np.asarray(allowed, dtype=bool), np.asarray(l, dtype=np.float64), -np.inf)


def round_to_element(x, dtype: str) -> np.ndarray:
    """x rounded to the element type of the logits: float32 by round to nearest
    even, and for bf16 from that float32 to bf16, again to nearest even on the
    16 dropped bits. NaN and infinities pass unchanged. Returned as float64."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype != "bf16":
        return f.astype(np.float64)
    b = f.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1                      # ties go to the even bf16 neighbour
    rounded = ((b + 0x7FFF + lsb) >> 16) << 16
    keep = ~np.isfinite(f)                   # inf and NaN as they are
    out = np.where(keep, b, rounded).astype(np.uint32)
    return out.view(np.float32).astype(np.float64)


def repetition_penalty(l: np.ndarray, history, r: float, dtype: str = "f32") -> np.ndarray:
    """The CTRL repetition penalty as P5 "The repetition penalty" states it:
    before anything else, every token found in the look-back window (the last
    HISTORY_MAX tokens) has its logit rescaled by r: z / r if z > 0, z * r if
    z <= 0, so for r > 1 both branches lower it.

    Readings: a token that occurs several times in the window is rescaled once
    (the page rescales "each token it finds there", a set); ids outside
    [0, V) are ignored (window padding); r >= 1 and r = 1 changes nothing. The
    rescaled logit is rounded to the logits' element type (round_to_element):
    the sampler keeps each row in its input type, so both sides take every
    later decision on the same rounded value."""
    l = np.array(l, dtype=np.float64)
    ids = np.unique([int(h) for h in history if 0 <= int(h) < l.size]).astype(np.int64)
    if r == 1.0 or ids.size == 0:
        return l
    z = l[ids]
    with np.errstate(over="ignore"):
        pen = np.where(z > 0, z / r, z * r)
    l[ids] = round_to_element(pen, dtype)
    return l


def log_p_tilde(l: np.ndarray, keep: np.ndarray, token: int, temperature: float) -> float:
    """log p~(token) under eq. 39.2: z_token - log sum_{j in S} e^{z_j},
    z = (l - max l) / T, in float64 (shifted so no weight of S underflows
    before the log)."""
    l = np.asarray(l, dtype=np.float64)
    z = (l - l.max()) / temperature
    return float(z[token] - np.log(np.sum(np.exp(z[keep]))))


def greedy_token(l: np.ndarray) -> int:
    """x = argmax_i p_i (P2 section 39.1); ties go to the lowest token id."""
    return int(np.argmax(l))


def softmax(z: np.ndarray) -> np.ndarray:
    """Stable float64 softmax: shift by the max, exponentiate, divide (P2 Listing 39.2)."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - np.max(z))
    return e / e.sum()


@dataclass
class Support:
    keep: np.ndarray          # bool [V]: the kept set S
    p: np.ndarray             # float64 [V]: softmax(z / T)
    p_tilde: np.ndarray       # float64 [V]: eq. 39.2
    kept_count: int
    kept_mass: float          # sum of p over S
    threshold: float          # smallest kept logit
    margin_p: float           # distance of the nearest top-p decision from its cut
    margin_m: float           # distance of the nearest min-p decision from its cut


def support(l: np.ndarray, prm: Params, p: np.ndarray | None = None) -> Support:
    """The kept set S and eq. 39.2 for one row of logits (temperature > 0).

    Order key: tokens are ranked by their logit value (temperature is monotone),
    so equal logits form one group that is kept or dropped whole.

    top-k   keep i iff fewer than k tokens have a strictly larger logit. Tokens
            tied with the k-th largest stay (P2 Listing 39.2 keeps p >= cutoff;
            P5's loop masks only logits below the k-th value).
    top-p   sort by logit, descending; keep a group iff the mass strictly above
            it is below top_p * Z_ref, and always keep the top group. This is
            the smallest head whose mass reaches top_p (P5's k* formula; P2's
            searchsorted side="left" then stop + 1). Z_ref is 1 in JOINT mode
            and the top-k survivors' mass in SEQUENTIAL mode.
    min-p   keep i iff p_i >= min_p * max_j p_j (P1 "Picking the next token").
    renorm  p~ = p 1{S} / sum_S p (eq. 39.2).

    ``p`` may be given directly (tests that state probabilities); it defaults
    to softmax(l / T).
    """
    l = np.asarray(l, dtype=np.float64)
    V = l.size
    if p is None:
        p = softmax(l / prm.temperature)
    finite = np.isfinite(l)
    lmax = l.max()
    keep_k = np.ones(V, dtype=bool)
    keep_p = np.ones(V, dtype=bool)
    keep_m = np.ones(V, dtype=bool)
    k_on = 0 < prm.top_k < V
    p_on = prm.top_p < 1.0
    m_on = 0.0 < prm.min_p < 1.0

    if k_on:
        ascending = np.sort(l)
        n_greater = V - np.searchsorted(ascending, l, side="right")
        keep_k = n_greater < prm.top_k

    mass_above = None
    z_ref = 1.0
    if p_on:
        order = np.argsort(-l, kind="stable")
        sl, sp = l[order], p[order]
        cum = np.cumsum(sp)
        first = np.searchsorted(-sl, -sl, side="left")
        above_sorted = np.where(first > 0, cum[np.maximum(first - 1, 0)], 0.0)
        mass_above = np.empty(V)
        mass_above[order] = above_sorted
        if prm.mode == SEQUENTIAL and k_on:
            z_ref = float(p[keep_k & finite].sum())
        keep_p = (mass_above < prm.top_p * z_ref) | (l == lmax)

    if m_on:
        keep_m = p >= prm.min_p * p.max()

    keep = finite & keep_k & keep_p & keep_m

    margin_p = np.inf
    if p_on:
        cand = finite & keep_k & keep_m & (l != lmax)
        if cand.any():
            margin_p = float(np.min(np.abs(mass_above[cand] - prm.top_p * z_ref)) / z_ref)
    margin_m = np.inf
    if m_on:
        cand = finite & keep_k & keep_p
        if cand.any():
            margin_m = float(np.min(np.abs(p[cand] - prm.min_p * p.max())) / p.max())

    kept_mass = float(p[keep].sum())
    p_tilde = np.where(keep, p, 0.0) / kept_mass
    return Support(keep, p, p_tilde, int(keep.sum()), kept_mass,
                   float(l[keep].min()), margin_p, margin_m)


def draw_from(weights: np.ndarray, keep: np.ndarray, u: float):
    """Inverse-CDF draw over the kept tokens in ascending token id.

    Walk the kept tokens adding their weights and stop at the first whose
    running total passes u (P5 "Where the randomness comes from"): the first
    i in S with u * Z < C_i, C_i = sum of weights of kept j <= i. If rounding
    leaves u * Z at or past the last total, the last kept token of positive
    weight is taken. Returns (token, margin): margin is the distance of u from
    the nearer end of the token's interval, in units of the total.
    """
    idx = np.flatnonzero(keep)
    w = np.asarray(weights, dtype=np.float64)[idx]
    C = np.cumsum(w)
    Z = C[-1]
    target = u * Z
    pos = int(np.searchsorted(C, target, side="right"))
    if pos >= idx.size:
        pos = int(np.flatnonzero(w > 0)[-1])
    lo = C[pos - 1] if pos > 0 else 0.0
    margin = float(min(target - lo, C[pos] - target) / Z)
    return int(idx[pos]), margin


@dataclass
class RowResult:
    token: int
    status: int
    support: Support | None = None
    u: float = float("nan")
    margin_draw: float = float("inf")
    logprob: float = float("nan")   # log p~(token); 0 for greedy; nan for bad rows

    @property
    def margin_support(self) -> float:
        """Nearest top-p or min-p decision of the kept set (inf without one)."""
        if self.support is None:
            return float("inf")
        return min(self.support.margin_p, self.support.margin_m)

    @property
    def margin(self) -> float:
        """Nearest decision of any kind: the kept set's or the draw's."""
        return min(self.margin_draw, self.margin_support)


def sample_row(l: np.ndarray, params, seed: int, row: int, step: int,
               allowed=None, history=None, penalty: float = 1.0,
               dtype: str = "f32") -> RowResult:
    """One row of the sampler: status, greedy or chain + draw.

    The uniform is u = w0 * 2^-32 with w0 the first Philox4x32-10 word of
    counter (row, 0 | SAMPLE << 16, step) under key = seed. ``history`` (ids
    of the recent tokens, or None) and ``penalty`` apply the repetition
    penalty to the raw logits first (P5), ``dtype`` being the logits' element
    type; ``allowed`` (a bool [V], or None for every token) then masks the row
    (P2 section 39.3); an allowed set without a finite logit is the empty
    state. The result carries log p~ of the drawn token (0 under greedy
    decoding, where p~ is a point mass).
    """
    prm = Params.of(params)
    check_params(prm)
    l = np.asarray(l, dtype=np.float64)
    if history is not None:
        l = repetition_penalty(l, history, penalty, dtype)
    if allowed is not None:
        l = mask_logits(l, allowed)
    st = row_status(l)
    if st != ROW_OK:
        return RowResult(-1, st)
    if prm.temperature == 0.0:
        return RowResult(greedy_token(l), ROW_OK, logprob=0.0)
    s = support(l, prm)
    u = float(uniforms_from_words(draw_words(seed, [row], 0, step, DOMAIN_SAMPLE)[:, 0])[0])
    tok, margin = draw_from(s.p, s.keep, u)
    return RowResult(tok, ROW_OK, s, u, margin, log_p_tilde(l, s.keep, tok, prm.temperature))


def sample_batch(values: np.ndarray, params, seed: int, step: int, rows=None, allowed=None):
    """sample_row over a [B, V] float64 batch; ``rows`` picks a subset of rows;
    ``allowed`` is a bool [B, V] mask or None."""
    rows = range(values.shape[0]) if rows is None else rows
    return [sample_row(values[b], params, seed, b, step,
                       None if allowed is None else allowed[b]) for b in rows]


def greedy_batch(values: np.ndarray):
    out = []
    for l in values:
        st = row_status(l)
        out.append((greedy_token(l) if st == ROW_OK else -1, st))
    return out


# ---------------------------------------------------------------- verify step

def accept_probability(p_t: np.ndarray, q_t: np.ndarray, x: int) -> float:
    """a(x) = min(1, p(x) / q(x)) (eq. 39.3), with q floored at 1e-300 as in
    P2 Listing 39.4 so that a zero draft probability cannot divide by zero."""
    return min(1.0, float(p_t[x]) / max(float(q_t[x]), 1e-300))


def residual(p_t: np.ndarray, q_t: np.ndarray) -> np.ndarray:
    """Unnormalised residual max(0, p - q) (eq. 39.4)."""
    return np.maximum(0.0, p_t - q_t)


def acceptance_probability(p_t: np.ndarray, q_t: np.ndarray) -> float:
    """alpha = sum_x min(p(x), q(x)) (P2 Listing 39.5)."""
    return float(np.minimum(p_t, q_t).sum())


def expected_accepted_prefix(alphas) -> float:
    """Expected accepted drafts before the first rejection: sum_i prod_{j<=i} alpha_j."""
    total, prefix = 0.0, 1.0
    for a in alphas:
        prefix *= a
        total += prefix
    return total


@dataclass
class Decision:
    """Margins of the comparisons taken at one verify position (or tree node),
    each the distance of a quantity from the cut that decides it:
      accept   |u0 - a| for the acceptance test(s) u0 < a (eq. 39.3), the
               smallest over the candidates tested there; inf if none;
      support  the nearest top-p or min-p decision of the chains that shape
               p~ and q~ there (they move a, the residual and the draw);
      draw     the draw's uniform from the nearer end of the drawn token's
               CDF interval (residual, fallback or bonus draw); inf if no
               token was drawn there."""
    accept: float = float("inf")
    support: float = float("inf")
    draw: float = float("inf")

    def smallest(self) -> float:
        return min(self.accept, self.support, self.draw)


@dataclass
class VerifyResult:
    tokens: list                  # K + 1 entries, -1 padded
    n_accepted: int
    status: int
    margins: list                 # one Decision per consulted position, in order


def spec_verify_row(target: np.ndarray, draft: np.ndarray, draft_tokens, params,
                    seed: int, row: int, step: int, uniforms=None) -> VerifyResult:
    """Verify K drafted tokens of one sequence [P3 "The Algorithm"; P1
    "Speculative decoding"; P4 "Speculative decoding"; P2 section 39.4].

    target: [K+1, V] logits of the target at the K draft positions plus the
    next one; draft: [K, V] draft logits; draft_tokens: K ids.

    Reading of the pages: the same chain (temperature, filters, eq. 39.2) shapes
    both p and q before verification (P3 "Temperature and Sampling" tempers
    both). For j = 0..K-1 in order, with (w0, w1) the Philox words of counter
    (row, j | SPEC << 16, step): accept x_j iff w0 * 2^-32 < a(x_j) (eq. 39.3);
    at the first rejection draw a replacement from max(0, p - q) / Z_r with
    w1 (eq. 39.4; from p itself if Z_r = 0, which exact arithmetic never
    reaches), then stop. If all K are kept, draw a bonus token from the
    target's row K with w0 of position K.

    Greedy (temperature 0): keep a draft iff it is the target's argmax, on the
    first mismatch emit the argmax, and the bonus is the argmax of row K
    (P1 "Speculative decoding"); draft rows are not read.

    ``uniforms`` (tests only) replaces the Philox pair (u0[j], u1[j]) of every
    position by the given [K+1, 2] array.
    """
    prm = Params.of(params)
    check_params(prm)
    target = np.asarray(target, dtype=np.float64)
    draft = np.asarray(draft, dtype=np.float64)
    K = draft.shape[0]
    V = target.shape[1]
    bad = [-1] * (K + 1)
    rows_read = [target[j] for j in range(K + 1)]
    if prm.temperature != 0.0:
        rows_read += [draft[j] for j in range(K)]
    for r in rows_read:
        st = row_status(r)
        if st != ROW_OK:
            return VerifyResult(bad, 0, st, [])
    xs = [int(x) for x in draft_tokens]
    if any(x < 0 or x >= V for x in xs):
        return VerifyResult(bad, 0, ROW_BADTOKEN, [])

    out = []
    margins = []
    if prm.temperature == 0.0:
        for j in range(K):
            a = greedy_token(target[j])
            if xs[j] == a:
                out.append(a)
                continue
            out.append(a)
            return VerifyResult(out + [-1] * (K + 1 - len(out)), j, ROW_OK, margins)
        out.append(greedy_token(target[K]))
        return VerifyResult(out, K, ROW_OK, margins)

    if uniforms is None:
        words = draw_words(seed, [row] * (K + 1), np.arange(K + 1), step, DOMAIN_SPEC)
        u0 = uniforms_from_words(words[:, 0])
        u1 = uniforms_from_words(words[:, 1])
    else:
        u0, u1 = np.asarray(uniforms, dtype=np.float64).T
    for j in range(K):
        sp = support(target[j], prm)
        sq = support(draft[j], prm)
        x = xs[j]
        a = accept_probability(sp.p_tilde, sq.p_tilde, x)
        d = Decision(accept=abs(u0[j] - a),
                     support=min(sp.margin_p, sp.margin_m, sq.margin_p, sq.margin_m))
        margins.append(d)
        if u0[j] < a:
            out.append(x)
            continue
        r = residual(sp.p_tilde, sq.p_tilde)
        if r.sum() > 0.0:
            tok, d.draw = draw_from(r, r > 0.0, u1[j])
        else:
            tok, d.draw = draw_from(sp.p_tilde, sp.keep, u1[j])
        out.append(tok)
        return VerifyResult(out + [-1] * (K + 1 - len(out)), j, ROW_OK, margins)
    sp = support(target[K], prm)
    tok, md = draw_from(sp.p, sp.keep, u0[K])
    out.append(tok)
    margins.append(Decision(support=min(sp.margin_p, sp.margin_m), draw=md))
    return VerifyResult(out, K, ROW_OK, margins)


def spec_verify_batch(target, draft, draft_tokens, params, seed, step, rows=None):
    rows = range(target.shape[0]) if rows is None else rows
    return [spec_verify_row(target[b], draft[b], draft_tokens[b], params, seed, b, step)
            for b in rows]
