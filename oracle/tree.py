"""Float64 oracle of the tree (multi-candidate) verify step. Test
infrastructure only (see the package docstring).

Pages cited:
  [P3] brentwoodlivery.com "Speculative decoding - Hinglish notes", sections
       "The Algorithm (Step-by-Step)" and "Extensions and Variants"
       ("Multi-candidate speculation": the draft proposes a tree of
       candidates with several branches and the target verifies every path).
  [P2] gowda.ai "Chapter 39 Decoding & Speculative Sampling", section 39.4
       (eqs. 39.3, 39.4: accept with min(1, p/q), else draw from the
       normalised residual max(0, p - q)).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .philox import DOMAIN_TREE, draw_words, uniforms_from_words
from .sampler import (ROW_BADTOKEN, ROW_OK, Decision, Params, check_params, draw_from,
                      greedy_token, row_status, support)

__all__ = ["TREE_MAX_NODES", "TreeResult", "tree_children", "tree_verify_row", "INVALID_TREE"]

TREE_MAX_NODES = 32
INVALID_TREE = 5   # a parent index that is not an earlier node


@dataclass
class TreeResult:
    tokens: list       # emitted tokens: the accepted nodes' tokens, then one drawn token
    path: list         # the accepted nodes, root first excluded
    status: int
    margins: list      # one Decision per visited node (the root first), in order


def tree_children(parent) -> list:
    """Children of every node in increasing node order."""
    ch = [[] for _ in parent]
    for n, pa in enumerate(parent):
        if n > 0:
            ch[int(pa)].append(n)
    return ch


def tree_verify_row(target, draft, parent, tokens, params, seed: int, row: int,
                    step: int) -> TreeResult:
    """Verify one sequence's draft tree.

    Node 0 is the current context; node n > 0 extends node parent[n] < n by
    tokens[n]. target[n] / draft[n]: the target's / draft's logits for the
    token after node n's path. The children of a node are its candidates for
    the next position, taken as independent draws from the draft distribution
    q~ at that node.

    Reading of the pages (P3 gives the tree in one sentence, P2 the rule for
    one candidate): starting at the root, the children of the current node v
    are tested in node order, each against the target distribution left by
    the previous rejections: with p_1 = p~_v, child c is kept iff u < min(1,
    p_c(x_c) / q~_v(x_c)) (eq. 39.3); after a rejection p_{c+1} = max(0, p_c -
    q~_v) normalised (eq. 39.4; unchanged if that is all zero, which exact
    arithmetic never reaches). A kept child becomes v. When every child of v
    is rejected, or v has none, one token is drawn from the current p and the
    step ends: the output is then exactly distributed as p~ at every position
    (the multi-candidate generalisation of speculative sampling). Uniforms:
    child c of v uses w0 of the Philox counter (row, v * 32 + c | TREE << 16,
    step); the draw at v uses w1 of (row, v * 32 | TREE << 16, step).

    Greedy (temperature 0): the first child whose token is the target's argmax
    at v is kept; otherwise the argmax is emitted and the step ends.
    """
    prm = Params.of(params)
    check_params(prm)
    target = np.asarray(target, dtype=np.float64)
    draft = np.asarray(draft, dtype=np.float64)
    N, V = target.shape
    parent = [int(x) for x in parent]
    toks = [int(x) for x in tokens]
    if N < 1 or N > TREE_MAX_NODES or parent[0] != -1 or \
            any(not (0 <= parent[n] < n) for n in range(1, N)):
        return TreeResult([], [], INVALID_TREE, [])
    ch = tree_children(parent)
    reads = [target[n] for n in range(N)]
    if prm.temperature != 0.0:
        reads += [draft[n] for n in range(N) if ch[n]]
    for r in reads:
        st = row_status(r)
        if st != ROW_OK:
            return TreeResult([], [], st, [])
    if any(not (0 <= toks[n] < V) for n in range(1, N)):
        return TreeResult([], [], ROW_BADTOKEN, [])

    out, path, margins = [], [], []
    v = 0
    if prm.temperature == 0.0:
        while True:
            a = greedy_token(target[v])
            nxt = next((c for c in ch[v] if toks[c] == a), None)
            out.append(a)
            if nxt is None:
                return TreeResult(out, path, ROW_OK, margins)
            path.append(nxt)
            v = nxt
    while True:
        sp = support(target[v], prm)
        d = Decision(support=min(sp.margin_p, sp.margin_m))
        margins.append(d)
        p = sp.p_tilde.copy()
        kept = None
        if ch[v]:
            sq = support(draft[v], prm)
            d.support = min(d.support, sq.margin_p, sq.margin_m)
            q = sq.p_tilde
            pos = [v * 32 + c for c in range(len(ch[v]))]
            u0 = uniforms_from_words(draw_words(seed, [row] * len(pos), np.array(pos), step,
                                                DOMAIN_TREE)[:, 0])
            for c, child in enumerate(ch[v]):
                x = toks[child]
                a = min(1.0, p[x] / max(q[x], 1e-300))
                d.accept = min(d.accept, abs(u0[c] - a))
                if u0[c] < a:
                    kept = child
                    break
                r = np.maximum(0.0, p - q)
                if r.sum() > 0.0:
                    p = r / r.sum()
        if kept is not None:
            out.append(toks[kept])
            path.append(kept)
            v = kept
            continue
        u1 = float(uniforms_from_words(draw_words(seed, [row], v * 32, step, DOMAIN_TREE)[:, 1])[0])
        keep = p > 0.0
        tok, d.draw = draw_from(p, keep, u1)
        out.append(tok)
        return TreeResult(out, path, ROW_OK, margins)
