"""Philox4x32-10, from its published definition (test infrastructure only).

Source: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3", SC'11, section on the Philox bijection. One round
maps a 4-word counter X = (X0, X1, X2, X3) under a 2-word key K = (K0, K1) to

    (hi_a, lo_a) = 64-bit product M_a * X0      M_a = 0xD2511F53
    (hi_b, lo_b) = 64-bit product M_b * X2      M_b = 0xCD9E8D57
    Y = (hi_b ^ X1 ^ K0,  lo_b,  hi_a ^ X3 ^ K1,  lo_a)

and the key is advanced by the Weyl constants (0x9E3779B9, 0xBB67AE85),
modulo 2^32, between rounds. Philox4x32-10 applies 10 rounds.

The pages only say that the sampler's uniforms come from a seeded 32-bit
generator and that the same seed and knobs give the same text token for token
(legost.in "Choosing the next word", section "Where the randomness comes
from"). The counter-based generator makes a draw depend only on
(seed, row, position, step, domain), never on the parameters or the batch size.
"""
from __future__ import annotations

import numpy as np

M_A = 0xD2511F53
M_B = 0xCD9E8D57
W_0 = 0x9E3779B9
W_1 = 0xBB67AE85
ROUNDS = 10
MASK32 = 0xFFFFFFFF

# Domains of the counter's second word (bits 16..31).
DOMAIN_SAMPLE = 0   # one draw per row of sample_rows
DOMAIN_SPEC = 1     # the verify step: accept test, residual draw, bonus draw
DOMAIN_TREE = 2     # the tree verify step: node v, child c at position v * 32 + c


def philox4x32_10(counters: np.ndarray, key) -> np.ndarray:
    """Apply Philox4x32-10 to ``counters`` ([n, 4] uint32) under ``key`` = (K0, K1).

    Returns [n, 4] uint32 words. Vectorised over n with uint64 products.
    """
    x = np.asarray(counters, dtype=np.uint64).reshape(-1, 4) & MASK32
    x0, x1, x2, x3 = (x[:, i].copy() for i in range(4))
    k0 = np.uint64(int(key[0]) & MASK32)
    k1 = np.uint64(int(key[1]) & MASK32)
    mask = np.uint64(MASK32)
    sh = np.uint64(32)
    for r in range(ROUNDS):
        pa = x0 * np.uint64(M_A)          # < 2^64, exact in uint64
        pb = x2 * np.uint64(M_B)
        hi_a, lo_a = pa >> sh, pa & mask
        hi_b, lo_b = pb >> sh, pb & mask
        x0, x1, x2, x3 = (hi_b ^ x1 ^ k0), lo_b, (hi_a ^ x3 ^ k1), lo_a
        if r + 1 < ROUNDS:
            k0 = (k0 + np.uint64(W_0)) & mask
            k1 = (k1 + np.uint64(W_1)) & mask
    return np.stack([x0, x1, x2, x3], axis=1).astype(np.uint32)


def philox_scalar(counter, key):
    """The same bijection with Python integers, one counter at a time."""
    x = [int(c) & MASK32 for c in counter]
    k0, k1 = int(key[0]) & MASK32, int(key[1]) & MASK32
    for r in range(ROUNDS):
        pa, pb = M_A * x[0], M_B * x[2]
        x = [((pb >> 32) ^ x[1] ^ k0) & MASK32, pb & MASK32,
             ((pa >> 32) ^ x[3] ^ k1) & MASK32, pa & MASK32]
        if r + 1 < ROUNDS:
            k0 = (k0 + W_0) & MASK32
            k1 = (k1 + W_1) & MASK32
    return x


def seed_key(seed: int):
    """Key words from a 64-bit seed: (low 32 bits, high 32 bits)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return (seed & MASK32, seed >> 32)


def sampler_counters(rows, position, step: int, domain: int) -> np.ndarray:
    """Counters for draws: (row, position | domain << 16, step low, step high)."""
    rows = np.atleast_1d(np.asarray(rows, dtype=np.uint64))
    pos = np.broadcast_to(np.asarray(position, dtype=np.uint64), rows.shape)
    step = int(step) & 0xFFFFFFFFFFFFFFFF
    c = np.empty((rows.size, 4), dtype=np.uint64)
    c[:, 0] = rows & MASK32
    c[:, 1] = (pos & 0xFFFF) | (np.uint64(domain & 0xFFFF) << np.uint64(16))
    c[:, 2] = step & MASK32
    c[:, 3] = step >> 32
    return c.astype(np.uint32)


def uniforms_from_words(words: np.ndarray) -> np.ndarray:
    """u = w * 2^-32 in float64: exact, in [0, 1 - 2^-32]."""
    return np.asarray(words, dtype=np.float64) * (2.0 ** -32)


def draw_words(seed: int, rows, position, step: int, domain: int) -> np.ndarray:
    """The four Philox words for each row at (position, step, domain)."""
    return philox4x32_10(sampler_counters(rows, position, step, domain), seed_key(seed))
