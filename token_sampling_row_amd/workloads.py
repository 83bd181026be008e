"""Seeded synthetic logits for the sampler and the verify step.

This module only draws inputs. It holds none of the sampler's arithmetic
(no softmax, no filter, no draw), so the HIP path and the float64 oracle can
both read the same stored bits without sharing any of the method.

The shape of the data follows the pages: a next-token distribution with a head
and a very long tail over a vocabulary of 8k-152k tokens (legost.in "Choosing
the next word", section "The sampling desk"). Each row is Zipf-like:

    logit_i = -a * ln(rank_i) + N(0, sigma^2),   rank = a random permutation of 1..V

drawn in float64, rounded to float32 (round to nearest even) and, where the
workload is bf16, rounded again from float32 to bf16 (round to nearest even).
Row b of workload c uses ``numpy.random.default_rng([1000 + c, b])``.

bf16 values are carried as ``uint16`` bit patterns because numpy has no bf16
type; :func:`bf16_bits_to_f32` widens them exactly (a 16-bit shift).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F32 = "f32"
BF16 = "bf16"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest even); return the uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def zipf_row(seed_pair, vocab: int, a: float, sigma: float) -> np.ndarray:
    """One float64 row of Zipf-like logits with Gaussian noise (see module doc)."""
    rng = np.random.default_rng(seed_pair)
    rank = rng.permutation(vocab).astype(np.float64) + 1.0
    return -a * np.log(rank) + rng.normal(0.0, sigma, vocab)


@dataclass
class Workload:
    """A batch of logits as stored bits plus the parameters it is sampled with."""

    name: str
    dtype: str                    # "f32" or "bf16"
    rows: int
    vocab: int
    data: np.ndarray              # [rows, vocab] float32, or uint16 bf16 bits
    runs: list = field(default_factory=list)   # list of parameter dicts
    extra: dict = field(default_factory=dict)

    def values_f32(self) -> np.ndarray:
        """The stored values as float32 (exact for both dtypes)."""
        if self.dtype == BF16:
            return bf16_bits_to_f32(self.data)
        return self.data


def _round_rows(rows64: np.ndarray, dtype: str) -> np.ndarray:
    f32 = rows64.astype(np.float32)
    return f32_to_bf16_bits(f32) if dtype == BF16 else f32


def _zipf_batch(cfg: int, rows: int, vocab: int, a_of_row, sigma: float,
                row_offset: int = 0) -> np.ndarray:
    out = np.empty((rows, vocab), dtype=np.float64)
    for b in range(rows):
        out[b] = zipf_row([1000 + cfg, row_offset + b], vocab, a_of_row(b), sigma)
    return out


def sampler_params(temperature=1.0, top_k=0, top_p=1.0, min_p=0.0, mode=0) -> dict:
    """Parameter dict in the boundary's units (0 / 1.0 / 0.0 switch a filter off)."""
    return dict(temperature=float(temperature), top_k=int(top_k), top_p=float(top_p),
                min_p=float(min_p), mode=int(mode))


# Philox key (seed) used for each workload; the step is the run index.
def philox_seed(cfg: int) -> int:
    return 0x5EED0000 + cfg


def config(cfg: int, rows: int | None = None) -> Workload:
    """Workload ``cfg`` (1..5). ``rows`` truncates the batch to its first rows.

    1: 64 x 8192 fp32, a=1.1, sigma=0.3; T=0.8, top_k=40, top_p=0.9, min_p=0.05.
    2: 256 x 32000 fp32, a=1.0, sigma=0.5; greedy / T=1 / T=0.7 + min_p=0.1.
    3: 256 x 128256 bf16, a=1.2, sigma=0.5, 13 near-flat rows (a=0.2);
       T=0.9, top_k=50, top_p=0.95, min_p=0.1.
    4: verify, 64 rows, K=4, V=32000 fp32; target a=1.0 sigma=0.5 per (b, j);
       draft = target[:, :K] + N(0, 0.8^2); verify at T=1 and at T=0.
    5: 1024 x 151936 bf16, a=1.0, sigma=0.5; T=1.5 top_p=0.9 / T=1.5 top_k=1024.
    """
    if cfg == 1:
        B, V = 64, 8192
        B = B if rows is None else min(rows, B)
        d = _round_rows(_zipf_batch(1, B, V, lambda b: 1.1, 0.3), F32)
        return Workload("tiny_8192_f32", F32, B, V, d,
                        [sampler_params(0.8, 40, 0.9, 0.05)])
    if cfg == 2:
        B, V = 256, 32000
        B = B if rows is None else min(rows, B)
        d = _round_rows(_zipf_batch(2, B, V, lambda b: 1.0, 0.5), F32)
        return Workload("batch256_32000_f32", F32, B, V, d,
                        [sampler_params(0.0), sampler_params(1.0),
                         sampler_params(0.7, min_p=0.1)])
    if cfg == 3:
        B, V = 256, 128256
        flat = set(np.random.default_rng(1003).choice(256, 13, replace=False).tolist())
        B = B if rows is None else min(rows, B)
        d = _round_rows(_zipf_batch(3, B, V, lambda b: 0.2 if b in flat else 1.2, 0.5), BF16)
        return Workload("batch256_128256_bf16", BF16, B, V, d,
                        [sampler_params(0.9, 50, 0.95, 0.1)],
                        extra={"flat_rows": sorted(x for x in flat if x < B)})
    if cfg == 4:
        B, K, V = 64, 4, 32000
        B = B if rows is None else min(rows, B)
        tgt = np.empty((B, K + 1, V), dtype=np.float64)
        for b in range(B):
            for j in range(K + 1):
                tgt[b, j] = zipf_row([1004, b, j], V, 1.0, 0.5)
        noise = np.random.default_rng([1004, 1 << 20]).normal(0.0, 0.8, (64, K, V))[:B]
        dft = tgt[:, :K, :] + noise
        w = Workload("verify64_k4_32000_f32", F32, B, V,
                     _round_rows(tgt.reshape(B * (K + 1), V), F32).reshape(B, K + 1, V),
                     [sampler_params(1.0), sampler_params(0.0)])
        w.extra["K"] = K
        w.extra["draft"] = _round_rows(dft.reshape(B * K, V), F32).reshape(B, K, V)
        return w
    if cfg == 5:
        B, V = 1024, 151936
        B = B if rows is None else min(rows, B)
        d = _round_rows(_zipf_batch(5, B, V, lambda b: 1.0, 0.5), BF16)
        return Workload("batch1024_151936_bf16", BF16, B, V, d,
                        [sampler_params(1.5, top_p=0.9), sampler_params(1.5, top_k=1024)])
    raise ValueError(f"unknown workload {cfg}")


def random_rows(seed: int, rows: int, vocab: int, a: float = 1.0, sigma: float = 0.5,
                dtype: str = F32) -> np.ndarray:
    """Extra Zipf-like rows for tests (arbitrary sizes), stored bits as above."""
    out = np.empty((rows, vocab), dtype=np.float64)
    for b in range(rows):
        out[b] = zipf_row([seed, b], vocab, a, sigma)
    return _round_rows(out, dtype)


def verify_batch(seed: int, rows: int, K: int, vocab: int, dtype: str = BF16, a: float = 1.0,
                 sigma: float = 0.5, noise: float = 0.8):
    """A speculative-verify batch of any size, generated as workload 4 is:
    target rows [rows, K + 1, vocab] of Zipf-like logits, one per (sequence,
    position); draft rows [rows, K, vocab] = the target's first K positions
    plus N(0, noise^2). Returns the two as stored bits."""
    tgt = np.empty((rows, K + 1, vocab), dtype=np.float64)
    for b in range(rows):
        for j in range(K + 1):
            tgt[b, j] = zipf_row([seed, b, j], vocab, a, sigma)
    dft = tgt[:, :K, :] + np.random.default_rng([seed, 1 << 20]).normal(0.0, noise,
                                                                         (rows, K, vocab))
    return (_round_rows(tgt.reshape(rows * (K + 1), vocab), dtype).reshape(rows, K + 1, vocab),
            _round_rows(dft.reshape(rows * K, vocab), dtype).reshape(rows, K, vocab))


def allowed_words(seed: int, rows: int, vocab: int, kind: str) -> np.ndarray:
    """Seeded allowed-token bitmasks for constrained decoding, packed as the
    sampler reads them: uint32 [rows, ceil(vocab / 32)], token i allowed iff
    bit i % 32 of word i // 32 is set. The bits past ``vocab`` in the last
    word are random (they must be ignored). ``kind``:

      "all"        every token allowed
      "none"       no token allowed (the invalid state of an empty set)
      "p=<x>"      each token allowed independently with probability x
      "few=<n>"    n tokens drawn without replacement (a grammar that allows a
                   handful of continuations: digits, a quote, a brace)
      "block"      one contiguous id range of a random length
    """
    words = (vocab + 31) // 32
    out = np.zeros((rows, words * 32), dtype=bool)
    for b in range(rows):
        rng = np.random.default_rng([7000, seed, b])
        if kind == "all":
            out[b, :vocab] = True
        elif kind == "none":
            pass
        elif kind.startswith("p="):
            out[b, :vocab] = rng.random(vocab) < float(kind[2:])
        elif kind.startswith("few="):
            n = min(int(kind[4:]), vocab)
            out[b, rng.choice(vocab, n, replace=False)] = True
        elif kind == "block":
            lo = int(rng.integers(0, vocab))
            hi = int(rng.integers(lo + 1, vocab + 1))
            out[b, lo:hi] = True
        else:
            raise ValueError(f"unknown mask kind {kind}")
        out[b, vocab:] = rng.random(words * 32 - vocab) < 0.5
    bits = out.reshape(rows, words, 32).astype(np.uint64)
    return (bits << np.arange(32, dtype=np.uint64)).sum(axis=2).astype(np.uint32)
