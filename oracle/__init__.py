"""CPU oracle for the batched logits-to-token sampler and the speculative verify step.

TEST INFRASTRUCTURE ONLY. Plain, slow, float64 NumPy code that states what the
sampler computes, written from the pages, with no blocking, fusion or reordering
beyond what the definitions say. Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it. The product path (the
HIP library and its Python binding) never imports, calls or links anything here,
and nothing here imports the product path: the two share no code. The only
module both sides read is the seeded input generator
``token_sampling_row_amd/workloads.py``, which holds none of the method.

Modules
-------
philox   Philox4x32-10 counter-based generator (Salmon, Moraes, Dror, Shaw,
         "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11), written from its
         published definition, and the counter layout the sampler uses.
tree     The tree (multi-candidate) verify step.
beam     One beam-search step (eq. 39.1, Listing 39.1) and the search built on it.
sampler  The filter chain (temperature, softmax, top-k, top-p, min-p,
         renormalisation by eq. 39.2), the draw, greedy decoding, and the
         speculative verify step (eqs. 39.3 and 39.4).

Parity pins: every function here is checked by ``tests/test_oracle_*.py`` against
values the pages print, closed forms, brute force on tiny vocabularies and, for
Philox, an independent library implementation (rocRAND's host-callable engine).
"""
from .philox import philox4x32_10, sampler_counters, uniforms_from_words  # noqa: F401
from .sampler import *  # noqa: F401,F403
from .beam import *  # noqa: F401,F403
from .tree import *  # noqa: F401,F403
