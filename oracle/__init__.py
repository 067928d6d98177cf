"""CPU oracle for ring / zigzag / striped / Ulysses-hybrid sequence-parallel attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP library.

Modules
  index_ref      integer token-order formulas (which positions each virtual
                 rank holds; Ulysses seq<->head relayout) in plain Python ints
  attention_ref  the definition: naive full-matrix masked softmax attention
                 in float64 over the unpermuted sequence, with the visibility
                 predicate on global positions
  ring_ref       the ring-decomposed float64 reference: per (rank, step)
                 block attention with its partial output and log-sum-exp, and
                 the associative max/logsumexp merge of partials
  backward_ref   the gradients (dQ, dK, dV) of masked softmax attention from
                 the chain rule, per ring step and summed over the ring
  decode_ref     decode-time attention of new queries over a KV cache, the
                 partials of cache pieces, and their pairwise tree merge

Every function is pinned by ``tests/test_oracle_*.py`` against brute force,
a library routine, closed forms, or values and invariants the pages state.
"""
from . import index_ref, attention_ref, ring_ref, backward_ref, decode_ref  # noqa: F401
