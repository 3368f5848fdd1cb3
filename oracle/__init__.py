"""fp64 CPU oracle for split tree-verify attention.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, calls or links anything here, and nothing here
imports the product path.

``commit.py`` covers the step after verification (greedy acceptance of a
tree path and committing it into the paged cache), written as the plain
per-sequence loops of its stated reading.

What it computes is the plain definition: for every tree node and query head,
unsplit softmax attention over the sequence's whole committed prefix plus the
tree nodes on that node's root path (itself included).  The split method
(prefix pass + suffix pass + log-sum-exp merge) reaches exactly this result in
real arithmetic; the oracle does not split.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against hand-derived tables, closed forms, a library attention routine and
invariants.  Numeric values at the five synthetic configs themselves are pinned
only through those invariants (the pages print no output values).
"""
from .commit import accept_greedy, commit, commit_incache  # noqa: F401
from .tree_attention import (  # noqa: F401
    ancestor_or_self_mask,
    ancestor_or_self_words,
    build_masks,
    build_masks_words,
    merge,
    prefix_only,
    suffix_only,
    to_f64,
    tree_rows_from_cache,
    verify,
    verify_incache,
    verify_rows,
    visibility,
)
