"""CPU float64 oracle for tiled fused attention forward.

TEST INFRASTRUCTURE ONLY. This package is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``,
and by nothing else. The product path (the HIP library and its Python
binding) never imports, calls or links anything here, and nothing here
imports the product path: the two share no code.

What it computes, and the passages it follows (the source pages are the four
TileLang web pages the work is based on; citations name the page and its
section):

* ``attention`` -- multi-head attention forward by the plain definition
  S = scale*Q*K^T, P = softmax(S) row-wise, O = P*V, with the natural-log
  log-sum-exp of each score row ("TileLang study notes", section
  "FlashAttention implementation", the standard attention definition).
  The score block is materialised and the softmax taken in two passes
  (row max, then exponentials and sums).
* ``mla_decode`` -- the MLA decode variant from the FlashMLA walk-through
  ("TileLang programming model and FlashMLA", sections 2.1-2.2 and 3.1):
  many query heads against one shared latent KV head plus a rotary part,
  scores from the two products summed, values taken from the latent itself.
* ``online_attention`` -- the tiled online-softmax recurrence (running row
  max m, running sum l, rescaled accumulator), in the order the study notes'
  "Online Softmax" subsection states it. It is used only to check that the
  recurrence reaches the two-pass result.
* ``attention_masked`` / ``visible_keys`` -- the attention variants of
  "TileLang programming model and FlashMLA", section 5.1: grouped and single KV heads
  (multi-query), a sliding key window around the query position, and a
  block mask that decides which (query block, key block) pairs are
  computed. Same definition as ``attention`` over each row's visible keys.
* ``attention_partial`` / ``combine_partials`` -- per-key-range normalised
  partial outputs with their log-sum-exp, and the exact merge of such
  partials. The pages do not describe a split; this is the split-KV reading
  recorded in the design notes, and its identity with the unsplit result is
  pinned by the tests.

* ``ssd`` (submodule) -- the Mamba-2 state-space scan that the pages name as
  their linear-attention workload (chunk-state and chunk-scan; "TileLang
  paper summary", appendix A.4, and the tiled Mamba scan sketch of "From
  FlashAttention to general kernels", section 4): the step-by-step
  recurrence and its chunked form.

Parity status: every function above is pinned by ``tests/test_oracle.py``,
``tests/test_oracle_variants.py`` and ``tests/test_oracle_ssd.py`` (closed
forms, invariants, a high-precision brute force on tiny inputs, an
independent library routine). Nothing is "parity unpinned".
"""

from . import ssd  # noqa: F401
from .core import (  # noqa: F401
    attention,
    attention_masked,
    attention_partial,
    combine_partials,
    mla_decode,
    mla_decode_rows,
    online_attention,
    visible_keys,
)
