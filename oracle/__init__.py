"""CPU oracle for the speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 numpy
statement of what the verify step computes.  It exists so that the HIP path
can be checked against something obviously correct.  Only the tests, the
smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the product path never does, and it shares no
code with the HIP kernels or their binding.

Modules
-------
attention  -- grouped-query attention of the K+1 verifier query positions
              over a paged KV cache, causal inside the draft window.
reject     -- the lossless rejection-sampling verifier (accept test,
              first-rejection scan, residual / bonus sample, greedy mode)
              and the commit of the logical KV length.
exact_law  -- the closed-form joint law of one verify call, used to pin the
              oracle by brute-force enumeration.
tree       -- attention and the lossless verifier over a flattened draft
              tree.
kv         -- the window's K/V in the paged cache (append, commit) and the
              host page pool.
bandit     -- the epsilon-greedy draft-length controller and the
              per-position acceptance statistics.
filter     -- top-k / top-p filtering of both laws before the verifier
              (chain and tree).

Sources (the pages the method is taken from):
  [AIE]  AI Engineering from Scratch, lesson "Speculative decoding and
         EAGLE-3" -- sections "Concept" (the Leviathan rejection rule, the
         residual, the bonus token), "What determines the speed-up"
         (expected accepted tokens), "Rolling back the KV cache", and
         "Build it" steps 1-5.
  [QS]   quickscale.ai, "Quand et pourquoi utiliser le speculative
         decoding" -- section 2 (mechanism, losslessness), section 4
         (per-position acceptance, mean acceptance length).
  [SGL]  sglang_spec_decode README -- the provisional KV layer and the
         acceptance rule (letters p/q swapped relative to [AIE]).
  [PHX]  devpost "phoenix" -- greedy verification gives the target's own
         output.

Parity status: every function here is pinned by the CPU tests
(closed forms, brute-force enumeration, invariants, an independent dense
attention); none is "parity unpinned".
"""

from . import attention, reject, exact_law, tree, kv, bandit, filter  # noqa: F401
