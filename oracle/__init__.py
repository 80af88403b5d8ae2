"""fp64 CPU oracle for vocabulary-scale LM-head scoring.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the HIP library or its Python
binding; the two meet only through the seeded input generators in
``workloads/``, which hold none of the method's arithmetic.

Every function is a plain, slow, obviously correct numpy fp64 rendering of
what the method computes, written from these pages:

* SkyRL PR #2004 "perf(sample-support): reuse replay scores for entropy"
  (sections Problem, Implementation, and the review's suggested
  ``_selected_hidden_projection``): recorded-support logprob and entropy,
  synthetic-EOS fallback, singleton support => zero entropy, the cast of the
  hidden state to the weight dtype and the division by temperature after
  the dot product.
* xorl issue #71 "Consolidate the exact and generic scoring paths"
  (section 1's description of the LM-head op, section 3's transform
  program name): chunked projection -> log-sum-exp -> sampling support ->
  selected logprob; temperature, then stable token-id top-k, inclusive
  top-p, min-p against the original row max; the same program over the
  projection ("Proposed direction" item 3), on its bf16-rounded logits.
* DeepSpec PR #87 "[Perf] Reuse DSpark probability distance" (sections
  Purpose and Test Plan): per-token L1 distance between draft and target
  softmaxes, accept_rate = clamp(1 - 0.5 * L1, 0, 1), and the weighted L1
  distillation loss with its draft-logit gradient.

Pinned by ``tests/test_oracle_*.py`` against closed forms, library routines
(scipy, torch CPU), brute force on tiny inputs and hand-derived fixtures in
``tests/golden/``.  ``sampling`` holds the seeded Gumbel draw that ends the
transform program; the pages name it without defining its generator, so it
follows a stated reading (Philox4x32-10 from its published definition, pinned
by that generator's known-answer vectors, and the Gumbel-max draw, pinned by
the softmax frequencies it must produce).
"""

from . import sampling  # noqa: F401
from .scoring import (  # noqa: F401
    ST_OK,
    ST_EMPTY_SUPPORT,
    ST_TARGET_OUTSIDE_SUPPORT,
    ST_BAD_INPUT,
    ST_FULL_VOCAB_FALLBACK,
    ST_SUPPORT_TRUNCATED,
    widen_bf16,
    round_f32_to_bf16,
    round_f64_to_bf16,
    logits_from_logits,
    logits_from_hidden,
    bf16_logits_from_hidden,
    score_full,
    score_support,
    score_transforms,
    score_prefix_support,
    l1_distance,
    weighted_l1_loss,
    logit_vjp,
    score_full_vjp,
    score_support_vjp,
)
