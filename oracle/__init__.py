"""fp64 CPU oracle for one DFlash draft-and-verify step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library
and its Python binding) never imports, links or executes anything here, and
this package imports nothing from the product.

Parity status per function (what pins it is listed in the tests that check
it; see ``tests/test_oracle_*.py``):

* ``rms_norm``, ``rope``, ``silu``, ``linear``, ``attention``,
  ``argmax_lowest``, ``accept``, ``inject``, ``draft_forward``,
  ``draft_anchors``, ``verify``, ``gumbel``, ``sample_categorical``,
  ``build_tree``, ``topk_logprobs``, ``tree_mask``, ``masked_attention``,
  ``tree_accept``, ``commit_path`` (brute-force enumeration of the best
  continuations, chain trees equal to the causal pass and the chain accept,
  a tree pass plus its commit equal to a causal pass over the path);
  ``causal_attention``, ``target_forward``, ``commit`` (brute force,
  causality, incremental passes over a committed cache, a closed form);
  ``draft_sample``, ``speculative_verify`` (the last four by closed-form
  distribution tests: chi-square against softmax and against the target's
  distribution at every emitted position),
  ``speedup``: pinned by brute force, closed forms and invariants.
* End-to-end drafted token values on random weights have no external
  reference value; they are pinned only through the invariants above
  (permutation equivariance, position-shift invariance, incremental
  injection) and compared with the GPU under the logit-gap rule.
"""
from .dflash_oracle import (  # noqa: F401
    OracleCache,
    accept,
    argmax_lowest,
    attention,
    build_tree,
    causal_attention,
    commit,
    commit_path,
    draft_anchors,
    draft_block,
    draft_forward,
    draft_sample,
    gumbel,
    inject,
    linear,
    masked_attention,
    rms_norm,
    rope,
    silu,
    sample_categorical,
    speculative_verify,
    speedup,
    target_feature_layers,
    target_forward,
    topk_logprobs,
    tree_accept,
    tree_mask,
    verify,
)
