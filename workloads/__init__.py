"""Seeded synthetic inputs for paged decode/verify attention and speculative verification.

This module only draws inputs: context lengths, query/KV values, block-table placement,
probability rows, draft tokens and uniforms.  It holds none of the attention or
rejection-sampling arithmetic, so both the CPU oracle (``oracle/``) and the HIP path
(``verify_attention_paged_amd``) can be fed from it without sharing any of the method.

Shapes and distributions follow the workloads described for continuous-batching serving
steps: long-tailed (lognormal / Pareto) context lengths, 16- or 32-token KV blocks placed at
non-contiguous pool slots through a per-sequence block table, GQA head groups, and
speculative drafts of k tokens verified with k+1 query rows, or token trees verified under
their ancestor masks.
"""

from .generate import (  # noqa: F401
    AttnInputs,
    VerifyInputs,
    CONFIG_NAMES,
    make_attention_inputs,
    make_verify_inputs,
    attention_config,
    config_lengths,
    DEFAULT_SEEDS,
    verify_config,
    open_uniforms,
    random_tree_parents,
    tree_masks,
    TreeVerifyInputs,
    make_tree_verify_from_probs,
    tree_verify_config,
    new_kv_rows,
    LogitsVerifyInputs,
    make_logits_verify_inputs,
    logits_verify_config,
)
