"""Seeded synthetic workloads shared by the tests, the benchmark and the smoke check.

This package produces inputs only: logits, draft tokens, tree topologies, prompts
and the uniforms that the verification method consumes.  It contains none of the
method's arithmetic (no softmax, acceptance ratio, residual or inverse-CDF step),
and it imports neither the oracle nor the HIP library.
"""

from .workloads import (  # noqa: F401
    ChainInputs,
    TreeInputs,
    NgramPrompts,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    philox,
    uniforms_open_closed,
    chain_inputs,
    chain_shared_rows,
    chain_config_small_f32,
    chain_config_high_accept_bf16,
    chain_config_low_accept_bf16,
    tree_inputs,
    tree_config_eagle_bf16,
    tree_parents,
    SampledTreeInputs,
    tree_sampled_inputs,
    tree_sampled_config_bf16,
    random_parents,
    kv_entries,
    commit_requests,
    ngram_prompts,
    ngram_config_prompts,
    ngram_target_inputs,
)
