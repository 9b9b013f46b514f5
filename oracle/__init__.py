"""CPU oracle for batched speculative-decoding draft verification.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, float64 definition of
what the GPU library computes.  It exists so that tests, the smoke check and the
CPU-baseline leg of the benchmark can check and time the GPU path against it.
No product code path may import or call it, and it shares no code with the HIP
library (it does its own bf16 widening, softmax, scans and searches).

Pages cited (by title; section, step or figure given at each use):
  * "Speculative Decoding in Production: From Draft Models to EAGLE-3 Dynamic Trees
    for 3x-5x Lossless Acceleration" (blog.llmgo.top) -- the method: section I.1
    (modified rejection sampling, its three steps, and the invariance theorem),
    section III.1 (linear chains) and III.2 (tree attention verification).
  * "Accelerating Autoregressive LLM Inference 3x with Lossless Speculative Decoding
    and EAGLE Heads" (x078.com) -- prompt n-gram lookup drafting, K = 5,
    lookup maximum n = 4 (the deployment snippet in section 1).
  * "Breaking the Memory Bandwidth Wall: 3.42x Generation Speedup with EAGLE
    Speculative Decoding" (acefleet.dev) -- "Technical Foundations" (draft, then
    one verification pass; acceptance restated).
  * "Speculative decoding: Medusa, EAGLE, vLLM" (vikram-blog.pages.dev) -- the
    "System Topology & Data Flow" tree figure (and the commit of the accepted branch)
    and the greedy (temperature 0) usage.
  * "Breaking the Memory Bandwidth Wall ..." (acefleet.dev), "Closed-Loop Real-Time
    Adaptive Gating" -- the temperature gate and the per-tenant acceptance breaker.

Where the pages are silent the oracle takes one stated reading (temperature
divides the logits; a bonus token is drawn from the target row after the last
draft when every draft is accepted; inverse-CDF sampling in vocabulary order with
the smallest index whose inclusive prefix reaches u*W; temperature 0 as greedy chain
verification; greedy tree acceptance by
argmax with smallest-index ties; n-gram lookup by the longest suffix and its
earliest occurrence).  Each function names the reading it takes.

Parity status: every function here is pinned by the "not gpu" tests (closed forms,
exact enumeration of the invariance theorem, brute force, and the pages' worked
examples under tests/golden/).  No function is "parity unpinned".
"""

from .common import widen_logits  # noqa: F401
from .chain import (  # noqa: F401
    ChainSequenceResult,
    ChainBatchResult,
    acceptance_probability,
    inverse_cdf_sample,
    residual_weights,
    softmax_at_temperature,
    verify_chain,
    verify_chain_greedy_sequence,
    verify_chain_sequence,
)
from .tree import TreeBatchResult, argmax_first, verify_tree_greedy, verify_tree_greedy_sequence  # noqa: F401
from .ngram import NgramResult, ngram_propose, ngram_propose_sequence  # noqa: F401
from .tree_io import commit_path, tree_attention_mask  # noqa: F401
from .gate import Gate  # noqa: F401
from .tree_sampled import verify_tree_sampled, verify_tree_sampled_sequence  # noqa: F401
