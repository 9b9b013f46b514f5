"""Batched speculative-decoding draft verification on AMD Instinct MI355X (gfx950).

The work runs in libspecverify.so (HIP kernels behind a C ABI, include/spec_verify.h);
this package holds the kernel sources (csrc/), the build step (build.py) and a thin
ctypes binding (binding.py) whose functions carry the C entry points' names.
"""

from .binding import (  # noqa: F401
    FLAG_INVALID,
    FLAG_TIMED_OUT,
    SPEC_KNOB_CHUNK_VECTORS,
    SPEC_KNOB_POLL_LIMIT,
    ChainResult,
    GATE_CLOSED,
    GATE_HALF_OPEN,
    GATE_OPEN,
    NgramResult,
    PreparedCall,
    SpecError,
    SpecGate,
    TreeMaskResult,
    TreeResult,
    knob,
    lib,
    loaded_library_path,
    ngram_propose,
    prepare_ngram_propose,
    prepare_spec_commit_path,
    prepare_spec_verify_chain,
    prepare_spec_tree_mask,
    prepare_spec_verify_tree,
    prepare_spec_verify_tree_greedy,
    spec_chain_phase_stamps,
    spec_commit_path,
    spec_get_knob,
    spec_set_knob,
    spec_probe_copy,
    spec_probe_read,
    spec_timing_collect,
    spec_timing_enable,
    spec_timing_reset,
    spec_tree_mask,
    spec_verify_chain,
    spec_verify_chain_noalloc,
    spec_verify_chain_workspace_size,
    spec_verify_tree,
    spec_verify_tree_greedy,
)
