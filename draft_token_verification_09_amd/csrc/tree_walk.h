// Tree walks shared between translation units: the greedy walk serves
// spec_verify_tree_greedy when no per-node argmax is asked for.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

namespace specv {

// Workspace bytes of the walks for this shape (0 if V needs too many slices).
size_t tree_walk_workspace_bytes(int B, int N1, int V, spec_dtype_t dtype);

// Greedy tree verification reading only the accepted nodes' rows.  Arguments as for
// spec_verify_tree_greedy (out_argmax is not produced); host checks done by the caller.
spec_status_t tree_greedy_walk(const void* target_logits, spec_dtype_t dtype, const int32_t* parent,
                               const int32_t* node_token, int B, int N1, int V, int max_depth,
                               int32_t* out_accept_len, int32_t* out_tokens, int32_t* out_path_nodes,
                               void* workspace, size_t workspace_bytes, hipStream_t s);

}  // namespace specv
