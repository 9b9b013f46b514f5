// Greedy tree verification, batched over sequences.
//
// "Speculative Decoding in Production: From Draft Models to EAGLE-3 Dynamic Trees"
// (blog.llmgo.top), section III.2: every branch of the flattened draft tree is
// scored in one target pass and a matching branch is accepted even if a sibling
// is rejected.  "Speculative decoding: Medusa, EAGLE, vLLM" (vikram-blog.pages.dev),
// "System Topology & Data Flow" figure, and its temperature-0 usage example.
// Readings: node i is accepted iff its parent is accepted and token[i] equals the
// argmax of the parent's row (smallest index on ties, raw logits); the path ends at
// the deepest accepted node (smallest node index on ties); the bonus is that node's
// row argmax.
//
// Two kernels.  tree_argmax (grid = B x N1 x C): each workgroup finds (max, first index)
// over one chunk of one node row (non-temporal loads).  tree_select (grid = B) combines
// the chunks into per-node argmaxes, validates the topology, walks each node's path to
// the root in parallel (one lane per node), picks the deepest accepted node and writes
// the compacted path.  Nothing in the workspace outlives a call.
#include <math.h>

#include "device_common.h"
#include "host_runtime.h"
#include "spec_verify.h"
#include "tree_walk.h"

namespace specv {

struct ArgMax {
  float v;
  int i;
};

struct TreeArgs {
  const void* target;
  const int32_t* parent;
  const int32_t* token;
  int B, N1, V, C, max_depth;
  int32_t* out_len;
  int32_t* out_tokens;
  int32_t* out_nodes;
  int32_t* out_argmax;
  ArgMax* part;  // [B, N1, C]
};

constexpr int kStageT = 2048;  // chunk partials staged in shared memory per batch of rows

// grid = B.  Topology and partials are staged in shared memory first, so the path walks
// below touch no global memory.
__global__ __launch_bounds__(kThreads) void tree_select_kernel(TreeArgs a) {
  const int b = blockIdx.x;
  __shared__ int s_amax[SPEC_MAX_TREE_NODES];
  __shared__ int s_par[SPEC_MAX_TREE_NODES];
  __shared__ int s_tok[SPEC_MAX_TREE_NODES];
  __shared__ float st_v[kStageT];
  __shared__ int st_i[kStageT];
  __shared__ int s_key[kWaves];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int N1 = a.N1;
  const int C = a.C;
  const int32_t* par = a.parent + static_cast<size_t>(b) * N1;
  const int32_t* tok = a.token + static_cast<size_t>(b) * N1;
  for (int i = tid; i < N1; i += kThreads) {
    s_par[i] = par[i];
    s_tok[i] = tok[i];
  }
  if (tid == 0) s_bad = 0;

  // Row argmax per node from the chunk partials: each 16-lane row of the workgroup
  // combines one node row (16 at a time), lane r taking partials r, r+16, ...
  const int rows_per_batch = max(1, kStageT / C);
  for (int r0 = 0; r0 < N1; r0 += rows_per_batch) {
    const int r1 = min(N1, r0 + rows_per_batch);
    const int items = (r1 - r0) * C;
    const ArgMax* ps = a.part + (static_cast<size_t>(b) * N1 + r0) * C;
    for (int i = tid; i < items; i += kThreads) {
      const ArgMax p = ps[i];
      st_v[i] = p.v;
      st_i[i] = p.i;
    }
    __syncthreads();
    for (int g0 = r0; g0 < r1; g0 += kThreads / 16) {
      const int r = g0 + (tid >> 4);
      const int q = tid & 15;
      float v = -INFINITY;
      int i = INT_MAX;
      if (r < r1) {
        const int base = (r - r0) * C;
        for (int c = q; c < C; c += 16) {
          if (better(st_v[base + c], st_i[base + c], v, i)) {
            v = st_v[base + c];
            i = st_i[base + c];
          }
        }
      }
      row16_argmax(v, i);
      if (r < r1 && q == 15) s_amax[r] = i;
    }
    __syncthreads();
  }
  // Topology and token checks.
  if (tid == 0 && s_par[0] != -1) s_bad = 1;
  for (int i = 1 + tid; i < N1; i += kThreads) {
    const int p = s_par[i];
    const int t = s_tok[i];
    if (p < 0 || p >= i || t < 0 || t >= a.V) atomicOr(&s_bad, 1);
  }
  __syncthreads();
  const bool bad = s_bad != 0;

  // Each lane walks its node's path: accepted iff every edge matches the parent's argmax.
  // Key = depth * 2^16 + (65535 - node) so that the maximum is the deepest, then smallest index.
  int best_key = 65535;  // root: depth 0, node 0
  if (!bad) {
    for (int i = 1 + tid; i < N1; i += kThreads) {
      int v = i, depth = 0;
      bool ok = true;
      while (v != 0) {
        const int p = s_par[v];
        ok = ok && (s_tok[v] == s_amax[p]);
        v = p;
        ++depth;
      }
      if (ok) best_key = max(best_key, (depth << 16) | (65535 - i));
    }
  }
  best_key = block_max_int(best_key, s_key);
  const int best = 65535 - (best_key & 0xffff);
  const int depth = best_key >> 16;
  const bool invalid = bad || depth > a.max_depth;

  const int D1 = a.max_depth + 1;
  int32_t* ot = a.out_tokens + static_cast<size_t>(b) * D1;
  int32_t* on = a.out_nodes + static_cast<size_t>(b) * D1;
  if (invalid) {
    for (int k = tid; k < D1; k += kThreads) {
      ot[k] = -1;
      on[k] = -1;
    }
    if (tid == 0) a.out_len[b] = -1;
  } else {
    // Lane k (k < depth) finds the node at depth k+1 on the path by walking up
    // (depth - 1 - k) steps from `best`.
    for (int k = tid; k < D1; k += kThreads) {
      if (k < depth) {
        int v = best;
        for (int s = 0; s < depth - 1 - k; ++s) v = s_par[v];
        on[k] = v;
        ot[k] = s_tok[v];
      } else {
        on[k] = -1;
        ot[k] = (k == depth) ? s_amax[best] : -1;
      }
    }
    if (tid == 0) a.out_len[b] = depth;
  }
  if (a.out_argmax)
    for (int i = tid; i < N1; i += kThreads) a.out_argmax[static_cast<size_t>(b) * N1 + i] = s_amax[i];
}

template <int DT, int NV, bool VEC>
__global__ __launch_bounds__(kThreads) void tree_argmax_kernel(TreeArgs a) {
  __shared__ float s_v[kWaves];
  __shared__ int s_i[kWaves];
  using EL = Elem<DT>;
  constexpr int E = EL::kPerVec;
  constexpr int kChunk = ChunkShape<DT, NV>::kChunk;
  const int g = xcd_blocked_index();  // chunk of this workgroup
  const int c = g % a.C;
  const int r = (g / a.C) % a.N1;
  const int b = g / (a.C * a.N1);
  const void* row = static_cast<const char*>(a.target) +
                    (static_cast<size_t>(b) * a.N1 + r) * static_cast<size_t>(a.V) * EL::kBytes;
  u32x4 raw[NV];
  load_chunk<DT, NV, VEC, true>(raw, row, a.V, c);
  // Lane-local scan in increasing vocabulary order; strict '>' keeps the first maximum.
  const int first = c * kChunk + threadIdx.x * E;
  float bv = -INFINITY;
  int bi = first < a.V ? first : INT_MAX;
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float x = EL::get(raw[j], i);
      if (x > bv) {
        bv = x;
        bi = c * kChunk + (j * kThreads + threadIdx.x) * E + i;
      }
    }
  wave_argmax(bv, bi);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_v[w] = bv;
    s_i[w] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = s_v[0];
    int i = s_i[0];
    for (int k = 1; k < kWaves; ++k)
      if (better(s_v[k], s_i[k], v, i)) {
        v = s_v[k];
        i = s_i[k];
      }
    a.part[(static_cast<size_t>(b) * a.N1 + r) * a.C + c] = ArgMax{v, i};
  }
}

struct TreeLayout {
  int nv, C;
  size_t off_part, bytes;
};

static TreeLayout tree_layout(int B, int N1, int V, spec_dtype_t dtype) {
  TreeLayout L{};
  const int epv = dtype == SPEC_BF16 ? 8 : 4;
  L.nv = choose_nv(static_cast<long long>(B) * N1, V, epv, 1024);
  const long long chunk = static_cast<long long>(L.nv) * kThreads * epv;
  L.C = static_cast<int>((V + chunk - 1) / chunk);
  size_t off = 0;
  L.off_part = off;
  off = align_up(off + sizeof(ArgMax) * static_cast<size_t>(B) * N1 * L.C, 256);
  L.bytes = off;
  return L;
}

template <int DT, int NV, bool VEC>
static spec_status_t launch_tree(const TreeArgs& a, hipStream_t s) {
  {
    const long long g = static_cast<long long>(a.B) * a.N1 * a.C;
    LaunchScope scope("tree_argmax", s);
    scope.launch((tree_argmax_kernel<DT, NV, VEC>), dim3(static_cast<unsigned>(g)), dim3(kThreads), s, a);
    const spec_status_t st = scope.finish();
    if (st != SPEC_OK) return st;
  }
  LaunchScope scope("tree_select", s);
  scope.launch(tree_select_kernel, dim3(static_cast<unsigned>(a.B)), dim3(kThreads), s, a);
  return scope.finish();
}

template <int DT>
static spec_status_t dispatch_tree(int nv, bool vec, const TreeArgs& a, hipStream_t s) {
  switch (nv) {
    case 8: return vec ? launch_tree<DT, 8, true>(a, s) : launch_tree<DT, 8, false>(a, s);
    case 4: return vec ? launch_tree<DT, 4, true>(a, s) : launch_tree<DT, 4, false>(a, s);
    case 2: return vec ? launch_tree<DT, 2, true>(a, s) : launch_tree<DT, 2, false>(a, s);
    default: return vec ? launch_tree<DT, 1, true>(a, s) : launch_tree<DT, 1, false>(a, s);
  }
}

}  // namespace specv

using namespace specv;

extern "C" {

size_t spec_verify_tree_greedy_workspace_size(int B, int N1, int V, spec_dtype_t dtype) {
  if (B <= 0 || N1 < 1 || N1 > SPEC_MAX_TREE_NODES || V < 1) return 0;
  const size_t full = tree_layout(B, N1, V, dtype).bytes;
  const size_t walk = tree_walk_workspace_bytes(B, N1, V, dtype);
  return full > walk ? full : walk;
}

spec_status_t spec_verify_tree_greedy(const void* target_logits, spec_dtype_t dtype,
                                      const int32_t* parent, const int32_t* node_token,
                                      int B, int N1, int V, int max_depth,
                                      int32_t* out_accept_len, int32_t* out_tokens, int32_t* out_path_nodes,
                                      int32_t* out_argmax,
                                      void* workspace, size_t workspace_bytes, spec_stream_t stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return fail(SPEC_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (B < 0 || N1 < 1 || V < 1 || max_depth < 0)
    return fail(SPEC_ERR_INVALID_ARG, "need B >= 0, N1 >= 1, V >= 1, max_depth >= 0");
  if (N1 > SPEC_MAX_TREE_NODES) return fail(SPEC_ERR_UNSUPPORTED, "N1 = %d exceeds SPEC_MAX_TREE_NODES", N1);
  if (max_depth > N1) return fail(SPEC_ERR_INVALID_ARG, "max_depth = %d exceeds N1 = %d", max_depth, N1);
  if (B == 0) return SPEC_OK;
  if (!target_logits || !parent || !node_token || !out_accept_len || !out_tokens || !out_path_nodes)
    return fail(SPEC_ERR_INVALID_ARG, "a required pointer is NULL");
  if (static_cast<double>(B) * N1 * V >= 140737488355328.0) return fail(SPEC_ERR_UNSUPPORTED, "B*N1*V too large");
  const TreeLayout L = tree_layout(B, N1, V, dtype);
  if (static_cast<double>(B) * N1 * L.C > 2147483647.0) return fail(SPEC_ERR_UNSUPPORTED, "grid too large");
  if (L.C > kStageT) return fail(SPEC_ERR_UNSUPPORTED, "V = %d needs more than %d chunks", V, kStageT);
  if (!workspace) return fail(SPEC_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(SPEC_ERR_WORKSPACE, "workspace not 256-byte aligned");
  // Without per-node argmaxes only the accepted nodes' rows are needed: walk the tree.
  if (!out_argmax && tree_walk_workspace_bytes(B, N1, V, dtype) > 0)
    return tree_greedy_walk(target_logits, dtype, parent, node_token, B, N1, V, max_depth, out_accept_len, out_tokens,
                            out_path_nodes, workspace, workspace_bytes, s);
  if (workspace_bytes < L.bytes)
    return fail(SPEC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.bytes);
  TreeArgs a{};
  a.target = target_logits;
  a.parent = parent;
  a.token = node_token;
  a.B = B;
  a.N1 = N1;
  a.V = V;
  a.C = L.C;
  a.max_depth = max_depth;
  a.out_len = out_accept_len;
  a.out_tokens = out_tokens;
  a.out_nodes = out_path_nodes;
  a.out_argmax = out_argmax;
  char* ws = static_cast<char*>(workspace);
  a.part = reinterpret_cast<ArgMax*>(ws + L.off_part);
  const int esize = dtype == SPEC_BF16 ? 2 : 4;
  const bool vec = (static_cast<size_t>(V) * esize) % 16 == 0 && aligned16(target_logits);
  if (dtype == SPEC_BF16) return dispatch_tree<kBF16>(L.nv, vec, a, s);
  return dispatch_tree<kF32>(L.nv, vec, a, s);
}

}  // extern "C"
