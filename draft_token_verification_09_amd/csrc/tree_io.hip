// The steps on either side of tree verification.
//
// Before it: "Speculative Decoding in Production: From Draft Models to EAGLE-3 Dynamic
// Trees ..." (blog.llmgo.top), section III.2 "The Tree Attention Verification
// Mechanism": the candidate tree is flattened into one sequence and scored in one
// target pass under a 2-D mask.  spec_tree_mask builds that mask (node i sees node j
// iff j lies on the root path of i, i included) and every node's depth.
//
// After it: "Speculative decoding: Medusa, EAGLE, vLLM" (vikram-blog.pages.dev),
// "System Topology & Data Flow": the accepted branch goes into the KV cache.
// spec_commit_path copies the cache entries of the root and the accepted nodes from
// the pass's per-node buffer to the sequence's next cache positions.
//
// tree_mask: one workgroup per (tree, block of 64 rows).  The parent array sits in
// shared memory; each row's ancestor set is a bitset there, built by one lane walking
// up to the root; the rows' bytes are then written as 16-byte vectors (the block's
// rows are one contiguous byte range of the output).
// commit_path: a pure copy, bound by HBM.  One workgroup moves 16 KB of one entry with
// 16-byte non-temporal loads and stores; entries past the accepted length exit at once.
#include "device_common.h"
#include "host_runtime.h"
#include "spec_verify.h"

namespace specv {

constexpr int kMaskThreads = 256;
constexpr int kMaskRows = 64;  // mask rows per workgroup
constexpr int kMaskWords = SPEC_MAX_TREE_NODES / 32;

__global__ __launch_bounds__(kMaskThreads) void tree_mask_kernel(const int32_t* parent, int N1, int blocks_per_tree,
                                                                 uint8_t* mask, int32_t* depth_out) {
  __shared__ int s_par[SPEC_MAX_TREE_NODES];
  __shared__ uint32_t s_bits[kMaskRows * kMaskWords];
  const int tid = threadIdx.x;
  const int b = blockIdx.x / blocks_per_tree;
  const int r0 = (blockIdx.x - b * blocks_per_tree) * kMaskRows;
  const int rows = min(kMaskRows, N1 - r0);
  const int W32 = (N1 + 31) >> 5;
  const int32_t* par = parent + static_cast<size_t>(b) * N1;
  int bad = 0;
  for (int i = tid; i < N1; i += kMaskThreads) {
    const int p = par[i];
    s_par[i] = p;
    bad |= i == 0 ? p != -1 : (p < 0 || p >= i);
  }
  for (int w = tid; w < rows * W32; w += kMaskThreads) s_bits[w] = 0u;
  bad = __syncthreads_or(bad);
  if (tid < rows) {
    // Parents precede their children, so the walk ends at the root within i steps.
    const int i = r0 + tid;
    int d = -1;
    if (!bad) {
      uint32_t* row = s_bits + tid * W32;
      int v = i;
      d = 0;
      row[v >> 5] |= 1u << (v & 31);
      while (v != 0) {
        v = s_par[v];
        row[v >> 5] |= 1u << (v & 31);
        ++d;
      }
    }
    if (depth_out) depth_out[static_cast<size_t>(b) * N1 + i] = d;
  }
  if (!mask) return;
  __syncthreads();
  // Rows [r0, r0 + rows) of tree b are the byte range [0, nbytes) from `base`.
  uint8_t* base = mask + static_cast<size_t>(b) * N1 * N1 + static_cast<size_t>(r0) * N1;
  const int nbytes = rows * N1;
  const int head = min(static_cast<int>((16u - (reinterpret_cast<uintptr_t>(base) & 15u)) & 15u), nbytes);
  const int nvec = (nbytes - head) >> 4;
  const int tail0 = head + (nvec << 4);
  auto bit_at = [&](int r, int c) -> uint32_t { return (s_bits[r * W32 + (c >> 5)] >> (c & 31)) & 1u; };
  if (tid < head) base[tid] = static_cast<uint8_t>(bit_at(tid / N1, tid % N1));
  if (tid < nbytes - tail0) {
    const int f = tail0 + tid;
    base[f] = static_cast<uint8_t>(bit_at(f / N1, f % N1));
  }
  for (int v = tid; v < nvec; v += kMaskThreads) {
    const int f = head + (v << 4);
    int r = f / N1, c = f - r * N1;
    u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      out[e >> 2] |= bit_at(r, c) << (8 * (e & 3));
      if (++c == N1) {
        c = 0;
        ++r;
      }
    }
    *reinterpret_cast<u32x4*>(base + f) = out;
  }
}

constexpr int kCommitThreads = 256;
constexpr int kCommitUnroll = 4;                                 // vectors per lane
constexpr int kCommitVecs = kCommitThreads * kCommitUnroll;      // 16-byte vectors per workgroup

struct CommitArgs {
  const char* src;
  char* dst;
  const int32_t* path;  // [B, P] accepted nodes, root excluded; NULL = chain
  const int32_t* acc;
  const int32_t* clen;
  int32_t* out_len;
  int B, N1, P, L_cap, E_max, chunks;
  uint32_t vpp;  // 16-byte vectors per plane of one entry
  uint32_t vpe;  // 16-byte vectors per entry (all planes)
  size_t entry_bytes, src_plane, dst_plane;
};

__global__ __launch_bounds__(kCommitThreads) void commit_path_kernel(CommitArgs a) {
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x % a.chunks;
  const int rest = blockIdx.x / a.chunks;
  const int k = rest % a.E_max;
  const int b = rest / a.E_max;
  const bool reporter = chunk == 0 && k == 0;  // writes the sequence's new length
  const int n = a.acc[b];
  const int c0 = a.clen[b];
  const bool ok = n >= 0 && c0 >= 0 && static_cast<long long>(c0) + n + 1 <= a.L_cap &&
                  (a.path ? n <= a.P : n <= a.N1 - 1);
  if (!ok) {
    if (reporter && tid == 0 && a.out_len) a.out_len[b] = -1;
    return;
  }
  if (k > n) return;
  if (a.path) {
    int bad = 0;
    for (int t = tid; t < n; t += kCommitThreads) {
      const int v = a.path[static_cast<size_t>(b) * a.P + t];
      bad |= v < 0 || v >= a.N1;
    }
    if (__syncthreads_or(bad)) {
      if (reporter && tid == 0 && a.out_len) a.out_len[b] = -1;
      return;
    }
  }
  if (reporter && tid == 0 && a.out_len) a.out_len[b] = c0 + n + 1;
  const int node = k == 0 ? 0 : (a.path ? a.path[static_cast<size_t>(b) * a.P + k - 1] : k);
  const char* src = a.src + (static_cast<size_t>(b) * a.N1 + node) * a.entry_bytes;
  char* dst = a.dst + (static_cast<size_t>(b) * a.L_cap + c0 + k) * a.entry_bytes;
  const uint32_t v0 = static_cast<uint32_t>(chunk) * kCommitVecs + tid;
  u32x4 r[kCommitUnroll];
#pragma unroll
  for (int j = 0; j < kCommitUnroll; ++j) {
    const uint32_t v = v0 + j * kCommitThreads;
    if (v < a.vpe) {
      const uint32_t plane = v / a.vpp;
      const uint32_t off = v - plane * a.vpp;
      r[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + plane * a.src_plane) + off);
    }
  }
#pragma unroll
  for (int j = 0; j < kCommitUnroll; ++j) {
    const uint32_t v = v0 + j * kCommitThreads;
    if (v < a.vpe) {
      const uint32_t plane = v / a.vpp;
      const uint32_t off = v - plane * a.vpp;
      __builtin_nontemporal_store(r[j], reinterpret_cast<u32x4*>(dst + plane * a.dst_plane) + off);
    }
  }
}

}  // namespace specv

using namespace specv;

extern "C" {

spec_status_t spec_tree_mask(const int32_t* parent, int B, int N1, uint8_t* out_mask, int32_t* out_depth,
                             spec_stream_t stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B < 0 || N1 < 1) return fail(SPEC_ERR_INVALID_ARG, "need B >= 0, N1 >= 1");
  if (N1 > SPEC_MAX_TREE_NODES) return fail(SPEC_ERR_UNSUPPORTED, "N1 = %d exceeds SPEC_MAX_TREE_NODES", N1);
  if (B == 0) return SPEC_OK;
  if (!parent) return fail(SPEC_ERR_INVALID_ARG, "parent is NULL");
  if (!out_mask && !out_depth) return fail(SPEC_ERR_INVALID_ARG, "out_mask and out_depth are both NULL");
  const int bpt = (N1 + kMaskRows - 1) / kMaskRows;
  if (static_cast<long long>(B) * bpt > 2147483647LL) return fail(SPEC_ERR_UNSUPPORTED, "grid too large");
  LaunchScope scope("tree_mask", s);
  scope.launch(tree_mask_kernel, dim3(static_cast<unsigned>(B * bpt)), dim3(kMaskThreads), s, parent, N1, bpt,
               out_mask, out_depth);
  return scope.finish();
}

spec_status_t spec_commit_path(const void* kv_nodes, const int32_t* path_nodes, int path_stride,
                               const int32_t* accept_len, const int32_t* cache_len,
                               int B, int N1, int L_cap, int planes, size_t entry_bytes,
                               size_t node_plane_stride, size_t cache_plane_stride,
                               void* kv_cache, int32_t* out_cache_len, spec_stream_t stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B < 0 || N1 < 1 || L_cap < 1 || planes < 1)
    return fail(SPEC_ERR_INVALID_ARG, "need B >= 0, N1 >= 1, L_cap >= 1, planes >= 1");
  if (entry_bytes == 0 || entry_bytes % 16)
    return fail(SPEC_ERR_INVALID_ARG, "entry_bytes = %zu is not a positive multiple of 16", entry_bytes);
  if (path_nodes && (path_stride < 1 || path_stride > SPEC_MAX_TREE_NODES + 1))
    return fail(SPEC_ERR_INVALID_ARG, "path_stride = %d outside [1, SPEC_MAX_TREE_NODES + 1]", path_stride);
  if (planes > 1) {
    if (node_plane_stride % 16 || cache_plane_stride % 16)
      return fail(SPEC_ERR_INVALID_ARG, "plane strides must be multiples of 16 bytes");
    if (node_plane_stride < static_cast<size_t>(B) * N1 * entry_bytes ||
        cache_plane_stride < static_cast<size_t>(B) * L_cap * entry_bytes)
      return fail(SPEC_ERR_INVALID_ARG, "a plane stride is smaller than one plane");
  }
  if (B == 0) return SPEC_OK;
  if (!kv_nodes || !kv_cache || !accept_len || !cache_len) return fail(SPEC_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(kv_nodes) || !aligned16(kv_cache))
    return fail(SPEC_ERR_INVALID_ARG, "kv_nodes and kv_cache must be 16-byte aligned");
  const unsigned long long vpe = static_cast<unsigned long long>(planes) * (entry_bytes / 16);
  if (vpe > 2147483647ULL) return fail(SPEC_ERR_UNSUPPORTED, "entry of %llu vectors is too large", vpe);
  CommitArgs a{};
  a.src = static_cast<const char*>(kv_nodes);
  a.dst = static_cast<char*>(kv_cache);
  a.path = path_nodes;
  a.acc = accept_len;
  a.clen = cache_len;
  a.out_len = out_cache_len;
  a.B = B;
  a.N1 = N1;
  a.P = path_nodes ? path_stride : 0;
  a.L_cap = L_cap;
  a.E_max = path_nodes ? path_stride + 1 : N1;
  a.chunks = static_cast<int>((vpe + kCommitVecs - 1) / kCommitVecs);
  a.vpp = static_cast<uint32_t>(entry_bytes / 16);
  a.vpe = static_cast<uint32_t>(vpe);
  a.entry_bytes = entry_bytes;
  a.src_plane = node_plane_stride;
  a.dst_plane = cache_plane_stride;
  const long long grid = static_cast<long long>(B) * a.E_max * a.chunks;
  if (grid > 2147483647LL) return fail(SPEC_ERR_UNSUPPORTED, "grid too large");
  LaunchScope scope("commit_path", s);
  scope.launch(commit_path_kernel, dim3(static_cast<unsigned>(grid)), dim3(kCommitThreads), s, a);
  return scope.finish();
}

}  // extern "C"
