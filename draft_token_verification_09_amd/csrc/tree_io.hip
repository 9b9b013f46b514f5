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
// commit_path: a pure copy, bound by HBM.  One workgroup moves one 4 KB chunk of every
// committed entry of one sequence: 16-byte loads, the loads of four entries in flight
// together, then 16-byte non-temporal stores (measured: plain loads beat non-temporal
// ones here, non-temporal stores beat plain ones; 4 KB chunks with 4 entries in flight
// beat 8 and 16 KB chunks, and 8 entries in flight).
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
constexpr int kCommitUnroll = 1;                              // vectors per lane per entry
constexpr int kCommitBatch = 4;                               // entries whose loads are in flight together
constexpr int kCommitVecs = kCommitThreads * kCommitUnroll;   // 16-byte vectors per workgroup and entry

struct CommitArgs {
  const char* src;
  char* dst;
  const int32_t* path;  // [B, P] accepted nodes, root excluded; NULL = chain
  const int32_t* acc;
  const int32_t* clen;
  int32_t* out_len;
  int B, N1, P, L_cap, chunks;
  uint32_t vpp;  // 16-byte vectors per plane of one entry
  uint32_t vpe;  // 16-byte vectors per entry (all planes)
  size_t entry_bytes, src_plane, dst_plane;
};

// Node of the k-th committed entry (k >= 1): the path row is held one node per lane
// (`pv`, lanes 0..63) when it fits in a wave, else read from memory.
__device__ __forceinline__ int committed_node(const CommitArgs& a, const int32_t* prow, int pv, int k) {
  if (!a.path) return k;
  if (k - 1 < 64) return __builtin_amdgcn_readlane(pv, k - 1);
  return prow[k - 1];
}

// One workgroup per (sequence, 4 KB chunk of an entry), for every committed entry of
// that sequence: each wave reads the sequence's lengths and path row itself and checks
// them with a ballot, so the kernel has no barrier and three memory round trips (the
// row, the entries' chunks, the stores) however many entries are committed.
__global__ __launch_bounds__(kCommitThreads) void commit_path_kernel(CommitArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int b = blockIdx.x / a.chunks;
  const int chunk = blockIdx.x - b * a.chunks;
  const int32_t* prow = a.path ? a.path + static_cast<size_t>(b) * a.P : nullptr;
  // the path row's first 64 nodes, the lengths: loads with no dependence on each other
  const int pv = prow && lane < a.P ? prow[lane] : 0;
  const int n = a.acc[b];
  const int c0 = a.clen[b];
  bool bad = !(n >= 0 && c0 >= 0 && static_cast<long long>(c0) + n + 1 <= a.L_cap &&
               (prow ? n <= a.P : n <= a.N1 - 1));
  if (prow) {
    bad |= lane < n && (pv < 0 || pv >= a.N1);
    for (int t = lane + 64; t < n; t += 64) {
      const int v = prow[t];
      bad |= v < 0 || v >= a.N1;
    }
  }
  bad = __any(bad);
  if (chunk == 0 && tid == 0 && a.out_len) a.out_len[b] = bad ? -1 : c0 + n + 1;
  if (bad) return;
  // this lane's vectors: plane and offset do not depend on the entry
  size_t so[kCommitUnroll], dof[kCommitUnroll];
  bool live[kCommitUnroll];
#pragma unroll
  for (int j = 0; j < kCommitUnroll; ++j) {
    const uint32_t v = static_cast<uint32_t>(chunk) * kCommitVecs + j * kCommitThreads + tid;
    live[j] = v < a.vpe;
    const uint32_t plane = live[j] ? v / a.vpp : 0u;
    const uint32_t off = live[j] ? v - plane * a.vpp : 0u;
    so[j] = plane * a.src_plane + static_cast<size_t>(off) * 16;
    dof[j] = plane * a.dst_plane + static_cast<size_t>(off) * 16;
  }
  const char* sseq = a.src + static_cast<size_t>(b) * a.N1 * a.entry_bytes;
  char* dseq = a.dst + (static_cast<size_t>(b) * a.L_cap + c0) * a.entry_bytes;
  for (int k0 = 0; k0 <= n; k0 += kCommitBatch) {
    u32x4 r[kCommitBatch][kCommitUnroll];
#pragma unroll
    for (int e = 0; e < kCommitBatch; ++e) {
      const int k = k0 + e;
      if (k > n) break;
      const int node = k == 0 ? 0 : committed_node(a, prow, pv, k);
      const char* src = sseq + static_cast<size_t>(node) * a.entry_bytes;
#pragma unroll
      for (int j = 0; j < kCommitUnroll; ++j)
        if (live[j]) r[e][j] = *reinterpret_cast<const u32x4*>(src + so[j]);
    }
#pragma unroll
    for (int e = 0; e < kCommitBatch; ++e) {
      const int k = k0 + e;
      if (k > n) break;
      char* dst = dseq + static_cast<size_t>(k) * a.entry_bytes;
#pragma unroll
      for (int j = 0; j < kCommitUnroll; ++j)
        if (live[j]) __builtin_nontemporal_store(r[e][j], reinterpret_cast<u32x4*>(dst + dof[j]));
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
  a.chunks = static_cast<int>((vpe + kCommitVecs - 1) / kCommitVecs);
  a.vpp = static_cast<uint32_t>(entry_bytes / 16);
  a.vpe = static_cast<uint32_t>(vpe);
  a.entry_bytes = entry_bytes;
  a.src_plane = node_plane_stride;
  a.dst_plane = cache_plane_stride;
  const long long grid = static_cast<long long>(B) * a.chunks;
  if (grid > 2147483647LL) return fail(SPEC_ERR_UNSUPPORTED, "grid too large");
  LaunchScope scope("commit_path", s);
  scope.launch(commit_path_kernel, dim3(static_cast<unsigned>(grid)), dim3(kCommitThreads), s, a);
  return scope.finish();
}

}  // extern "C"
