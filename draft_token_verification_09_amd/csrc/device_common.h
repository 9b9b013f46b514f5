// Device-side building blocks shared by the verification kernels (gfx950, wave64).
//
// * Vocabulary streaming: a workgroup of 256 lanes covers one "chunk" of a row as
//   NV segments; in segment j lane t holds one 16-byte vector (4 fp32 or 8 bf16
//   logits) at element (j*256 + t)*E, so each wave instruction reads 1 KiB of
//   contiguous memory and, inside a segment, vocabulary order is lane order.
// * Reductions use cross-lane DPP within a wave and a small LDS array across the 4
//   waves of a workgroup.
// * Partial results pass between kernels through the workspace (the stream orders the
//   kernels); inside a kernel, workgroups hand values over through agent-scope atomic
//   loads and agent-scope or, within one XCD, workgroup-scope atomic stores (see
//   "cross-workgroup hand-off" below).
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

namespace specv {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.44269504088896340736f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum DType : int { kF32 = 0, kBF16 = 1 };

template <int DT>
struct Elem;

template <>
struct Elem<kF32> {
  static constexpr int kPerVec = 4;
  static constexpr int kBytes = 4;
  static constexpr uint32_t kNegInfBits = 0xff800000u;
  __device__ static __forceinline__ float get(const u32x4& v, int i) { return __uint_as_float(v[i]); }
  __device__ static __forceinline__ uint32_t bits(const void* base, size_t idx) {
    return reinterpret_cast<const uint32_t*>(base)[idx];
  }
  __device__ static __forceinline__ float value(const void* base, size_t idx) {
    return reinterpret_cast<const float*>(base)[idx];
  }
  __device__ static __forceinline__ float from_bits(uint32_t b) { return __uint_as_float(b); }
  // pack E element bit patterns (already in the low bits) into a vector
  __device__ static __forceinline__ void put(u32x4& v, int i, uint32_t b) { v[i] = b; }
};

template <>
struct Elem<kBF16> {
  static constexpr int kPerVec = 8;
  static constexpr int kBytes = 2;
  static constexpr uint32_t kNegInfBits = 0xff80u;
  __device__ static __forceinline__ float get(const u32x4& v, int i) {
    const uint32_t w = v[i >> 1];
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  __device__ static __forceinline__ uint32_t bits(const void* base, size_t idx) {
    return reinterpret_cast<const uint16_t*>(base)[idx];
  }
  __device__ static __forceinline__ float value(const void* base, size_t idx) {
    return __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(base)[idx]) << 16);
  }
  __device__ static __forceinline__ float from_bits(uint32_t b) { return __uint_as_float(b << 16); }
  __device__ static __forceinline__ void put(u32x4& v, int i, uint32_t b) {
    uint32_t w = v[i >> 1];
    w = (i & 1) ? ((w & 0x0000ffffu) | (b << 16)) : ((w & 0xffff0000u) | b);
    v[i >> 1] = w;
  }
};

template <int DT, int NV>
struct ChunkShape {
  static constexpr int E = Elem<DT>::kPerVec;
  static constexpr int kSegment = kThreads * E;  // elements per segment
  static constexpr int kChunk = NV * kSegment;   // elements per chunk
};

// 16-byte vector load; NT marks it non-temporal (streamed once: no reuse expected).
template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if (NT) return __builtin_nontemporal_load(p);
  return *p;
}

// Load chunk `c` of a row of V logits into registers.  Elements past V read as -inf.
// VEC: the row starts 16-byte aligned and holds a whole number of 16-byte vectors, so
// every vector lies either wholly inside the row or wholly past its end.
template <int DT, int NV, bool VEC, bool NT = false>
__device__ __forceinline__ void load_chunk(u32x4 (&raw)[NV], const void* row, int V, int c) {
  using EL = Elem<DT>;
  constexpr int E = EL::kPerVec;
  constexpr uint32_t kNegInf2 = EL::kNegInfBits | (E == 8 ? (EL::kNegInfBits << 16) : 0u);
  const int base = c * ChunkShape<DT, NV>::kChunk;
  const int lane = threadIdx.x;
  if (VEC) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const char*>(row) +
                                                    static_cast<size_t>(base) * EL::kBytes);
    if (base + ChunkShape<DT, NV>::kChunk <= V) {
#pragma unroll
      for (int j = 0; j < NV; ++j) raw[j] = load16<NT>(p + j * kThreads + lane);
    } else {
#pragma unroll
      for (int j = 0; j < NV; ++j)
        raw[j] = base + (j * kThreads + lane) * E < V ? load16<NT>(p + j * kThreads + lane)
                                                       : u32x4{kNegInf2, kNegInf2, kNegInf2, kNegInf2};
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int e0 = base + (j * kThreads + lane) * E;
    u32x4 v = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int e = e0 + i;
      EL::put(v, i, e < V ? EL::bits(row, e) : EL::kNegInfBits);
    }
    raw[j] = v;
  }
}

// Load the one vector of a row that starts at element e0 (a multiple of E); elements
// past V read as -inf.
template <int DT, bool VEC>
__device__ __forceinline__ u32x4 load_vector(const void* row, int V, int e0) {
  using EL = Elem<DT>;
  constexpr int E = EL::kPerVec;
  if (VEC) {
    constexpr uint32_t kNegInf2 = EL::kNegInfBits | (E == 8 ? (EL::kNegInfBits << 16) : 0u);
    if (e0 < V)
      return *reinterpret_cast<const u32x4*>(static_cast<const char*>(row) + static_cast<size_t>(e0) * EL::kBytes);
    return u32x4{kNegInf2, kNegInf2, kNegInf2, kNegInf2};
  }
  u32x4 v = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < E; ++i) EL::put(v, i, e0 + i < V ? EL::bits(row, e0 + i) : EL::kNegInfBits);
  return v;
}

// Raw buffer descriptor over `bytes` bytes from p (the word-3 value of raw buffer access on
// this architecture family); loads through it past `bytes` return zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0), bytes, 0x00020000);
}

// 16-byte load at byte offset `off` through a buffer descriptor; NT as for load16 (the
// cache-policy operand's non-temporal bit).
template <bool NT>
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, NT ? 2 : 0);
}

// Load chunk `c` of a row so that wave w of the workgroup holds the w-th quarter of it as
// one contiguous span: vector j of lane l of wave w is element ((w*NV + j)*64 + l)*E of the
// chunk.  Each wave instruction still reads 1 KiB of contiguous memory.  Elements past V
// read as -inf; VEC as for load_chunk.
template <int DT, int NV, bool VEC, bool NT = false>
__device__ __forceinline__ void load_wave_span(u32x4 (&raw)[NV], const void* row, int V, int c) {
  using EL = Elem<DT>;
  constexpr int E = EL::kPerVec;
  constexpr uint32_t kNegInf2 = EL::kNegInfBits | (E == 8 ? (EL::kNegInfBits << 16) : 0u);
  const int base = c * ChunkShape<DT, NV>::kChunk;
  const int first = (static_cast<int>(threadIdx.x >> 6) * NV * 64 + static_cast<int>(threadIdx.x & 63));  // vector index
  if (VEC) {
    // A buffer descriptor spans the chunk's bytes of the row (fewer in a ragged last chunk):
    // the hardware's range check reads vectors past the row's end as zeros, so every load
    // issues unconditionally from one 32-bit offset, and those vectors become -inf afterwards.
    constexpr int kChunkBytes = ChunkShape<DT, NV>::kChunk * EL::kBytes;
    const long long rem = static_cast<long long>(V - base) * EL::kBytes;
    const int nrec = rem < kChunkBytes ? static_cast<int>(rem) : kChunkBytes;
    const __amdgpu_buffer_rsrc_t rs = chunk_rsrc(static_cast<const char*>(row) + static_cast<size_t>(base) * EL::kBytes,
                                                 nrec);
#pragma unroll
    for (int j = 0; j < NV; ++j) raw[j] = buffer_load16<NT>(rs, (first + j * 64) * 16);
    if (nrec < kChunkBytes) {
#pragma unroll
      for (int j = 0; j < NV; ++j)
        if (base + (first + j * 64) * E >= V) raw[j] = u32x4{kNegInf2, kNegInf2, kNegInf2, kNegInf2};
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int e0 = base + (first + j * 64) * E;
    u32x4 v = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int e = e0 + i;
      EL::put(v, i, e < V ? EL::bits(row, e) : EL::kNegInfBits);
    }
    raw[j] = v;
  }
}

// Workgroup -> chunk order for the streaming passes.  The chip deals consecutive workgroups
// of a launch to its 8 XCDs in turn (each XCD with its own L2 and address translation caches).
// When the grid is a multiple of 8, XCD x (workgroups x, x+8, x+16, ...) takes chunks
// [x*G/8, (x+1)*G/8) in order, so that each XCD streams one contiguous eighth of the rows;
// otherwise chunks follow the workgroup index.  (Measured: chain stats pass 31.0 -> 30.2 us
// at B=64, K=5, V=128256 bf16, 33.1 -> 32.4 us with one-hot drafts at B=128; tree argmax
// pass 74.9 -> 71.8 us at B=32, 61 rows, V=128256 bf16.)
constexpr int kXcds = 8;

// The same order for workgroup i of a range of G workgroups within a launch (where the range
// starts at a multiple of 8, its workgroup i sits on XCD i % 8 as well).
__device__ __forceinline__ int xcd_blocked(int i, int G) {
  return G % kXcds == 0 ? (i % kXcds) * (G / kXcds) + i / kXcds : i;
}

__device__ __forceinline__ int xcd_blocked_index() {
  return xcd_blocked(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
}

// ---------------------------------------------------------------- wave64 scans and reductions
//
// Cross-lane steps use DPP (data-parallel primitives: operands read from another lane
// inside the VALU, no LDS round trip): row_shr:1,2,4,8 scan each 16-lane row, then
// row_bcast:15 (rows 1, 3) and row_bcast:31 (rows 2, 3) carry the row totals across, which
// yields an inclusive scan over the wave; lane 63 then holds the total and
// v_readlane broadcasts it.  Every lane of the wave must be active.

namespace dppc {
constexpr int kRowShr1 = 0x111;
constexpr int kRowShr2 = 0x112;
constexpr int kRowShr4 = 0x114;
constexpr int kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;
}  // namespace dppc

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_int(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xf, false);
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_float(float old, float v) {
  return __int_as_float(dpp_int<CTRL, ROW_MASK>(__float_as_int(old), __float_as_int(v)));
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_double(double old, double v) {
  const long long o = __double_as_longlong(old), x = __double_as_longlong(v);
  const int lo = dpp_int<CTRL, ROW_MASK>(static_cast<int>(o), static_cast<int>(x));
  const int hi = dpp_int<CTRL, ROW_MASK>(static_cast<int>(o >> 32), static_cast<int>(x >> 32));
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}

// A value known to be the same in every lane, moved to a scalar register so that the
// compiler treats it as uniform (scalar branches, no per-lane copies).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uniform(float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); }
__device__ __forceinline__ double uniform(double v) {
  const long long x = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readfirstlane(static_cast<int>(x));
  const int hi = __builtin_amdgcn_readfirstlane(static_cast<int>(x >> 32));
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}

__device__ __forceinline__ float lane_broadcast(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ int lane_broadcast(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ double lane_broadcast(double v, int lane) {
  const long long x = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(x), lane);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(x >> 32), lane);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}

#define SPECV_WAVE_SCAN(T, DPP, OP, ID, x)              \
  do {                                                  \
    x = OP(x, DPP<dppc::kRowShr1>(ID, x));              \
    x = OP(x, DPP<dppc::kRowShr2>(ID, x));              \
    x = OP(x, DPP<dppc::kRowShr4>(ID, x));              \
    x = OP(x, DPP<dppc::kRowShr8>(ID, x));              \
    x = OP(x, (DPP<dppc::kRowBcast15, 0xa>(ID, x)));    \
    x = OP(x, (DPP<dppc::kRowBcast31, 0xc>(ID, x)));    \
  } while (0)

__device__ __forceinline__ double add_d(double a, double b) { return a + b; }
__device__ __forceinline__ int add_i(int a, int b) { return a + b; }
__device__ __forceinline__ int min_i(int a, int b) { return min(a, b); }
__device__ __forceinline__ int max_i(int a, int b) { return max(a, b); }
__device__ __forceinline__ float max_f(float a, float b) { return fmaxf(a, b); }

// Inclusive scans over the lanes of a wave (lane order).
__device__ __forceinline__ double wave_inclusive_scan(double v) {
  SPECV_WAVE_SCAN(double, dpp_double, add_d, 0.0, v);
  return v;
}
__device__ __forceinline__ int wave_inclusive_scan_int(int v) {
  SPECV_WAVE_SCAN(int, dpp_int, add_i, 0, v);
  return v;
}

// Inclusive max-scan within each 16-lane row of the wave (lane 15 of a row holds the max).
__device__ __forceinline__ float row16_inclusive_max(float v) {
  v = fmaxf(v, dpp_float<dppc::kRowShr1>(-INFINITY, v));
  v = fmaxf(v, dpp_float<dppc::kRowShr2>(-INFINITY, v));
  v = fmaxf(v, dpp_float<dppc::kRowShr4>(-INFINITY, v));
  v = fmaxf(v, dpp_float<dppc::kRowShr8>(-INFINITY, v));
  return v;
}

// Inclusive scan within each 16-lane row of the wave (lane 15 of a row holds its total).
__device__ __forceinline__ double row16_inclusive_sum(double v) {
  v += dpp_double<dppc::kRowShr1>(0.0, v);
  v += dpp_double<dppc::kRowShr2>(0.0, v);
  v += dpp_double<dppc::kRowShr4>(0.0, v);
  v += dpp_double<dppc::kRowShr8>(0.0, v);
  return v;
}

// Reductions: every lane receives the result.
__device__ __forceinline__ float wave_max(float v) {
  SPECV_WAVE_SCAN(float, dpp_float, max_f, -INFINITY, v);
  return lane_broadcast(v, 63);
}
__device__ __forceinline__ double wave_sum(double v) { return lane_broadcast(wave_inclusive_scan(v), 63); }
__device__ __forceinline__ int wave_min_int(int v) {
  SPECV_WAVE_SCAN(int, dpp_int, min_i, INT_MAX, v);
  return lane_broadcast(v, 63);
}
__device__ __forceinline__ int wave_max_int(int v) {
  SPECV_WAVE_SCAN(int, dpp_int, max_i, INT_MIN, v);
  return lane_broadcast(v, 63);
}

// ---- (max, first index) pairs

// (v, i) beats (w, j) if v > w, or v == w and i < j.
__device__ __forceinline__ bool better(float v, int i, float w, int j) { return v > w || (v == w && i < j); }

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float ov = dpp_float<CTRL, ROW_MASK>(-INFINITY, v);
  const int oi = dpp_int<CTRL, ROW_MASK>(INT_MAX, i);
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

// (max, first index) over each 16-lane row of the wave; lane 15 of a row holds the result.
__device__ __forceinline__ void row16_argmax(float& v, int& i) {
  argmax_step<dppc::kRowShr1>(v, i);
  argmax_step<dppc::kRowShr2>(v, i);
  argmax_step<dppc::kRowShr4>(v, i);
  argmax_step<dppc::kRowShr8>(v, i);
}

// Wave-wide (max, first index) with DPP steps; every lane gets it.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_step<dppc::kRowShr1>(v, i);
  argmax_step<dppc::kRowShr2>(v, i);
  argmax_step<dppc::kRowShr4>(v, i);
  argmax_step<dppc::kRowShr8>(v, i);
  argmax_step<dppc::kRowBcast15, 0xa>(v, i);
  argmax_step<dppc::kRowBcast31, 0xc>(v, i);
  v = lane_broadcast(v, 63);
  i = lane_broadcast(i, 63);
}

// Exclusive scan of one int per lane over the workgroup (lane order); *total gets the sum.
// NW = waves in the workgroup; lds holds NW ints.
template <int NW = kWaves>
__device__ __forceinline__ int block_exclusive_scan_int(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int incl = wave_inclusive_scan_int(v);
  __syncthreads();
  if (lane == 63) lds[w] = incl;
  __syncthreads();
  int before = incl - v, sum = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    if (i < w) before += lds[i];
    sum += lds[i];
  }
  *total = sum;
  return before;
}

// Workgroup-wide reductions (every lane receives the result).  Contain __syncthreads.
template <int NW = kWaves>
__device__ __forceinline__ float block_max(float v, float* lds) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[w] = v;
  __syncthreads();
  float r = lds[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = fmaxf(r, lds[i]);
  return r;
}

template <int NW = kWaves>
__device__ __forceinline__ double block_sum(double v, double* lds) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[w] = v;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int i = 0; i < NW; ++i) r += lds[i];
  return r;
}

template <int NW = kWaves>
__device__ __forceinline__ int block_min_int(int v, int* lds) {
  v = wave_min_int(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[w] = v;
  __syncthreads();
  int r = lds[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = min(r, lds[i]);
  return r;
}

template <int NW = kWaves>
__device__ __forceinline__ int block_max_int(int v, int* lds) {
  v = wave_max_int(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[w] = v;
  __syncthreads();
  int r = lds[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = max(r, lds[i]);
  return r;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- cross-workgroup hand-off
//
// The 8 XCDs of the chip each have their own L2, which is not coherent with the others
// for plain loads and stores.  A value one workgroup hands to another inside a kernel is
// therefore written with an agent-scope atomic store and read with an agent-scope atomic
// load (both coherent across XCDs), or between workgroups of one XCD with the XCD-local store
// below and the same load.  Nothing handed over goes through a plain store, so
// no L2 write-back fence is needed (such a fence costs tens of microseconds per kernel on
// this part).  Between kernels of one stream, plain stores and loads suffice.

template <class T>
__device__ __forceinline__ void store_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class T>
__device__ __forceinline__ T load_agent(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// XCD-local hand-over.  A workgroup-scope store lands in the writer's L2 and goes no further
// while the kernel runs; an agent-scope load reads through its own XCD's L2, which returns a
// line written there and fetches any other from memory.  So a word written that way by a
// workgroup and read with load_agent by a workgroup on the same XCD arrives in one L2 round
// trip instead of a trip through memory (two workgroups ping-ponging one word each way:
// 0.42-0.44 us a round trip against 0.82-1.03 us with agent-scope stores), while a reader on
// another XCD would never see it.  The hardware dispatches a grid's workgroups to the XCDs
// in turn (workgroup i to XCD i mod 8 in the single-partition mode; in the modes with fewer
// XCDs a partition, i mod 8 still fixes the XCD), so workgroups whose grid indices agree
// mod 8 share an L2.  A writer uses the local store only for words whose readers' indices
// agree with its own mod 8, and only when its XCD is the one its index names (so that a
// dispatch order other than this one falls back to agent-scope stores); every wait is
// bounded, so a word that did not arrive would flag its sequence rather than hang.
template <class T>
__device__ __forceinline__ void store_xcd(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

template <class T>
__device__ __forceinline__ void store_handover(T* p, T v, bool local) {
  if (local)
    store_xcd(p, v);
  else
    store_agent(p, v);
}

// Whether this workgroup runs on the XCD its grid index names (index mod 8).
__device__ __forceinline__ bool on_indexed_xcd() {
  constexpr int kXccIdReg = ((4 - 1) << 11) | 20;  // hwreg(HW_REG_XCC_ID, 0, 4)
  return static_cast<int>(__builtin_amdgcn_s_getreg(kXccIdReg)) == static_cast<int>(blockIdx.x % kXcds);
}

// Hand-over words.  A 64-bit word carries 32 payload bits in its low half and a 32-bit tag
// (the call's generation, possibly mixed with a step number) in its high half, written by
// one atomic store (agent scope, or XCD-local; see above).  A reader takes a value only when every word of it
// carries the tag it expects, so whatever a word held before (an earlier call's or step's
// words, or anything else) reads as "not written yet" unless 32 bits match by chance, and
// no clearing pass is needed.
__device__ __forceinline__ uint64_t tagged(uint32_t payload, uint32_t tag) {
  return static_cast<uint64_t>(payload) | (static_cast<uint64_t>(tag) << 32);
}

// (local: an XCD-local store, for a word whose readers share the writer's XCD)
__device__ __forceinline__ void put_tagged_u32(uint64_t* w, uint32_t v, uint32_t tag, bool local = false) {
  store_handover(w, tagged(v, tag), local);
}

__device__ __forceinline__ bool get_tagged_u32(const uint64_t* w, uint32_t tag, uint32_t* v) {
  const uint64_t x = load_agent(w);
  *v = static_cast<uint32_t>(x);
  return static_cast<uint32_t>(x >> 32) == tag;
}

// A double as two tagged words (w[0] low half of its bits, w[1] high half).
__device__ __forceinline__ void put_tagged_double(uint64_t* w, double v, uint32_t tag, bool local = false) {
  const uint64_t bits = static_cast<uint64_t>(__double_as_longlong(v));
  store_handover(w, tagged(static_cast<uint32_t>(bits), tag), local);
  store_handover(w + 1, tagged(static_cast<uint32_t>(bits >> 32), tag), local);
}

__device__ __forceinline__ bool get_tagged_double(const uint64_t* w, uint32_t tag, double* v) {
  const uint64_t lo = load_agent(w), hi = load_agent(w + 1);
  *v = __longlong_as_double(static_cast<long long>((hi << 32) | (lo & 0xffffffffull)));
  return static_cast<uint32_t>(lo >> 32) == tag && static_cast<uint32_t>(hi >> 32) == tag;
}

// Polls of a hand-over word that has not been written yet before a wait gives up (each
// poll takes at least a memory round trip, about a microsecond: a quarter of a second or
// more; the default of a host-side knob), and the pause between polls.  A sequence whose
// wait gave up is flagged with kFlagTimedOut in its count output (invalid input gives -1).
constexpr int kPollLimit = 1 << 18;
constexpr int kFlagTimedOut = -2;
__device__ __forceinline__ void short_pause() { __builtin_amdgcn_s_sleep(2); }

}  // namespace specv
