// Stochastic (temperature > 0) tree verification.
//
// "Speculative Decoding in Production: From Draft Models to EAGLE-3 Dynamic Trees ..."
// (blog.llmgo.top): section I.1 gives the rule for one drafted token (accept with
// min(1, p/q), else draw from max(0, p - q) normalised) and section III.2 verifies a tree
// whose rejected branch B1 leaves its sibling B2 free to be accepted.  Reading (the
// published multi-candidate form of the rule): the children of a node were drawn
// independently from the draft distribution q at that node and are tried in node order
// against a residual target r_j, r_1 = p and r_{j+1} = max(0, r_j - q) normalised; an
// accepted child continues the walk, a node whose children are all rejected emits a draw
// from the last residual, a leaf reached by acceptance emits a bonus draw from its p.
//
// The residual after j rejections has the closed form r_{j+1} = max(0, p - c q) / D with
// c_1 = 0, D_1 = 1, c_{j+1} = c_j + D_j and D_{j+1} = sum_v max(0, p(v) - c_{j+1} q(v)), so
// each rejection needs one sum over the vocabulary and nothing else.
//
// Only the rows on the walk are read: the accepted path's target rows and the draft rows
// of its internal nodes.  The walk is sequential in depth, so it is spread over W
// workgroups per sequence, each owning one slice of the vocabulary (256 lanes x 4 vectors
// of 16 bytes; smaller slices shorten each level, which is latency-bound, and 4 vectors
// per lane measured best).  A workgroup holds its slice of the current node's two rows in registers
// for every test at that node; the per-slice sums (row maxima and exp2 sums, residual
// masses) pass between the W workgroups through generation-tagged slots, and every
// workgroup combines them in the same order, so all of them take the same decisions.  The
// workgroup whose slice holds the final draw's point searches it and writes the outputs.
//
// The greedy walk (tg_walk) serves spec_verify_tree_greedy when no per-node argmax is
// asked for: node i is accepted iff its parent is accepted and its token is the argmax
// of the parent's row, so only the accepted nodes' rows matter.  It keeps the frontier of
// accepted nodes of the current depth (one node unless siblings repeat a token), finds
// each frontier node's row argmax across the W slices, and moves to the children that
// match; the deepest frontier's smallest node ends the path.
//
// ts_walk and tg_walk are the only kernels: every workgroup checks its sequence's inputs
// and lists a node's children (node order) when it gets there.  A sequence's hand-over
// generation mixes the host's number for the call with the sequence's epoch, a counter in
// the workspace that every workgroup of the sequence reads when it starts and increments
// once it has the first hand-over (by then all of them have read it), so every run, graph
// replays included, tags its words anew without a kernel of its own.  The workgroups of a
// sequence wait for each other, so
// a launch holds at most half of the workgroups that fit on the device at once, and every
// wait is bounded.
#include <atomic>

#include "device_common.h"
#include "host_runtime.h"
#include "spec_verify.h"
#include "tree_walk.h"

namespace specv {

constexpr int kTsNV = 4;                          // 16-byte vectors per lane per row slice
constexpr int kTsMaxSlices = 64;                  // workgroups per sequence
constexpr int kTsWords = 8;                       // tagged 64-bit words per slot

// Keeps the scheduler from interleaving the unpacked elements of several vectors, which
// would hold all of them in registers at once.
__device__ __forceinline__ void ts_vector_done() { __builtin_amdgcn_sched_barrier(0); }

// Marks the packed slice registers as rewritten, so that each pass over them unpacks the
// elements again instead of keeping every unpacked element alive from the first pass.
__device__ __forceinline__ void ts_fresh(u32x4 (&r)[kTsNV]) {
#pragma unroll
  for (int j = 0; j < kTsNV; ++j) asm volatile("" : "+v"(r[j]));
}

struct TsArgs {
  const void* target;
  const void* draft;
  const int32_t* parent;
  const int32_t* token;
  const float* temperature;
  const float* u_accept;
  const float* u_final;
  int B, N1, V, max_depth, W;
  int greedy;       // no temperature and uniforms (greedy walk)
  int32_t* out_len;
  int32_t* out_tokens;
  int32_t* out_nodes;
  uint32_t gen;     // the host's number for this call
  int poll_limit;   // polls of a missing hand-over word before a wait gives up
  uint32_t* epoch;  // [B] run counters
  uint64_t* slots;  // [B, 2, W, kTsWords]
  int xcd_local;    // a launch of a multiple of 8 sequences keeps each on one XCD (see ts_place)
};

// Sequence and slice of this workgroup in a launch of W workgroups a sequence from sequence b0
// on.  With xcd_local, when the launch holds a multiple of 8 sequences, XCD x (grid index
// mod 8) takes sequences [x nb/8, (x+1) nb/8) of its nb whole and a sequence's slice exchanges
// stay in its L2 (store_xcd); otherwise W consecutive workgroups a sequence, spread over the
// XCDs.  (Measured at B=32 trees of 60 nodes, V=128256 bf16, stochastic walk: 57.7 us per call
// spread, 63.5 on one XCD with agent-scope stores, 52.7 on one XCD through its L2.)
struct TsPlace {
  int b, w;
  bool local;  // this workgroup's hand-over words may go through its XCD's L2
};

__device__ __forceinline__ TsPlace ts_place(const TsArgs& a, int b0) {
  const int i = static_cast<int>(blockIdx.x);
  const int W = a.W;
  const int nb = static_cast<int>(gridDim.x) / W;
  if (!a.xcd_local || nb % kXcds != 0) return TsPlace{b0 + i / W, i % W, false};
  const int m = i / kXcds;
  return TsPlace{b0 + (i % kXcds) * (nb / kXcds) + m / W, m % W, on_indexed_xcd()};
}

// ---------------------------------------------------------------- hand-over tags
//
// Slot words are the tagged words of device_common.h; the tag mixes the call's generation
// with the walk step.  Steps alternate between two slots per workgroup: a workgroup
// publishes step s + 2 only after it has read every workgroup's step s + 1, which each of
// them published only after reading step s, so no word is overwritten before all readers
// have it.
__device__ __forceinline__ uint32_t ts_tag(uint32_t gen, int step) {
  const uint32_t t = gen ^ (static_cast<uint32_t>(step) * 0x9e3779b1u);
  return t != 0u ? t : 0x2545f491u;
}

__device__ __forceinline__ bool ts_get_float(const uint64_t* w, uint32_t tag, float* v) {
  uint32_t x;
  const bool ok = get_tagged_u32(w, tag, &x);
  *v = __uint_as_float(x);
  return ok;
}

// Two workgroup reductions with one exchange through shared memory (lds: 2 * kWaves).
__device__ __forceinline__ void ts_block_max2(float& x, float& y, float* lds) {
  x = wave_max(x);
  y = wave_max(y);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    lds[w] = x;
    lds[kWaves + w] = y;
  }
  __syncthreads();
  float rx = lds[0], ry = lds[kWaves];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) {
    rx = fmaxf(rx, lds[i]);
    ry = fmaxf(ry, lds[kWaves + i]);
  }
  x = rx;
  y = ry;
}

__device__ __forceinline__ void ts_block_sum2(double& x, double& y, double* lds) {
  x = wave_sum(x);
  y = wave_sum(y);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    lds[w] = x;
    lds[kWaves + w] = y;
  }
  __syncthreads();
  double rx = 0.0, ry = 0.0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    rx += lds[i];
    ry += lds[kWaves + i];
  }
  x = rx;
  y = ry;
}

// ---------------------------------------------------------------- walk
// The sequence's generation.  Read before the sequence's first hand-over; ts_next_epoch
// runs only after it, so all workgroups of a run read the same epoch.
__device__ __forceinline__ uint32_t ts_generation(const TsArgs& a, int b) {
  const uint32_t g = a.gen ^ (load_agent(a.epoch + b) * 0x9e3779b1u);
  return g != 0u ? g : 0x2545f491u;
}

// Every workgroup of a valid sequence adds 1 after its first completed hand-over, so the
// next run of the sequence reads a new epoch.
__device__ __forceinline__ void ts_next_epoch(const TsArgs& a, int b) {
  if (threadIdx.x == 0) __hip_atomic_fetch_add(a.epoch + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Flags sequence b: out_len = code (-1 invalid input, -2 a hand-over wait gave up), path
// outputs -1.  Only workgroup 0 of a sequence writes its outputs, in every case, so that a
// flag never mixes with a result.
constexpr int kFlagInvalid = -1;

__device__ __forceinline__ void ts_write_flag(const TsArgs& a, int b, int code) {
  const int D1 = a.max_depth + 1;
  for (int k = threadIdx.x; k < D1; k += kThreads) {
    a.out_tokens[static_cast<size_t>(b) * D1 + k] = -1;
    a.out_nodes[static_cast<size_t>(b) * D1 + k] = -1;
  }
  if (threadIdx.x == 0) a.out_len[b] = code;
}

// Stage the sequence's parents and tokens (and uniforms) in shared memory and check them,
// as every workgroup of the sequence does.  True if valid.
__device__ __forceinline__ bool ts_stage(const TsArgs& a, int b, int* par, int* tok, float* ua) {
  const int tid = threadIdx.x, N1 = a.N1;
  const int32_t* gp = a.parent + static_cast<size_t>(b) * N1;
  const int32_t* gt = a.token + static_cast<size_t>(b) * N1;
  int bad = 0;
  for (int i = tid; i < N1; i += kThreads) {
    const int p = gp[i];
    const int x = gt[i];
    par[i] = p;
    tok[i] = x;
    if (i == 0) {
      bad |= p != -1;
    } else {
      bad |= p < 0 || p >= i;
      bad |= x < 0 || x >= a.V;
    }
    if (!a.greedy) {
      const float u = a.u_accept[static_cast<size_t>(b) * N1 + i];
      ua[i] = u;
      if (i > 0) bad |= !(u > 0.f && u <= 1.f);
    }
  }
  if (!a.greedy && tid == 0) {
    const float T = a.temperature[b];
    const float uf = a.u_final[b];
    bad |= !(T > 0.f && T <= 3.4e38f);
    bad |= !(uf > 0.f && uf <= 1.f);
  }
  return !__syncthreads_or(bad);
}

// The children of node u, in node order, into kids; returns their number (the same in
// every lane).  Parents precede children, so a node's children follow it.
__device__ __forceinline__ int ts_children(int u, int N1, const int* par, int* kids, int* red) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int total = 0;
  for (int base = (u + 1) & ~(kThreads - 1); base < N1; base += kThreads) {
    const int i = base + tid;
    const bool is = i < N1 && i > u && par[i] == u;
    const unsigned long long mask = __ballot(is);
    __syncthreads();
    if (lane == 0) red[wv] = __popcll(mask);
    __syncthreads();
    int before = total, add = 0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      before += k < wv ? red[k] : 0;
      add += red[k];
    }
    if (is) kids[before + __popcll(mask & ((1ull << lane) - 1ull))] = i;
    total += add;
  }
  __syncthreads();
  return total;
}

struct TsShared {
  double mass[kTsMaxSlices];  // slice masses of the current final-draw candidate
  float o[2][kTsMaxSlices];   // slice row maxima (target, draft) of the current step
  double s[2][kTsMaxSlices];  // slice exp2 sums
  double d[2 * kWaves];
  float f[2 * kWaves];
  int i[kWaves];
  int y;
  float lt[SPEC_MAX_TREE_NODES];  // logits of the current node's children tokens (target row)
  float ld[SPEC_MAX_TREE_NODES];  // (draft row)
  int path[SPEC_MAX_TREE_NODES + 1];
  // the sequence's topology, tokens and uniforms, staged once
  int par[SPEC_MAX_TREE_NODES];
  int kids[SPEC_MAX_TREE_NODES];  // children of the current node
  int tok[SPEC_MAX_TREE_NODES];
  float ua[SPEC_MAX_TREE_NODES];
  int ci[kWaves];
};

// Wait until every workgroup of the sequence has published `tag` in `slot_base[w]`, then
// copy its first `nd` doubles (words 0-1 and 2-3) and `nf` floats (words 4 and 5) into
// shared memory.  False if the wait gave up (after `limit` polls that found a word missing;
// at once when limit is 0).
__device__ __forceinline__ bool ts_gather(const uint64_t* slot_base, int W, uint32_t tag, int nd, int nf,
                                          int limit, double* dst_d0, double* dst_d1, float* dst_f0,
                                          float* dst_f1) {
  const int tid = threadIdx.x;
  for (int polls = 0;; ++polls) {
    if (polls >= limit) return false;
    int missing = 0;
    if (tid < W) {
      const uint64_t* sl = slot_base + static_cast<size_t>(tid) * kTsWords;
      double v;
      float f;
      if (nd > 0) {
        if (get_tagged_double(sl + 0, tag, &v)) dst_d0[tid] = v; else missing = 1;
      }
      if (nd > 1) {
        if (get_tagged_double(sl + 2, tag, &v)) dst_d1[tid] = v; else missing = 1;
      }
      if (nf > 0) {
        if (ts_get_float(sl + 4, tag, &f)) dst_f0[tid] = f; else missing = 1;
      }
      if (nf > 1) {
        if (ts_get_float(sl + 5, tag, &f)) dst_f1[tid] = f; else missing = 1;
      }
    }
    if (!__syncthreads_or(missing)) return true;
    short_pause();
  }
}

// Wait for one tagged 32-bit word (the drawn token that the drawing workgroup hands to
// workgroup 0); false if the wait gave up, as for ts_gather.
__device__ __forceinline__ bool ts_wait_word(const uint64_t* word, uint32_t tag, int limit, uint32_t* v) {
  for (int polls = 0;; ++polls) {
    if (polls >= limit) return false;
    if (!__syncthreads_or(get_tagged_u32(word, tag, v) ? 0 : 1)) return true;
    short_pause();
  }
}

// The accepted path (sh.path[0 .. plen-1]), its tokens, then y, then -1.
__device__ __forceinline__ void ts_write_path(const TsArgs& a, int b, const TsShared& sh, int plen, int y) {
  const int D1 = a.max_depth + 1;
  int32_t* ot = a.out_tokens + static_cast<size_t>(b) * D1;
  int32_t* on = a.out_nodes + static_cast<size_t>(b) * D1;
  for (int k = threadIdx.x; k < D1; k += kThreads) {
    const int node = k < plen ? sh.path[k] : -1;
    on[k] = node;
    ot[k] = k < plen ? sh.tok[node] : (k == plen ? y : -1);
  }
  if (threadIdx.x == 0) a.out_len[b] = plen;
}

template <int DT, bool VEC>
__device__ __forceinline__ void ts_walk_body(const TsArgs& a, const TsPlace& pl, uint32_t gen, TsShared& sh) {
  using EL = Elem<DT>;
  constexpr int E = EL::kPerVec;
  constexpr int kSlice = kThreads * kTsNV * E;  // elements per slice
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int W = a.W;
  const int b = pl.b;
  const int w = pl.w;
  const bool local = pl.local;
  const int N1 = a.N1, V = a.V;
  if (!ts_stage(a, b, sh.par, sh.tok, sh.ua)) {
    if (w == 0) ts_write_flag(a, b, kFlagInvalid);
    return;
  }
  const float T = a.temperature[b];
  const float scale = kLog2e / T;
  const size_t rowb = static_cast<size_t>(V) * EL::kBytes;
  const char* tbase = static_cast<const char*>(a.target) + static_cast<size_t>(b) * N1 * rowb;
  const char* dbase = static_cast<const char*>(a.draft) + static_cast<size_t>(b) * N1 * rowb;
  const int sl0 = w * kSlice;
  u32x4 rt[kTsNV], rd[kTsNV];
  // the root's slices first: they depend on nothing staged below
#pragma unroll
  for (int j = 0; j < kTsNV; ++j) rt[j] = load_vector<DT, VEC>(tbase, V, sl0 + (j * kThreads + tid) * E);
#pragma unroll
  for (int j = 0; j < kTsNV; ++j) rd[j] = load_vector<DT, VEC>(dbase, V, sl0 + (j * kThreads + tid) * E);
  uint64_t* slots = a.slots + static_cast<size_t>(b) * 2 * W * kTsWords;

  int step = 0, cur = 0, plen = 0;
  bool residual = false;            // final draw from the residual (else the bonus from p)
  double c = 0.0, D = 1.0;          // residual max(0, p - c q) / D
  float Op = 0.f, Oq = 0.f;
  double Sp = 1.0, Sq = 1.0;

  for (;;) {
    // (ts_children waits for every lane to be done with the previous node's shared values)
    const int m = uniform(ts_children(cur, N1, sh.par, sh.kids, sh.ci));
    const char* row_t = tbase + static_cast<size_t>(cur) * rowb;
    const char* row_d = dbase + static_cast<size_t>(cur) * rowb;
    if (cur != 0) {  // the root's slices are loaded already
#pragma unroll
      for (int j = 0; j < kTsNV; ++j) rt[j] = load_vector<DT, VEC>(row_t, V, sl0 + (j * kThreads + tid) * E);
      if (m > 0) {
#pragma unroll
        for (int j = 0; j < kTsNV; ++j) rd[j] = load_vector<DT, VEC>(row_d, V, sl0 + (j * kThreads + tid) * E);
      }
    }
    for (int j = tid; j < m; j += kThreads) {
      const int x = sh.tok[sh.kids[j]];
      sh.lt[j] = EL::value(row_t, x);
      sh.ld[j] = EL::value(row_d, x);
    }
    // ---- this slice's row maxima and exp2 sums (target, and draft when the node has children)
    float mt = -INFINITY, md = -INFINITY;
    ts_fresh(rt);
    ts_fresh(rd);
#pragma unroll
    for (int j = 0; j < kTsNV; ++j) {
#pragma unroll
      for (int i = 0; i < E; ++i) {
        mt = fmaxf(mt, EL::get(rt[j], i));
        if (m > 0) md = fmaxf(md, EL::get(rd[j], i));
      }
      ts_vector_done();
    }
    ts_block_max2(mt, md, sh.f);
    const float ot = mt * scale;
    const float od = m > 0 ? md * scale : -INFINITY;
    float st = 0.f, sd = 0.f;
    ts_fresh(rt);
    ts_fresh(rd);
    if (ot > -INFINITY) {
      float st2 = 0.f;
#pragma unroll
      for (int j = 0; j < kTsNV; ++j)
#pragma unroll
        for (int i = 0; i < E; i += 2) {
          st += exp2_fast(fmaf(EL::get(rt[j], i), scale, -ot));
          st2 += exp2_fast(fmaf(EL::get(rt[j], i + 1), scale, -ot));
        }
      st += st2;
    }
    if (m > 0 && od > -INFINITY) {
      float sd2 = 0.f;
#pragma unroll
      for (int j = 0; j < kTsNV; ++j)
#pragma unroll
        for (int i = 0; i < E; i += 2) {
          sd += exp2_fast(fmaf(EL::get(rd[j], i), scale, -od));
          sd2 += exp2_fast(fmaf(EL::get(rd[j], i + 1), scale, -od));
        }
      sd += sd2;
    }
    double St = static_cast<double>(st), Sd = static_cast<double>(sd);
    ts_block_sum2(St, Sd, sh.d);
    uint64_t* mine = slots + (static_cast<size_t>(step & 1) * W + w) * kTsWords;
    uint32_t tag = ts_tag(gen, step);
    if (tid == 0) {
      put_tagged_double(mine + 0, St, tag, local);
      put_tagged_double(mine + 2, Sd, tag, local);
      store_handover(mine + 4, tagged(__float_as_uint(ot), tag), local);
      store_handover(mine + 5, tagged(__float_as_uint(od), tag), local);
    }
    if (!ts_gather(slots + static_cast<size_t>(step & 1) * W * kTsWords, W, tag, 2, 2, a.poll_limit, sh.s[0],
                   sh.s[1], sh.o[0], sh.o[1])) {
      if (w == 0) ts_write_flag(a, b, kFlagTimedOut);
      return;
    }
    if (step == 0) ts_next_epoch(a, b);
    ++step;
    // ---- the node's p and q: lane q of every wave takes slice q, and the wave reductions
    // (a fixed DPP order) give the same values in every wave of every workgroup
    {
      const float o0 = lane < W ? sh.o[0][lane] : -INFINITY;
      const float o1 = lane < W && m > 0 ? sh.o[1][lane] : -INFINITY;
      Op = uniform(wave_max(o0));
      Oq = uniform(wave_max(o1));
      const double mp = o0 > -INFINITY ? sh.s[0][lane] * static_cast<double>(exp2_fast(o0 - Op)) : 0.0;
      const double mq = o1 > -INFINITY ? sh.s[1][lane] * static_cast<double>(exp2_fast(o1 - Oq)) : 0.0;
      Sp = uniform(wave_sum(mp));
      Sq = uniform(wave_sum(mq));
      __syncthreads();
      if (tid < W) sh.mass[tid] = mp;  // bonus draw candidate: slice masses of p (scaled by Sp)
    }
    __syncthreads();
    if (m == 0) {
      residual = false;
      break;
    }
    // ---- the children in node order against the residual
    c = 0.0;
    D = 1.0;
    bool moved = false;
    for (int j = 0; j < m; ++j) {
      const int kid = uniform(sh.kids[j]);
      const double px = static_cast<double>(exp2_fast(fmaf(uniform(sh.lt[j]), scale, -Op))) / Sp;
      const double qx = static_cast<double>(exp2_fast(fmaf(uniform(sh.ld[j]), scale, -Oq))) / Sq;
      const double rx = fmax(0.0, px - c * qx) / D;
      const double alpha = uniform(qx > 0.0 ? fmin(1.0, rx / qx) : (rx > 0.0 ? 1.0 : 0.0));
      if (static_cast<double>(sh.ua[kid]) <= alpha) {
        if (plen >= a.max_depth) {  // the path outgrows its output row
          if (w == 0) ts_write_flag(a, b, kFlagInvalid);
          return;
        }
        if (tid == 0) sh.path[plen] = kid;
        ++plen;
        cur = kid;
        moved = true;
        break;
      }
      // rejected: D' = sum over the vocabulary of max(0, p - c' q), c' = c + D
      const double cn = c + D;
      const float cf = static_cast<float>(cn);
      const float ip = static_cast<float>(1.0 / Sp), iq = static_cast<float>(1.0 / Sq);
      float acc = 0.f;
      ts_fresh(rt);
      ts_fresh(rd);
#pragma unroll
      for (int jj = 0; jj < kTsNV; ++jj) {
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const float pv = exp2_fast(fmaf(EL::get(rt[jj], i), scale, -Op)) * ip;
          const float qv = exp2_fast(fmaf(EL::get(rd[jj], i), scale, -Oq)) * iq;
          acc += fmaxf(0.f, pv - cf * qv);
        }
        ts_vector_done();
      }
      const double part = block_sum(static_cast<double>(acc), sh.d);
      mine = slots + (static_cast<size_t>(step & 1) * W + w) * kTsWords;
      tag = ts_tag(gen, step);
      if (tid == 0) put_tagged_double(mine, part, tag, local);
      double* tmp = sh.s[0];  // reuse: the stats of this node are combined already
      if (!ts_gather(slots + static_cast<size_t>(step & 1) * W * kTsWords, W, tag, 1, 0, a.poll_limit, tmp,
                     nullptr, nullptr, nullptr)) {
        if (w == 0) ts_write_flag(a, b, kFlagTimedOut);
        return;
      }
      ++step;
      const double Dn = uniform(wave_sum(lane < W ? tmp[lane] : 0.0));
      if (Dn > 0.0) {  // else no mass left after rounding: keep the previous residual (p at first)
        c = cn;
        D = Dn;
        residual = true;
        __syncthreads();
        if (tid < W) sh.mass[tid] = tmp[tid];
      }
      __syncthreads();
    }
    if (!moved) break;
    residual = false;
  }
  // After the loop: a leaf reached by acceptance (bonus from p; residual == false), or
  // every child of `cur` rejected (draw from max(0, p - c q) / D; if no residual ever had
  // mass, c = 0 and the draw is from p).
  const bool use_q = residual;
  const double total = uniform(wave_sum(lane < W ? sh.mass[lane] : 0.0));
  const double tt = uniform(static_cast<double>(a.u_final[b]) * total);
  int wsel = -1, wlast = -1;
  {
    double run = 0.0;
    for (int q = 0; q < W; ++q) {
      run += sh.mass[q];
      if (sh.mass[q] > 0.0) {
        wlast = q;
        if (wsel < 0 && run >= tt) wsel = q;
      }
    }
    if (wsel < 0) wsel = wlast >= 0 ? wlast : 0;
  }
  const int D1 = a.max_depth + 1;
  if (w != wsel) {
    if (w != 0) return;
    // workgroup 0 writes the row once the drawing workgroup has handed the token over
    uint32_t yv = 0;
    if (!ts_wait_word(slots + (static_cast<size_t>(step & 1) * W + wsel) * kTsWords + 4, ts_tag(gen, step),
                      a.poll_limit, &yv)) {
      ts_write_flag(a, b, kFlagTimedOut);
      return;
    }
    ts_write_path(a, b, sh, plen, static_cast<int>(yv));
    return;
  }
  double before = 0.0;
  for (int q = 0; q < wsel; ++q) before += sh.mass[q];
  const double t_loc = uniform(tt - before);
  const float ip = static_cast<float>(1.0 / Sp), iq = static_cast<float>(1.0 / Sq);
  const float cf = static_cast<float>(c);
  // draw weights in the same scale as the slice masses: p's masses are sums of
  // exp2(l * scale - Op); residual masses are sums of max(0, p - c q)
  auto weight = [&](float l_t, float l_d) -> float {
    const float et = exp2_fast(fmaf(l_t, scale, -Op));
    if (!use_q) return et;
    const float pv = et * ip;
    const float qv = exp2_fast(fmaf(l_d, scale, -Oq)) * iq;
    return fmaxf(0.f, pv - cf * qv);
  };
  // the vector round j holding t_loc (rounds are vocabulary-ordered inside the slice)
  ts_fresh(rt);
  ts_fresh(rd);
  double rb = 0.0;
  int jsel = -1, jlast = -1;
  double jbase = 0.0;
  for (int j = 0; j < kTsNV; ++j) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) s += weight(EL::get(rt[j], i), EL::get(rd[j], i));
    const double tot = block_sum(static_cast<double>(s), sh.d);
    if (tot > 0.0) {
      jlast = j;
      if (jsel < 0 && rb + tot >= t_loc) {
        jsel = j;
        jbase = rb;
      }
    }
    rb += tot;
  }
  if (jsel < 0) {  // rounding left t_loc above the slice total: its last round with mass
    jsel = jlast >= 0 ? jlast : 0;
    jbase = 0.0;
    for (int j = 0; j < jsel; ++j) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) s += weight(EL::get(rt[j], i), EL::get(rd[j], i));
      jbase += block_sum(static_cast<double>(s), sh.d);
    }
  }
  const double t_round = t_loc - jbase;
  // the lane, then the element
  u32x4 vt = rt[0], vd = rd[0];
#pragma unroll
  for (int j = 1; j < kTsNV; ++j)
    if (j == jsel) {
      vt = rt[j];
      vd = rd[j];
    }
  const int e0 = sl0 + (jsel * kThreads + tid) * E;
  float wl[E];
  float lsum = 0.f;
  int last_pos = -1;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    wl[i] = e0 + i < V ? weight(EL::get(vt, i), EL::get(vd, i)) : 0.f;
    lsum += wl[i];
    last_pos = wl[i] > 0.f ? e0 + i : last_pos;
  }
  const double lincl = wave_inclusive_scan(static_cast<double>(lsum));
  __syncthreads();
  if (lane == 63) sh.d[wv] = lincl;
  __syncthreads();
  double lbefore = lincl - static_cast<double>(lsum);
  for (int i = 0; i < wv; ++i) lbefore += sh.d[i];
  const int key = (lsum > 0.f && lbefore + static_cast<double>(lsum) >= t_round) ? tid : INT_MAX;
  const int kmin = block_min_int(key, sh.i);
  int y;
  if (kmin == INT_MAX) {
    y = block_max_int(last_pos, sh.i);
    if (y < 0) y = sl0;
  } else {
    if (tid == kmin) {
      double run = lbefore;
      int pick = -1;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        run += wl[i];
        if (pick < 0 && wl[i] > 0.f && run >= t_round) pick = e0 + i;
      }
      sh.y = pick >= 0 ? pick : last_pos;
    }
    __syncthreads();
    y = sh.y;
  }
  if (w != 0) {  // hand the token to workgroup 0, which writes the row
    // (this workgroup's slot of parity `step` held its word of step - 2, which every
    // workgroup had read before publishing step - 1, read here in the last gather)
    if (tid == 0)
      store_handover(slots + (static_cast<size_t>(step & 1) * W + w) * kTsWords + 4,
                     tagged(static_cast<uint32_t>(y), ts_tag(gen, step)), local);
    return;
  }
  ts_write_path(a, b, sh, plen, y);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void ts_walk_kernel(TsArgs a, int b0) {
  __shared__ TsShared sh;
  const TsPlace pl = ts_place(a, b0);
  ts_walk_body<DT, VEC>(a, pl, ts_generation(a, pl.b), sh);
}

// ---------------------------------------------------------------- greedy walk
struct TgShared {
  float v[kTsMaxSlices];  // slice maxima of the current node's row
  float i[kTsMaxSlices];  // their first indices (int bits)
  float wv[kWaves];
  int wi[kWaves];
  int nf, nn;             // frontier and next-frontier sizes
  int front[SPEC_MAX_TREE_NODES];
  int nxt[SPEC_MAX_TREE_NODES];
  int amax[SPEC_MAX_TREE_NODES];  // row argmax of each frontier node
  int tok[SPEC_MAX_TREE_NODES];
  int par[SPEC_MAX_TREE_NODES];
};

// Same hand-over as ts_gather, for the (max, first index) pair of each slice.
__device__ __forceinline__ bool tg_gather(const uint64_t* slot_base, int W, uint32_t tag, int limit, TgShared& sh) {
  const int tid = threadIdx.x;
  for (int polls = 0;; ++polls) {
    if (polls >= limit) return false;
    int missing = 0;
    if (tid < W) {
      const uint64_t* sl = slot_base + static_cast<size_t>(tid) * kTsWords;
      float f;
      if (ts_get_float(sl + 4, tag, &f)) sh.v[tid] = f; else missing = 1;
      if (ts_get_float(sl + 5, tag, &f)) sh.i[tid] = f; else missing = 1;
    }
    if (!__syncthreads_or(missing)) return true;
    short_pause();
  }
}

template <int DT, bool VEC>
__device__ __forceinline__ void tg_walk_body(const TsArgs& a, const TsPlace& pl, uint32_t gen, TgShared& sh) {
  using EL = Elem<DT>;
  constexpr int E = EL::kPerVec;
  constexpr int kSlice = kThreads * kTsNV * E;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int W = a.W;
  const int b = pl.b;
  const int w = pl.w;
  const int N1 = a.N1, V = a.V;
  const size_t rowb = static_cast<size_t>(V) * EL::kBytes;
  const char* tbase = static_cast<const char*>(a.target) + static_cast<size_t>(b) * N1 * rowb;
  const int sl0 = w * kSlice;
  u32x4 rt[kTsNV];
#pragma unroll
  for (int j = 0; j < kTsNV; ++j) rt[j] = load_vector<DT, VEC>(tbase, V, sl0 + (j * kThreads + tid) * E);
  if (!ts_stage(a, b, sh.par, sh.tok, nullptr)) {
    if (w == 0) ts_write_flag(a, b, kFlagInvalid);
    return;
  }
  if (tid == 0) {
    sh.nf = 1;
    sh.front[0] = 0;
  }
  uint64_t* slots = a.slots + static_cast<size_t>(b) * 2 * W * kTsWords;
  int step = 0, depth = 0;
  bool loaded = true;  // rt holds the root's slice
  for (;;) {
    __syncthreads();
    const int F = uniform(sh.nf);
    if (tid == 0) sh.nn = 0;
    for (int fi = 0; fi < F; ++fi) {
      const int f = uniform(sh.front[fi]);
      if (!loaded) {
        const char* row = tbase + static_cast<size_t>(f) * rowb;
#pragma unroll
        for (int j = 0; j < kTsNV; ++j) rt[j] = load_vector<DT, VEC>(row, V, sl0 + (j * kThreads + tid) * E);
      }
      loaded = false;
      // (max, first index) over this lane's elements in vocabulary order, then the slice
      float bv = -INFINITY;
      int bi = INT_MAX;
#pragma unroll
      for (int j = 0; j < kTsNV; ++j)
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const int e = sl0 + (j * kThreads + tid) * E + i;
          const float x = EL::get(rt[j], i);
          if (e < V && better(x, e, bv, bi)) {
            bv = x;
            bi = e;
          }
        }
      wave_argmax(bv, bi);
      __syncthreads();
      if (lane == 0) {
        sh.wv[wv] = bv;
        sh.wi[wv] = bi;
      }
      __syncthreads();
      float sv = sh.wv[0];
      int si = sh.wi[0];
      for (int k = 1; k < kWaves; ++k)
        if (better(sh.wv[k], sh.wi[k], sv, si)) {
          sv = sh.wv[k];
          si = sh.wi[k];
        }
      const uint32_t tag = ts_tag(gen, step);
      uint64_t* mine = slots + (static_cast<size_t>(step & 1) * W + w) * kTsWords;
      if (tid == 0) {
        store_handover(mine + 4, tagged(__float_as_uint(sv), tag), pl.local);
        store_handover(mine + 5, tagged(static_cast<uint32_t>(si), tag), pl.local);
      }
      if (!tg_gather(slots + static_cast<size_t>(step & 1) * W * kTsWords, W, tag, a.poll_limit, sh)) {
        if (w == 0) ts_write_flag(a, b, kFlagTimedOut);
        return;
      }
      if (step == 0) ts_next_epoch(a, b);
      ++step;
      // every slice's pair: lane q takes slice q; (max, first index) does not depend on order
      float gv = lane < W ? sh.v[lane] : -INFINITY;
      int gi = lane < W ? __float_as_int(sh.i[lane]) : INT_MAX;
      wave_argmax(gv, gi);
      gi = uniform(gi);
      // the children whose token is the argmax join the next frontier, in node order
      // (children follow their parent)
      if (wv == 0) {
        int base = sh.nn;
        for (int k = (f + 1) & ~63; k < N1; k += 64) {
          const int c = k + lane;
          const bool match = c > f && c < N1 && sh.par[c] == f && sh.tok[c] == gi;
          const unsigned long long mask = __ballot(match);
          if (match) sh.nxt[base + __popcll(mask & ((1ull << lane) - 1ull))] = c;
          base += __popcll(mask);
        }
        if (lane == 0) {
          sh.nn = base;
          sh.amax[fi] = gi;
        }
      }
      __syncthreads();
    }
    const int nn = uniform(sh.nn);
    if (nn == 0) break;
    if (++depth > a.max_depth) {  // the accepted path outgrows its output row
      if (w == 0) ts_write_flag(a, b, kFlagInvalid);
      return;
    }
    if (tid == 0) {
      for (int k = 0; k < nn; ++k) sh.front[k] = sh.nxt[k];
      sh.nf = nn;
    }
  }
  if (w != 0) return;
  // the deepest accepted level is the frontier: its smallest node ends the path
  const int F = uniform(sh.nf);
  int best = INT_MAX, bonus = -1;
  for (int fi = 0; fi < F; ++fi)
    if (sh.front[fi] < best) {
      best = sh.front[fi];
      bonus = sh.amax[fi];
    }
  const int D1 = a.max_depth + 1;
  int32_t* ot = a.out_tokens + static_cast<size_t>(b) * D1;
  int32_t* on = a.out_nodes + static_cast<size_t>(b) * D1;
  if (tid == 0) {
    int v = best;
    for (int k = depth - 1; k >= 0; --k) {  // root-first: position k holds the node at depth k + 1
      on[k] = v;
      ot[k] = sh.tok[v];
      v = sh.par[v];
    }
    ot[depth] = bonus;
    a.out_len[b] = depth;
  }
  for (int k = depth + 1 + tid; k < D1; k += kThreads) ot[k] = -1;
  for (int k = depth + tid; k < D1; k += kThreads) on[k] = -1;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void tg_walk_kernel(TsArgs a, int b0) {
  __shared__ TgShared sh;
  const TsPlace pl = ts_place(a, b0);
  tg_walk_body<DT, VEC>(a, pl, ts_generation(a, pl.b), sh);
}

// ---------------------------------------------------------------- host
struct TsLayout {
  size_t off_slots, bytes;
  int W;
};

static TsLayout ts_layout(int B, int N1, int V, spec_dtype_t dtype) {
  TsLayout L{};
  const int E = dtype == SPEC_BF16 ? 8 : 4;
  const long long slice = static_cast<long long>(kThreads) * kTsNV * E;
  L.W = static_cast<int>((V + slice - 1) / slice);
  (void)N1;
  size_t off = align_up(sizeof(uint32_t) * B, 256);  // epochs
  L.off_slots = off;
  off = align_up(off + sizeof(uint64_t) * static_cast<size_t>(B) * 2 * L.W * kTsWords, 256);
  L.bytes = off;
  return L;
}

template <int DT, bool VEC>
static int ts_slots_per_device() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(ts_walk_kernel<DT, VEC>),
                                                   kThreads, 0) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 1;
  v = per_cu * cus;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

static uint32_t ts_next_generation() {
  static std::atomic<uint32_t> counter{0x6a09e667u};
  uint32_t g = counter.fetch_add(0x9e3779b9u, std::memory_order_relaxed);
  return g != 0u ? g : 0x2545f491u;
}

template <int DT, bool VEC>
static spec_status_t ts_launch(const TsArgs& a, hipStream_t s) {
  const int slots = ts_slots_per_device<DT, VEC>();
  const int per_launch = (slots / 2) / a.W;
  if (per_launch < 1) return fail(SPEC_ERR_UNSUPPORTED, "V needs %d workgroups per sequence, more than fit", a.W);
  for (int b0 = 0; b0 < a.B; b0 += per_launch) {
    const int nb = a.B - b0 < per_launch ? a.B - b0 : per_launch;
    LaunchScope scope("ts_walk", s);
    scope.launch(ts_walk_kernel<DT, VEC>, dim3(static_cast<unsigned>(nb * a.W)), dim3(kThreads), s, a, b0);
    const spec_status_t st = scope.finish();
    if (st != SPEC_OK) return st;
  }
  return SPEC_OK;
}

template <int DT, bool VEC>
static int tg_slots_per_device() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(tg_walk_kernel<DT, VEC>),
                                                   kThreads, 0) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 1;
  v = per_cu * cus;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

template <int DT, bool VEC>
static spec_status_t tg_launch(const TsArgs& a, hipStream_t s) {
  const int per_launch = (tg_slots_per_device<DT, VEC>() / 2) / a.W;
  if (per_launch < 1) return fail(SPEC_ERR_UNSUPPORTED, "V needs %d workgroups per sequence, more than fit", a.W);
  for (int b0 = 0; b0 < a.B; b0 += per_launch) {
    const int nb = a.B - b0 < per_launch ? a.B - b0 : per_launch;
    LaunchScope scope("tg_walk", s);
    scope.launch(tg_walk_kernel<DT, VEC>, dim3(static_cast<unsigned>(nb * a.W)), dim3(kThreads), s, a, b0);
    const spec_status_t st = scope.finish();
    if (st != SPEC_OK) return st;
  }
  return SPEC_OK;
}

size_t tree_walk_workspace_bytes(int B, int N1, int V, spec_dtype_t dtype) {
  const TsLayout L = ts_layout(B, N1, V, dtype);
  return L.W > kTsMaxSlices ? 0 : L.bytes;
}

spec_status_t tree_greedy_walk(const void* target_logits, spec_dtype_t dtype, const int32_t* parent,
                               const int32_t* node_token, int B, int N1, int V, int max_depth,
                               int32_t* out_accept_len, int32_t* out_tokens, int32_t* out_path_nodes,
                               void* workspace, size_t workspace_bytes, hipStream_t s) {
  const TsLayout L = ts_layout(B, N1, V, dtype);
  if (L.W > kTsMaxSlices) return fail(SPEC_ERR_UNSUPPORTED, "V = %d needs more than %d slices", V, kTsMaxSlices);
  if (workspace_bytes < L.bytes)
    return fail(SPEC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.bytes);
  TsArgs a{};
  a.target = target_logits;
  a.parent = parent;
  a.token = node_token;
  a.B = B;
  a.N1 = N1;
  a.V = V;
  a.max_depth = max_depth;
  a.W = L.W;
  a.greedy = 1;
  a.out_len = out_accept_len;
  a.out_tokens = out_tokens;
  a.out_nodes = out_path_nodes;
  a.gen = ts_next_generation();
  a.poll_limit = knob(SPEC_KNOB_POLL_LIMIT);
  a.xcd_local = knob(SPEC_KNOB_XCD_LOCAL);
  char* ws = static_cast<char*>(workspace);
  a.epoch = reinterpret_cast<uint32_t*>(ws);
  a.slots = reinterpret_cast<uint64_t*>(ws + L.off_slots);
  const int esize = dtype == SPEC_BF16 ? 2 : 4;
  const bool vec = (static_cast<size_t>(V) * esize) % 16 == 0 && aligned16(target_logits);
  if (dtype == SPEC_BF16) return vec ? tg_launch<kBF16, true>(a, s) : tg_launch<kBF16, false>(a, s);
  return vec ? tg_launch<kF32, true>(a, s) : tg_launch<kF32, false>(a, s);
}

}  // namespace specv

using namespace specv;

extern "C" {

size_t spec_verify_tree_workspace_size(int B, int N1, int V, spec_dtype_t dtype) {
  if (B <= 0 || N1 < 1 || N1 > SPEC_MAX_TREE_NODES || V < 1 || (dtype != SPEC_F32 && dtype != SPEC_BF16)) return 0;
  const TsLayout L = ts_layout(B, N1, V, dtype);
  if (L.W > kTsMaxSlices) return 0;
  return L.bytes;
}

spec_status_t spec_verify_tree(const void* target_logits, const void* draft_logits, spec_dtype_t dtype,
                               const int32_t* parent, const int32_t* node_token, const float* temperature,
                               const float* u_accept, const float* u_final, int B, int N1, int V, int max_depth,
                               int32_t* out_accept_len, int32_t* out_tokens, int32_t* out_path_nodes,
                               void* workspace, size_t workspace_bytes, spec_stream_t stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return fail(SPEC_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (B < 0 || N1 < 1 || V < 1 || max_depth < 0)
    return fail(SPEC_ERR_INVALID_ARG, "need B >= 0, N1 >= 1, V >= 1, max_depth >= 0");
  if (N1 > SPEC_MAX_TREE_NODES) return fail(SPEC_ERR_UNSUPPORTED, "N1 = %d exceeds SPEC_MAX_TREE_NODES", N1);
  if (max_depth > N1) return fail(SPEC_ERR_INVALID_ARG, "max_depth = %d exceeds N1 = %d", max_depth, N1);
  const TsLayout L = ts_layout(B > 0 ? B : 1, N1, V, dtype);
  if (L.W > kTsMaxSlices) return fail(SPEC_ERR_UNSUPPORTED, "V = %d needs more than %d slices", V, kTsMaxSlices);
  if (B == 0) return SPEC_OK;
  if (!target_logits || !draft_logits || !parent || !node_token || !temperature || !u_accept || !u_final ||
      !out_accept_len || !out_tokens || !out_path_nodes)
    return fail(SPEC_ERR_INVALID_ARG, "a required pointer is NULL");
  if (static_cast<double>(B) * N1 * V >= 140737488355328.0) return fail(SPEC_ERR_UNSUPPORTED, "B*N1*V too large");
  if (!workspace) return fail(SPEC_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(SPEC_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (workspace_bytes < L.bytes)
    return fail(SPEC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.bytes);
  TsArgs a{};
  a.target = target_logits;
  a.draft = draft_logits;
  a.parent = parent;
  a.token = node_token;
  a.temperature = temperature;
  a.u_accept = u_accept;
  a.u_final = u_final;
  a.B = B;
  a.N1 = N1;
  a.V = V;
  a.max_depth = max_depth;
  a.W = L.W;
  a.out_len = out_accept_len;
  a.out_tokens = out_tokens;
  a.out_nodes = out_path_nodes;
  a.gen = ts_next_generation();
  a.poll_limit = knob(SPEC_KNOB_POLL_LIMIT);
  a.xcd_local = knob(SPEC_KNOB_XCD_LOCAL);
  char* ws = static_cast<char*>(workspace);
  a.epoch = reinterpret_cast<uint32_t*>(ws);
  a.slots = reinterpret_cast<uint64_t*>(ws + L.off_slots);
  const int esize = dtype == SPEC_BF16 ? 2 : 4;
  const bool vec = (static_cast<size_t>(V) * esize) % 16 == 0 && aligned16(target_logits) && aligned16(draft_logits);
  if (dtype == SPEC_BF16) return vec ? ts_launch<kBF16, true>(a, s) : ts_launch<kBF16, false>(a, s);
  return vec ? ts_launch<kF32, true>(a, s) : ts_launch<kF32, false>(a, s);
}

}  // extern "C"
